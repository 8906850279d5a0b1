// fva_route.hip -- block router kernels for gfx950.
//
// FVAttn abstract: the sparse-routing frontend is Top-p routing with a Top-k
// safety floor over video-aware blocks, and the materialised mask is repaired
// at runtime.  The block score of a (query block, key block) pair is the dot
// product of the block-mean pooled Q and K rows scaled by head_dim^-0.5
// (scale rule: VSA guide, section 5).
//
// Three kernels, all taking their integer decisions in fp64 (MI355X runs fp64
// FMA at the fp32 rate, so the router costs little and decides as an fp64
// reference would):
//   pool_kernel        HBM stream of Q and K -> fp64 block means [B,h,N,D]
//   scores_kernel      per (b,h): S = Qbar Kbar^T / sqrt(D), 64x64 tiles
//   route_rows_kernel  N <= 256: one wavefront per row: softmax, bitonic
//                      sort on (score desc, index asc), scan, Top-p count,
//                      floor, mask words and kept count
//   route_select_kernel N > 256: the same decisions by a search over
//                      order-preserving keys (no full sort)
#include <algorithm>
#include <mutex>

#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

// ---------------------------------------------------------------------------
// Block-mean pooling.  grid = (N * chunks, 2, B), 256 threads.  A chunk covers
// 64 vectors of 8 channels (512 of the heads*D channels of a token row), one
// vector per lane; the 4 waves split the block's (t, y) rows and their partial
// sums are added in a fixed order.  Every token row is read as contiguous
// 16-byte loads across the lanes of a wave.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pool_kernel(const bf16_bits* __restrict__ q, const bf16_bits* __restrict__ k,
                                                   Geo g, int L, Heads hd, int D, int chunks,
                                                   double* __restrict__ qbar, double* __restrict__ kbar,
                                                   uint32_t* __restrict__ status, bool clear_status) {
  const int n = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int which = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (clear_status && status && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *status = 0u;

  const bf16_bits* x = which == 0 ? q : k;
  double* out = which == 0 ? qbar : kbar;
  const int nvec = hd.n * D / 8;
  const int vec = chunk * 64 + lane;
  const bool active = vec < nvec;
  const Box bx = block_box(g, n);
  const int64_t row_stride = (int64_t)hd.stride * D;
  const bf16_bits* base = x + (int64_t)b * L * row_stride + (int64_t)hd.h0 * D + (int64_t)vec * 8;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;

  const int rows = bx.et * bx.eh;
  for (int r = wave; r < rows; r += 4) {
    const int dt = r / bx.eh, dy = r % bx.eh;
    const int64_t tok0 = ((int64_t)(bx.t0 + dt) * g.H + (bx.y0 + dy)) * g.W + bx.x0;
    if (active) {
      int dx = 0;
      for (; dx + 4 <= bx.ew; dx += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const u32x4*)(base + (tok0 + dx + u) * row_stride);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)__uint_as_float(v[u][e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(v[u][e] & 0xffff0000u);
          }
      }
      for (; dx < bx.ew; ++dx) {
        u32x4 v = *(const u32x4*)(base + (tok0 + dx) * row_stride);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += (double)__uint_as_float(v[e] << 16);
          acc[2 * e + 1] += (double)__uint_as_float(v[e] & 0xffff0000u);
        }
      }
    }
  }

  __shared__ double part[4][64][9];
#pragma unroll
  for (int e = 0; e < 8; ++e) part[wave][lane][e] = acc[e];
  __syncthreads();
  if (wave == 0 && active) {
    const double inv_cnt = (double)bx.count;
    const int c0 = vec * 8;
    const int h = c0 / D, d0 = c0 % D;
    double* o = out + (((int64_t)b * hd.n + h) * g.N + n) * D + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double s = part[0][lane][e];
      s += part[1][lane][e];
      s += part[2][lane][e];
      s += part[3][lane][e];
      o[e] = s / inv_cnt;
    }
  }
}

// ---------------------------------------------------------------------------
// Block scores of one slab.  The rows of all heads are cut into tiles of 64
// query blocks (tile t = bh * nIT + i / 64, nIT = ceil(N / 64) tiles per
// head); a slab is the tiles t0 .. t0 + gridDim.y - 1, and its scores go to
// S[(tile - t0) * 64 + i % 64][j] (rows past N in a head's last tile are
// left unwritten).  grid = (ceil(N/64) key tiles, tiles in the slab), 256
// threads.  fp64 matrix cores: wavefront w computes the 16 x 64 scores of
// query rows i0 + 16w .. + 15 as four 16 x 16 tiles of v_mfma_f64_16x16x4,
// with the 64 x 32 slices of Qbar and Kbar for each 32 channels staged in
// LDS.  Every (i, j) is summed over d in the same order (slices in order,
// steps of 4 channels in order, the instruction's fixed 4-term sum), so equal
// key blocks get bit-equal scores (exact ties stay exact).
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// Four wavefronts per SIMD: 112 registers hold a wavefront's accumulators,
// operands and next-slice loads without spilling, and four 33.8 KB staging
// buffers fit a CU's LDS (long-video route 2.39 -> 2.33 ms against three).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void scores_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar,
                                                     int N, int D, int t0, int nIT, double* __restrict__ S) {
  __shared__ double As[64][33];
  __shared__ double Bs[64][33];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int tile = t0 + blockIdx.y;
  const int64_t bh = tile / nIT;
  const int i0 = (tile % nIT) * 64, j0 = blockIdx.x * 64;
  const double* qa = qbar + bh * N * D;
  const double* kb = kbar + bh * N * D;
  f64x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};

  // staging: thread loads rows lr + 16u (u = 0..3) of both slices, channels
  // lc, lc + 1 as one 16-byte load; rows past N read row N - 1 and store 0
  const int lr = threadIdx.x >> 4, lc = (threadIdx.x & 15) * 2;
  f64x2 ra[4], rb[4];
  auto load = [&](int d0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = lr + 16 * u;
      ra[u] = *(const f64x2*)(qa + (int64_t)min(i0 + row, N - 1) * D + d0 + lc);
      rb[u] = *(const f64x2*)(kb + (int64_t)min(j0 + row, N - 1) * D + d0 + lc);
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = lr + 16 * u;
      const bool qa_in = i0 + row < N, kb_in = j0 + row < N;
      As[row][lc] = qa_in ? ra[u].x : 0.0;
      As[row][lc + 1] = qa_in ? ra[u].y : 0.0;
      Bs[row][lc] = kb_in ? rb[u].x : 0.0;
      Bs[row][lc + 1] = kb_in ? rb[u].y : 0.0;
    }
  };
  load(0);
  for (int d0 = 0; d0 < D; d0 += 32) {
    store();
    __syncthreads();
    if (d0 + 32 < D) load(d0 + 32);  // in flight under this slice's products
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // A: lane holds Qbar[16w + lane % 16][4s + lane / 16]; B: Kbar[16t + lane % 16][4s + lane / 16]
      const double a = As[16 * w + r16][4 * s + g];
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Bs[16 * t + r16][4 * s + g], acc[t], 0, 0, 0);
    }
    __syncthreads();
  }
  // D of tile t: lane holds rows 4v + lane / 16, v = 0..3, column lane % 16
  const double rs = sqrt((double)D);
  double* out = S + (int64_t)blockIdx.y * 64 * N;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = j0 + 16 * t + r16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * w + 4 * v + g;
      if (i0 + r < N && j < N) out[(int64_t)r * N + j] = acc[t][v] / rs;
    }
  }
}

// Slab row r of a router launch: its (b*heads + h) and query block i, from
// the slab's first tile t0 (i >= N: a padding row of a head's last tile).
struct SlabRow {
  int64_t out;  // the row of the mask and the counts: (b*stride + h0 + h)*N + i
  int i;
};
__device__ inline SlabRow slab_row(int64_t r, int t0, int nIT, int N, const Heads& hd) {
  const int64_t tile = t0 + r / 64;
  SlabRow x;
  x.i = (int)((tile % nIT) * 64 + r % 64);
  x.out = hd.global(tile / nIT) * N + x.i;
  return x;
}

// ---------------------------------------------------------------------------
// Row routing.  One workgroup per (b, h, i) row; SLOTS = next power of two of
// N.  Keys live in LDS as (score, index) pairs; padding slots hold -inf and
// an index >= N so they sort last.
// ---------------------------------------------------------------------------
template <int THREADS>
__device__ inline double block_sum(double v, double* red) {
  // fixed-order tree: xor butterfly inside each wave, then waves in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

template <int THREADS>
__device__ inline double block_max(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < THREADS / 64; ++w) s = fmax(s, red[w]);
  __syncthreads();
  return s;
}

template <int SLOTS, int THREADS>
__global__ __launch_bounds__(THREADS) void route_rows_kernel(const double* __restrict__ S, int N, int words, int t0,
                                                             int nIT, Heads hd, float top_p, int k_floor,
                                                             uint32_t* __restrict__ mask,
                                                             int32_t* __restrict__ kv_cnt,
                                                             uint32_t* __restrict__ status) {
  constexpr int E = SLOTS / THREADS;
  __shared__ double key[SLOTS];
  __shared__ uint16_t idx[SLOTS];
  __shared__ uint32_t mw[SLOTS / 32];
  __shared__ double red[THREADS / 64];
  __shared__ double wtot[THREADS / 64];
  __shared__ int nstar_s;

  const int tid = threadIdx.x;
  const SlabRow sr = slab_row(blockIdx.x, t0, nIT, N, hd);
  if (sr.i >= N) return;  // padding row of a head's last tile
  const int64_t row = sr.out;
  const double* s = S + (int64_t)blockIdx.x * N;

  bool bad = false;
  double lmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * THREADS + tid;
    double v = -INFINITY;
    if (j < N) {
      v = s[j];
      if (!isfinite(v)) bad = true;
      lmax = fmax(lmax, v);
    }
    key[j] = v;
    idx[j] = (uint16_t)j;
  }
  for (int w = tid; w < SLOTS / 32; w += THREADS) mw[w] = 0u;
  if (tid == 0) nstar_s = N;
  const bool row_bad = __syncthreads_or(bad);

  if (row_bad) {
    // repair: a row whose scores cannot be ranked keeps every block
    for (int w = tid; w < words; w += THREADS) {
      const int lo = w * 32;
      const int nb = min(32, N - lo);
      mask[row * words + w] = nb == 32 ? 0xffffffffu : ((1u << nb) - 1u);
    }
    if (tid == 0) {
      if (kv_cnt) kv_cnt[row] = N;
      if (status) atomicOr(status, 1u);
    }
    return;
  }

  // softmax normaliser over all N blocks (max subtracted)
  const double M = block_max<THREADS>(lmax, red);
  double lz = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * THREADS + tid;
    if (j < N) lz += exp(key[j] - M);
  }
  const double Z = block_sum<THREADS>(lz, red);

  // bitonic sort into (score desc, index asc)
  for (int kk = 2; kk <= SLOTS; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < SLOTS / 2; t += THREADS) {
        const int i = 2 * t - (t & (jj - 1));
        const int p = i + jj;
        const double ki = key[i], kp = key[p];
        const uint16_t xi = idx[i], xp = idx[p];
        const bool i_first = (ki > kp) || (ki == kp && xi < xp);
        const bool want_i_first = (i & kk) == 0;
        if (i_first != want_i_first) {
          key[i] = kp; key[p] = ki;
          idx[i] = xp; idx[p] = xi;
        }
      }
      __syncthreads();
    }
  }

  // cumulative mass in sorted order: each thread owns E consecutive slots
  const double p = (double)top_p;
  double pm[E];
  double run = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int m = tid * E + e;
    pm[e] = (m < N) ? exp(key[m] - M) / Z : 0.0;
    run += pm[e];
  }
  // exclusive prefix of the per-thread totals: inclusive scan in each wave,
  // then wave totals in order
  double incl = run;
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  double base = incl - run;
  for (int w = 0; w < wave; ++w) base += wtot[w];

  int nstar;
  if (p >= 1.0) {
    nstar = N;
  } else if (p <= 0.0) {
    nstar = 0;
  } else {
    double c = base;
    int first = N;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int m = tid * E + e;
      c += pm[e];
      if (m < N && c >= p && first == N) first = m + 1;
    }
    if (first < N) atomicMin(&nstar_s, first);
    __syncthreads();
    nstar = nstar_s;
  }
  const int keep = min(N, max(k_floor, nstar));

#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int m = tid * E + e;
    if (m < keep) atomicOr(&mw[idx[m] >> 5], 1u << (idx[m] & 31));
  }
  __syncthreads();
  for (int w = tid; w < words; w += THREADS) mask[row * words + w] = mw[w];
  if (tid == 0 && kv_cnt) kv_cnt[row] = keep;
}

// ---------------------------------------------------------------------------
// Row routing for 256 < N <= 8192: selection instead of a full sort.  One
// workgroup per row; lane t owns blocks E t .. E t + E - 1: for N <= 512 one
// wavefront with E = 8 (four lanes form a mask word), above that
// ceil(N/32) lanes (rounded up to whole wavefronts) with E = 32 (lane t
// writes mask word t).  Blocks are ranked
// by a 64-bit key that orders fp64 scores exactly (ties by lower index), and
//   n* = the smallest prefix whose probability mass reaches p is found by
//        bisecting the key for the largest K with mass(key >= K) >= p,
//   the kept set = the top `keep` blocks is found by bisecting the key for the
//        largest K with count(key >= K) >= keep, ties taken in index order.
// The bisections split the scores' values (not the key codes) and, once at
// most one block per lane is left inside the bracket, wavefront 0 finishes
// over those blocks alone.  Every sum is a per-lane sequential sum in a
// fixed order followed by a fixed tree over lanes and wavefronts, so results
// do not depend on timing.
// ---------------------------------------------------------------------------
__device__ inline uint64_t order_key(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
// the double whose order_key is k
__device__ inline double key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}
// candidates per lane of the workgroup kept after a select bracket is
// compacted (wavefront 0 then holds all of them)
constexpr int kCand = 1;
// passes of a select search that split the scores' values
constexpr int kValueSteps = 40;

// Wavefront reductions for the select kernel: four DPP steps (lane xor 1 and
// xor 2 inside quads, then the 8- and 16-lane mirrors) leave every lane of a
// 16-lane row with the row's total; the four row totals are then combined
// in a fixed order.  Deterministic, and all VALU (no LDS round trips).
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_MIRROR8 = 0x141, DPP_MIRROR16 = 0x140;

template <int CTRL>
__device__ inline uint32_t dpp_move(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline uint64_t dpp_move(uint64_t x) {
  return (uint64_t)dpp_move<CTRL>((uint32_t)x) | ((uint64_t)dpp_move<CTRL>((uint32_t)(x >> 32)) << 32);
}
template <int CTRL>
__device__ inline double dpp_move(double x) {
  return __longlong_as_double((long long)dpp_move<CTRL>((uint64_t)__double_as_longlong(x)));
}
__device__ inline uint32_t read_lane(uint32_t x, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)x, l); }
__device__ inline uint64_t read_lane(uint64_t x, int l) {
  return (uint64_t)read_lane((uint32_t)x, l) | ((uint64_t)read_lane((uint32_t)(x >> 32), l) << 32);
}
__device__ inline double read_lane(double x, int l) {
  return __longlong_as_double((long long)read_lane((uint64_t)__double_as_longlong(x), l));
}

// a value every lane holds alike, moved to a scalar register, so that the
// compiler treats branches on it as uniform
__device__ inline uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ inline uint64_t uniform(uint64_t x) {
  return (uint64_t)uniform((uint32_t)x) | ((uint64_t)uniform((uint32_t)(x >> 32)) << 32);
}
__device__ inline double uniform(double x) {
  return __longlong_as_double((long long)uniform((uint64_t)__double_as_longlong(x)));
}

template <typename T, typename Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, dpp_move<DPP_XOR1>(v));
  v = op(v, dpp_move<DPP_XOR2>(v));
  v = op(v, dpp_move<DPP_MIRROR8>(v));
  v = op(v, dpp_move<DPP_MIRROR16>(v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}
struct AddOp {
  template <typename T>
  __device__ T operator()(T a, T b) const { return a + b; }
};
struct MaxOp {
  __device__ double operator()(double a, double b) const { return fmax(a, b); }
  __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a > b ? a : b; }
};
struct MinOp {
  __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a < b ? a : b; }
};

// Workgroup reductions through a double-buffered slot per wavefront: one
// barrier per reduction (a slot is rewritten two reductions later, after
// every wavefront has passed the barrier in between).  The wavefront totals
// are combined in wavefront order; every lane gets the result.
struct GroupRed {
  uint64_t* slot;  // LDS [2][2][4]: two values per wavefront, two buffers
  int nwaves, flip;
  template <typename T, typename Op>
  __device__ T reduce(T v, Op op) {
    const T w = wave_reduce(v, op);
    uint64_t* buf = slot + flip * 8;
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = to_bits(w);
    __syncthreads();
    T r = from_bits<T>(buf[0]);
    for (int i = 1; i < nwaves; ++i) r = op(r, from_bits<T>(buf[i]));
    flip ^= 1;
    return uniform(r);
  }
  // two reductions in one round (a and b of the same width)
  template <typename T, typename OpA, typename OpB>
  __device__ void reduce2(T* a, T* b, OpA opa, OpB opb) {
    const T wa = wave_reduce(*a, opa), wb = wave_reduce(*b, opb);
    uint64_t* buf = slot + flip * 8;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      buf[wave] = to_bits(wa);
      buf[4 + wave] = to_bits(wb);
    }
    __syncthreads();
    T ra = from_bits<T>(buf[0]), rb = from_bits<T>(buf[4]);
    for (int w = 1; w < nwaves; ++w) {
      ra = opa(ra, from_bits<T>(buf[w]));
      rb = opb(rb, from_bits<T>(buf[4 + w]));
    }
    *a = uniform(ra);
    *b = uniform(rb);
    flip ^= 1;
  }
  // a sum over the lanes (fixed order) and a count that is already uniform
  // in each wavefront, in one round
  __device__ double reduce_sum_count(double v, uint32_t wave_count, uint32_t* total) {
    const double w = wave_reduce(v, AddOp());
    uint64_t* buf = slot + flip * 8;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      buf[wave] = to_bits(w);
      buf[4 + wave] = wave_count;
    }
    __syncthreads();
    double r = from_bits<double>(buf[0]);
    uint32_t c = (uint32_t)buf[4];
    for (int i = 1; i < nwaves; ++i) {
      r += from_bits<double>(buf[i]);
      c += (uint32_t)buf[4 + i];
    }
    flip ^= 1;
    *total = uniform(c);
    return uniform(r);
  }
  // a count that is already uniform in each wavefront, summed over wavefronts
  __device__ uint32_t reduce_count(uint32_t wave_count) {
    uint64_t* buf = slot + flip * 8;
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = wave_count;
    __syncthreads();
    uint32_t c = (uint32_t)buf[0];
    for (int i = 1; i < nwaves; ++i) c += (uint32_t)buf[i];
    flip ^= 1;
    return uniform(c);
  }
  __device__ static uint64_t to_bits(double x) { return (uint64_t)__double_as_longlong(x); }
  __device__ static uint64_t to_bits(uint64_t x) { return x; }
  __device__ static uint64_t to_bits(uint32_t x) { return x; }
  template <typename T>
  __device__ static T from_bits(uint64_t x) {
    if constexpr (sizeof(T) == 4) return (T)(uint32_t)x;
    else return __builtin_bit_cast(T, x);
  }
};

// Three wavefronts per SIMD (at most 168 registers): the 32 keys and
// probabilities per lane take 128, and the passes are bound by latency
// (reductions and a barrier each), so the extra occupancy is worth the few
// registers the compiler moves to scratch outside the passes (long video
// 640 -> 525 us per slab when the passes themselves still reloaded some).
template <int E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void route_select_kernel(const double* __restrict__ S, int N, int words, int t0,
                                                           int nIT, Heads hd, float top_p, int k_floor,
                                                           uint32_t* __restrict__ mask,
                                                           int32_t* __restrict__ kv_cnt,
                                                           uint32_t* __restrict__ status) {
  __shared__ uint64_t red_slot[16];
  const int nwaves = blockDim.x >> 6;
  GroupRed gr{red_slot, nwaves, 0};
  const int tid = threadIdx.x;
  // rows in reverse slab order: the scores kernel wrote the last rows last,
  // so the first rows read here are the ones still in the memory-side cache
  const int64_t slab_r = (int64_t)gridDim.x - 1 - blockIdx.x;
  const SlabRow sr = slab_row(slab_r, t0, nIT, N, hd);
  if (sr.i >= N) return;  // padding row of a head's last tile (uniform over the workgroup)
  const int64_t row = sr.out;
  const double* s = S + slab_r * N;
  const int j0 = tid * E;

  double pr[E];
  uint64_t key[E];
  bool bad = false;
  double lmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // blocks past N read block N - 1 and hold -inf (their exp below is 0)
    const int j = j0 + e;
    const double x = s[min(j, N - 1)];
    const double v = j < N ? x : -INFINITY;
    bad = bad || (j < N && !isfinite(x));
    lmax = fmax(lmax, v);
    pr[e] = v;
  }
  if (__syncthreads_or(bad)) {
    if (tid < words) {
      const int nb = min(32, N - 32 * tid);
      mask[row * words + tid] = nb == 32 ? 0xffffffffu : ((1u << nb) - 1u);
    }
    if (tid == 0) {
      if (kv_cnt) kv_cnt[row] = N;
      if (status) atomicOr(status, 1u);
    }
    return;
  }
  const double M = gr.reduce(lmax, MaxOp());
  double lz = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = j0 + e < N;
    key[e] = in ? order_key(pr[e]) : 0ull;  // below every finite score
    pr[e] = exp(pr[e] - M);                 // -inf - M: exactly 0
    lz += pr[e];
  }
  const double Z = gr.reduce(lz, AddOp());
#pragma unroll
  for (int e = 0; e < E; ++e) pr[e] = pr[e] / Z;
  uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (j0 + e < N) {
      kmin = key[e] < kmin ? key[e] : kmin;
      kmax = key[e] > kmax ? key[e] : kmax;
    }
  gr.reduce2(&kmin, &kmax, MinOp(), MaxOp());

  // Candidates of a search bracket [lo, hi) once it holds at most kCand per
  // lane: copied out of the per-lane registers into LDS (wavefronts in
  // order, then register slot, then lane); wavefront 0 then takes kSlots per
  // lane (entries lane, lane + 64, ...), padding with key 0 (below every
  // finite score) and probability 0, and finishes the search alone.
  constexpr int kSlots = kCand * (E == 32 ? 4 : 1);
  __shared__ uint64_t cand_key[kCand * 256];
  __shared__ double cand_pr[kCand * 256];
  __shared__ uint32_t wt[4];
  __shared__ uint64_t res_key[2];  // wavefront 0's lo, hi
  __shared__ double res_f64[2];    // its m_hi, tie probability
  __shared__ uint32_t res_cnt[2];  // its c_lo, c_hi
  const int lane = tid & 63, wave = tid >> 6;
  const int threads = blockDim.x;
  // exclusive prefix over the workgroup of a per-lane count (lanes in order)
  auto exclusive_prefix = [&](uint32_t mine) -> uint32_t {
    uint32_t incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) wt[wave] = incl;
    __syncthreads();
    uint32_t r = incl - mine;
    for (int w = 0; w < wave; ++w) r += wt[w];
    return r;
  };
  auto compact = [&](uint64_t lo, uint64_t hi, bool with_mass) {
    // order: wavefronts in order, then slot e, then lanes; each wavefront's
    // offset comes from its count, a position from the lanes below it
    uint32_t mine = 0;  // uniform in the wavefront
#pragma unroll
    for (int e = 0; e < E; ++e) mine += (uint32_t)__popcll(__ballot(key[e] >= lo && key[e] < hi));
    __syncthreads();
    if (lane == 0) wt[wave] = mine;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wt[w];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool in = key[e] >= lo && key[e] < hi;
      const uint64_t bal = __ballot(in);
      if (in) {
        const uint32_t pos = base + (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        cand_key[pos] = key[e];
        if (with_mass) cand_pr[pos] = pr[e];
      }
      base += (uint32_t)__popcll(bal);
    }
    __syncthreads();
  };
  // Mass (when with_mass) and count of the blocks with key >= K.  A block
  // past N has key 0 and never counts (every K searched is at least kmin).
  // A lane adds fma(sel, pr, m) with sel 1 or 0 (the same bits as adding the
  // selected probability) into four partial sums by register slot mod 4,
  // then (m0 + m1) + (m2 + m3); the masses are then summed over lanes by a
  // fixed tree and over wavefronts in order.  The count is the wavefront's:
  // the population of each comparison's lane mask, summed on the scalar unit.
  auto mass_count_ge = [&](uint64_t K, bool with_mass, uint32_t* cnt) -> double {
    double m4[4] = {0.0, 0.0, 0.0, 0.0};
    uint32_t wc = 0;  // uniform in the wavefront
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool ge = key[e] >= K;
      if (with_mass) m4[e & 3] = fma(ge ? 1.0 : 0.0, pr[e], m4[e & 3]);
      wc += (uint32_t)__popcll(__ballot(ge));
    }
    if (with_mass) return gr.reduce_sum_count((m4[0] + m4[1]) + (m4[2] + m4[3]), wc, cnt);
    *cnt = gr.reduce_count(wc);
    return 0.0;
  };
  // the only key in [lo, hi) (callers know there is exactly one)
  auto only_key_in = [&](uint64_t lo, uint64_t hi) -> uint64_t {
    uint64_t k = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] >= lo && key[e] < hi) k = key[e];
    return gr.reduce(k, MaxOp());
  };
  // the probability of the blocks with key K (every tied block has the same
  // probability; any holder reports it)
  auto tie_pr = [&](uint64_t K) -> double {
    double t = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] == K) t = pr[e];
    return gr.reduce(t, MaxOp());
  };
  // Bisection of the key range for the largest K with pred(K): pred holds
  // at lo and fails at hi, with the counts of keys >= lo and >= hi (and, for
  // the mass search, the mass at hi) at hand.  The pivot halves the scores
  // between the bracket's ends (keys that order doubles leave long runs of
  // unused codes between the exponents of the scores present) for the first
  // kValueSteps passes (two distinct scores close to zero could take a
  // thousand value halvings to part), then the key codes, which end within
  // 64 more; it falls back to the middle key when the value midpoint is not
  // strictly inside.  Passes go over all blocks until the bracket holds at
  // most kCand blocks per lane; those are compacted and wavefront 0
  // finishes alone over them (no workgroup barrier per pass), adding what
  // lies at or above the bracket's top.  Once a single key lies in [lo, hi),
  // that key is the answer and the search stops (otherwise it runs until
  // hi = lo + 1).  At the end lo is a key present, no key lies in (lo, hi),
  // so "keys > lo" are exactly "keys >= hi", and for the mass search *ptie
  // is the probability of key lo.
  auto search = [&](bool with_mass, double target, uint64_t& lo, uint64_t& hi, uint32_t& c_lo, uint32_t& c_hi,
                    double& m_hi, double* ptie) {
    int steps = 0;
    auto pivot = [&]() -> uint64_t {
      if (steps++ < kValueSteps) {
        const double a = key_value(lo), b = key_value(hi);
        const uint64_t mid = order_key(a + (b - a) * 0.5);
        if (mid > lo && mid < hi) return mid;
      }
      return lo + (hi - lo) / 2;
    };
    auto step = [&](uint64_t mid, double m, uint32_t c_mid) {
      if (with_mass ? m >= target : c_mid >= (uint32_t)target) {
        lo = mid;
        c_lo = c_mid;
      } else {
        hi = mid;
        c_hi = c_mid;
        m_hi = m;
      }
    };
    // passes over all blocks while the bracket holds more than kCand per lane
    while (hi - lo > 1 && c_lo - c_hi > (uint32_t)(kCand * threads)) {
      const uint64_t mid = pivot();
      uint32_t c_mid;
      const double m = mass_count_ge(mid, with_mass, &c_mid);
      step(mid, m, c_mid);
    }
    lo = uniform(lo);
    hi = uniform(hi);
    c_lo = uniform(c_lo);
    c_hi = uniform(c_hi);
    if (hi - lo <= 1 || c_lo - c_hi == 1) {
      if (hi - lo > 1) lo = only_key_in(lo, hi);
      if (with_mass) *ptie = tie_pr(lo);
      return;
    }
    // then wavefront 0 over the compacted candidates, kSlots per lane; sums
    // over its lanes by the fixed tree of wave_reduce
    compact(lo, hi, with_mass);
    if (wave == 0) {
      const uint32_t n_cand = c_lo - c_hi;
      uint64_t ck[kSlots];
      double cp[kSlots];
#pragma unroll
      for (int r = 0; r < kSlots; ++r) {
        const uint32_t idx = (uint32_t)(lane + 64 * r);
        ck[r] = idx < n_cand ? cand_key[idx] : 0ull;
        cp[r] = with_mass && idx < n_cand ? cand_pr[idx] : 0.0;
      }
      const double m_above = m_hi;
      const uint32_t c_above = c_hi;
      while (hi - lo > 1 && c_lo - c_hi > 1) {
        const uint64_t mid = pivot();
        double acc = 0.0;
        uint32_t c = 0;  // uniform in the wavefront
#pragma unroll
        for (int r = 0; r < kSlots; ++r) {
          const bool ge = ck[r] >= mid;
          if (with_mass) acc = fma(ge ? 1.0 : 0.0, cp[r], acc);
          c += (uint32_t)__popcll(__ballot(ge));
        }
        step(mid, with_mass ? m_above + wave_reduce(acc, AddOp()) : 0.0, c_above + c);
      }
      if (hi - lo > 1) {  // the only candidate in [lo, hi)
        uint64_t k = 0;
#pragma unroll
        for (int r = 0; r < kSlots; ++r)
          if (ck[r] >= lo && ck[r] < hi) k = ck[r];
        lo = wave_reduce(k, MaxOp());
      }
      double t = 0.0;
      if (with_mass) {
#pragma unroll
        for (int r = 0; r < kSlots; ++r)
          if (ck[r] == lo) t = cp[r];
        t = wave_reduce(t, MaxOp());
      }
      if (lane == 0) {
        res_key[0] = lo;
        res_key[1] = hi;
        res_f64[0] = m_hi;
        res_f64[1] = t;
        res_cnt[0] = c_lo;
        res_cnt[1] = c_hi;
      }
    }
    __syncthreads();
    lo = uniform(res_key[0]);
    hi = uniform(res_key[1]);
    m_hi = uniform(res_f64[0]);
    c_lo = uniform(res_cnt[0]);
    c_hi = uniform(res_cnt[1]);
    if (with_mass) *ptie = uniform(res_f64[1]);
    __syncthreads();  // the results and candidates are rewritten by the next search
  };

  const double p = (double)top_p;
  uint32_t n_real = 0;
  const double total = mass_count_ge(kmin, true, &n_real);
  int nstar;
  uint64_t cut = 0;        // crossing key of the Top-p search
  uint32_t cut_above = 0;  // blocks with key > cut
  uint32_t cut_at = 0;     // blocks with key >= cut
  bool have_cut = false;
  if (p >= 1.0) {
    nstar = N;
  } else if (p <= 0.0) {
    nstar = 0;
  } else if (total < p) {
    nstar = N;  // rounding left the total below p: every block
  } else {
    // largest K with mass(key >= K) >= p: the key of the crossing block
    uint64_t lo = kmin, hi = kmax;
    uint32_t c_lo = n_real, c_hi = 0;
    double m_hi = mass_count_ge(hi, true, &c_hi);
    double above, ptie;
    uint32_t n_above;
    if (m_hi >= p) {
      lo = hi;
      c_lo = c_hi;
      above = 0.0;  // nothing above the largest key
      n_above = 0;
      ptie = tie_pr(lo);
    } else {
      search(true, p, lo, hi, c_lo, c_hi, m_hi, &ptie);
      above = m_hi;
      n_above = c_hi;
    }
    // blocks above the crossing key, then as many tied blocks as needed
    int need = 1;
    double c = above + ptie;
    const int n_tie = (int)(c_lo - n_above);
    while (c < p && need < n_tie) {
      c += ptie;
      ++need;
    }
    nstar = (int)n_above + need;
    cut = lo;
    cut_above = n_above;
    cut_at = c_lo;
    have_cut = true;
  }
  const int keep = min(N, max(k_floor, nstar));

  uint32_t word = 0u;  // bit e: block j0 + e is kept
  if (keep >= N) {
    const int nb = min(E, N - j0);
    word = nb >= 32 ? 0xffffffffu : (nb > 0 ? ((1u << nb) - 1u) : 0u);
  } else {
    // largest K with count(key >= K) >= keep: the Top-p crossing key itself
    // when the floor does not reach below its ties, else a key below it
    uint64_t lo = kmin;
    uint32_t n_above;
    if (have_cut && cut_at >= (uint32_t)keep) {
      lo = cut;
      n_above = cut_above;
    } else {
      uint64_t hi = kmax;
      uint32_t c_lo = n_real, c_hi = 0;
      double m_unused = 0.0;
      bool done = false;
      if (have_cut) {
        hi = cut;
        c_hi = cut_at;
      } else {
        mass_count_ge(hi, false, &c_hi);
        if (c_hi >= (uint32_t)keep) {
          lo = hi;
          n_above = 0;
          done = true;
        }
      }
      if (!done) {
        search(false, (double)keep, lo, hi, c_lo, c_hi, m_unused, nullptr);
        n_above = c_hi;
      }
    }
    const uint32_t need = (uint32_t)keep - n_above;
    // ties at the cut key, in index order: exclusive prefix over lanes
    uint32_t my_ties = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) my_ties += (j0 + e < N && key[e] == lo) ? 1u : 0u;
    uint32_t rank = exclusive_prefix(my_ties);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = j0 + e;
      if (j >= N) continue;
      bool kept = key[e] > lo;
      if (key[e] == lo) {
        kept = rank < need;
        ++rank;
      }
      if (kept) word |= 1u << e;
    }
  }
  if constexpr (E == 32) {
    if (tid < words) mask[row * words + tid] = word;
  } else {
    // E = 8: lanes 4w .. 4w + 3 hold the four bytes of mask word w
    static_assert(E == 8, "8 or 32 blocks per lane");
    uint32_t part = word << (8 * (tid & 3));
    part |= dpp_move<DPP_XOR1>(part);
    part |= dpp_move<DPP_XOR2>(part);
    if ((tid & 3) == 0 && (tid >> 2) < words) mask[row * words + (tid >> 2)] = part;
  }
  if (tid == 0 && kv_cnt) kv_cnt[row] = keep;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
hipError_t launch_pool(const void* q, const void* k, const Geo& g, int B, int L, const Heads& hd, int D, double* qbar,
                       double* kbar, uint32_t* status, bool clear_status, hipStream_t st) {
  const int nvec = hd.n * D / 8;
  const int chunks = (nvec + 63) / 64;
  dim3 grid(g.N * chunks, 2, B);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(256), 0, st, (const bf16_bits*)q, (const bf16_bits*)k, g, L, hd, D,
                     chunks, qbar, kbar, status, clear_status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free router entry point: the pooled means
// and one score slab live in this file-scope array (one copy per GPU, held
// until the process ends) instead of in a caller's workspace.  Host code
// never passes the array's name to a kernel or a copy: it uses the device
// address hipGetSymbolAddress returns for the current device, looked up once
// per device on its first use and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kRouteScratchBytes];

hipError_t route_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_scores_slab(const double* qbar, const double* kbar, int N, int D, int t0, int nt, double* S,
                              hipStream_t st) {
  hipLaunchKernelGGL(scores_kernel, dim3((N + 63) / 64, nt), dim3(256), 0, st, qbar, kbar, N, D, t0, (N + 63) / 64, S);
  return hipGetLastError();
}

hipError_t launch_route_slabs(const double* qbar, const double* kbar, int B, const Heads& hd, int N, int D,
                              float top_p, int k_floor, double* S, int64_t slab_tiles, uint32_t* mask,
                              int32_t* kv_cnt, uint32_t* status, hipStream_t st) {
  const int words = (N + 31) / 32;
  const int nIT = (N + 63) / 64;
  const int64_t tiles = (int64_t)B * hd.n * nIT;
  for (int64_t t0 = 0; t0 < tiles; t0 += slab_tiles) {
    const int nt = (int)std::min<int64_t>(slab_tiles, tiles - t0);
    hipError_t e = launch_scores_slab(qbar, kbar, N, D, (int)t0, nt, S, st);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)nt * 64);
#define FVA_ROUTE_CASE(SL, TH)                                                                                  \
    if (N <= SL) {                                                                                              \
      hipLaunchKernelGGL((route_rows_kernel<SL, TH>), grid, dim3(TH), 0, st, S, N, words, (int)t0, nIT, hd,    \
                         top_p, k_floor, mask, kv_cnt, status);                                                 \
      continue;                                                                                                 \
    }
    FVA_ROUTE_CASE(64, 64)
    FVA_ROUTE_CASE(128, 64)
    FVA_ROUTE_CASE(256, 64)
#undef FVA_ROUTE_CASE
    if (N <= 512) {  // one wavefront, 8 blocks per lane
      hipLaunchKernelGGL(route_select_kernel<8>, grid, dim3(64), 0, st, S, N, words, (int)t0, nIT, hd, top_p, k_floor,
                         mask, kv_cnt, status);
      continue;
    }
    if (N > 8192) return hipErrorInvalidValue;
    const int threads = 64 * ((words + 63) / 64);
    hipLaunchKernelGGL(route_select_kernel<32>, grid, dim3(threads), 0, st, S, N, words, (int)t0, nIT, hd, top_p,
                       k_floor, mask, kv_cnt, status);
  }
  return hipGetLastError();
}

}  // namespace fva
