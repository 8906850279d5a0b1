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
//   route_rows_kernel  N <= 512: one wavefront per row: softmax, bitonic
//                      sort on (score desc, index asc), scan, Top-p count,
//                      floor, mask words and kept count
//   route_select_kernel N > 512: the same decisions by bisection on
//                      order-preserving keys (no full sort)
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
                                                   Geo g, int L, int heads, int D, int chunks,
                                                   double* __restrict__ qbar, double* __restrict__ kbar,
                                                   uint32_t* __restrict__ status) {
  const int n = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int which = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *status = 0u;

  const bf16_bits* x = which == 0 ? q : k;
  double* out = which == 0 ? qbar : kbar;
  const int nvec = heads * D / 8;
  const int vec = chunk * 64 + lane;
  const bool active = vec < nvec;
  const Box bx = block_box(g, n);
  const int64_t row_stride = (int64_t)heads * D;
  const bf16_bits* base = x + (int64_t)b * L * row_stride + (int64_t)vec * 8;

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
    double* o = out + (((int64_t)b * heads + h) * g.N + n) * D + d0;
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
// Block scores.  grid = (ceil(N/64), ceil(N/64), B*heads), 256 threads, each
// thread a 4x4 set of outputs i = i0 + ty + 16a, j = j0 + tx + 16c.  The dot
// product runs over d in increasing order for every (i, j), so equal key
// blocks get bit-equal scores (exact ties stay exact).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qbar, const double* __restrict__ kbar,
                                                     int N, int D, double* __restrict__ S) {
  __shared__ double As[64][33];
  __shared__ double Bs[64][33];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int64_t bh = blockIdx.z;
  const double* qa = qbar + bh * N * D;
  const double* kb = kbar + bh * N * D;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;

  for (int d0 = 0; d0 < D; d0 += 32) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = threadIdx.x + u * 256;  // 0..2047
      const int r = e >> 5, c = e & 31;
      As[r][c] = (i0 + r < N) ? qa[(int64_t)(i0 + r) * D + d0 + c] : 0.0;
      Bs[r][c] = (j0 + r < N) ? kb[(int64_t)(j0 + r) * D + d0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[ty + 16 * a][kk];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[tx + 16 * c][kk];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = fma(av[a], bv[c], acc[a][c]);
    }
    __syncthreads();
  }
  const double rs = sqrt((double)D);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty + 16 * a;
    if (i >= N) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tx + 16 * c;
      if (j < N) S[(bh * N + i) * N + j] = acc[a][c] / rs;
    }
  }
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
__global__ __launch_bounds__(THREADS) void route_rows_kernel(const double* __restrict__ S, int N, int words,
                                                             float top_p, int k_floor, uint32_t* __restrict__ mask,
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
  const int64_t row = blockIdx.x;
  const double* s = S + row * N;

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
// Row routing for large N (N > 512): selection instead of a full sort.
// One workgroup of ceil(N/32) lanes (rounded up to whole wavefronts) per row;
// lane t owns blocks 32t .. 32t+31 and writes mask word t.  Blocks are ranked
// by a 64-bit key that orders fp64 scores exactly (ties by lower index), and
//   n* = the smallest prefix whose probability mass reaches p is found by
//        bisecting the key for the largest K with mass(key >= K) >= p,
//   the kept set = the top `keep` blocks is found by bisecting the key for the
//        largest K with count(key >= K) >= keep, ties taken in index order.
// Every sum is a per-lane sequential sum in index order followed by a fixed
// tree over lanes and wavefronts, so results do not depend on timing.
// ---------------------------------------------------------------------------
__device__ inline uint64_t order_key(double d) {
  const uint64_t b = (uint64_t)__double_as_longlong(d);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

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
    return r;
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
    *a = ra;
    *b = rb;
    flip ^= 1;
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

__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ S, int N, int words,
                                                           float top_p, int k_floor, uint32_t* __restrict__ mask,
                                                           int32_t* __restrict__ kv_cnt,
                                                           uint32_t* __restrict__ status) {
  __shared__ uint64_t red_slot[16];
  const int nwaves = blockDim.x >> 6;
  GroupRed gr{red_slot, nwaves, 0};
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const double* s = S + row * N;
  const int j0 = tid * 32;

  double pr[32];
  uint64_t key[32];
  bool bad = false;
  double lmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int j = j0 + e;
    double v = -INFINITY;
    if (j < N) {
      v = s[j];
      if (!isfinite(v)) bad = true;
      lmax = fmax(lmax, v);
    }
    pr[e] = v;
  }
  if (__syncthreads_or(bad)) {
    if (tid < words) {
      const int nb = min(32, N - j0);
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
  for (int e = 0; e < 32; ++e) {
    const bool in = j0 + e < N;
    key[e] = in ? order_key(pr[e]) : 0ull;  // below every finite score
    pr[e] = in ? exp(pr[e] - M) : 0.0;
    lz += pr[e];
  }
  const double Z = gr.reduce(lz, AddOp());
#pragma unroll
  for (int e = 0; e < 32; ++e) pr[e] = pr[e] / Z;
  uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int e = 0; e < 32; ++e)
    if (j0 + e < N) {
      kmin = key[e] < kmin ? key[e] : kmin;
      kmax = key[e] > kmax ? key[e] : kmax;
    }
  gr.reduce2(&kmin, &kmax, MinOp(), MaxOp());
  // mass and count of the blocks with key >= K (fixed summation order)
  auto mass_count_ge = [&](uint64_t K, uint32_t* cnt) -> double {
    double m = 0.0;
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const bool ge = j0 + e < N && key[e] >= K;
      m += ge ? pr[e] : 0.0;
      c += ge ? 1u : 0u;
    }
    double cd = (double)c;  // counts are exact in double
    gr.reduce2(&m, &cd, AddOp(), AddOp());
    *cnt = (uint32_t)cd;
    return m;
  };
  // the only key in [lo, hi) (callers know there is exactly one)
  auto only_key_in = [&](uint64_t lo, uint64_t hi) -> uint64_t {
    uint64_t k = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (j0 + e < N && key[e] >= lo && key[e] < hi) k = key[e];
    return gr.reduce(k, MaxOp());
  };

  // Both searches bisect the key range [lo, hi] keeping a predicate true at
  // lo and false at hi, with the counts of keys >= lo and >= hi at hand:
  // once a single key lies in [lo, hi), that key is the answer and the
  // search stops (otherwise it runs until hi = lo + 1).  At the end no key
  // lies in (lo, hi), so "keys > lo" are exactly "keys >= hi".
  const double p = (double)top_p;
  uint32_t n_real = 0;
  const double total = mass_count_ge(kmin, &n_real);
  int nstar;
  uint64_t cut = 0;        // crossing key of the Top-p search
  uint32_t cut_above = 0;  // blocks with key > cut
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
    double m_hi = mass_count_ge(hi, &c_hi);
    double above;
    uint32_t n_above;
    if (m_hi >= p) {
      lo = hi;
      c_lo = c_hi;
      above = 0.0;  // nothing above the largest key
      n_above = 0;
    } else {
      while (hi - lo > 1) {
        if (c_lo - c_hi == 1) {
          lo = only_key_in(lo, hi);
          break;
        }
        const uint64_t mid = lo + (hi - lo) / 2;
        uint32_t c_mid;
        const double m = mass_count_ge(mid, &c_mid);
        if (m >= p) {
          lo = mid;
          c_lo = c_mid;
        } else {
          hi = mid;
          c_hi = c_mid;
          m_hi = m;
        }
      }
      above = m_hi;
      n_above = c_hi;
    }
    // blocks above the crossing key, then as many tied blocks as needed
    double ptie = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (key[e] == lo) ptie = pr[e];
    // every tied block has the same probability; any holder reports it
    ptie = gr.reduce(ptie, MaxOp());
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
    have_cut = true;
  }
  const int keep = min(N, max(k_floor, nstar));

  uint32_t word = 0u;
  if (keep >= N) {
    const int nb = min(32, N - j0);
    word = nb >= 32 ? 0xffffffffu : (nb > 0 ? ((1u << nb) - 1u) : 0u);
  } else {
    // largest K with count(key >= K) >= keep; when the floor does not bind,
    // that is the Top-p crossing key itself
    uint64_t lo = kmin;
    uint32_t n_above;
    if (have_cut && keep == nstar) {
      lo = cut;
      n_above = cut_above;
    } else {
      uint64_t hi = kmax;
      uint32_t c_lo = n_real, c_hi = 0;
      mass_count_ge(hi, &c_hi);
      if (c_hi >= (uint32_t)keep) {
        lo = hi;
        n_above = 0;
      } else {
        while (hi - lo > 1) {
          if (c_lo - c_hi == 1) {
            lo = only_key_in(lo, hi);
            break;
          }
          const uint64_t mid = lo + (hi - lo) / 2;
          uint32_t c_mid;
          mass_count_ge(mid, &c_mid);
          if (c_mid >= (uint32_t)keep) {
            lo = mid;
            c_lo = c_mid;
          } else {
            hi = mid;
            c_hi = c_mid;
          }
        }
        n_above = c_hi;
      }
    }
    const uint32_t need = (uint32_t)keep - n_above;
    // ties at the cut key, in index order: exclusive prefix over lanes
    uint32_t my_ties = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) my_ties += (j0 + e < N && key[e] == lo) ? 1u : 0u;
    uint32_t incl = my_ties;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    __shared__ uint32_t wt[4];
    __syncthreads();
    if (lane == 63) wt[wave] = incl;
    __syncthreads();
    uint32_t rank = incl - my_ties;
    for (int w = 0; w < wave; ++w) rank += wt[w];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
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
  if (tid < words) mask[row * words + tid] = word;
  if (tid == 0 && kv_cnt) kv_cnt[row] = keep;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
hipError_t launch_pool(const void* q, const void* k, const Geo& g, int B, int L, int heads, int D, double* qbar,
                       double* kbar, uint32_t* status, hipStream_t st) {
  const int nvec = heads * D / 8;
  const int chunks = (nvec + 63) / 64;
  dim3 grid(g.N * chunks, 2, B);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(256), 0, st, (const bf16_bits*)q, (const bf16_bits*)k, g, L, heads, D,
                     chunks, qbar, kbar, status);
  return hipGetLastError();
}

hipError_t launch_scores(const double* qbar, const double* kbar, int BH, int N, int D, double* S, hipStream_t st) {
  dim3 grid((N + 63) / 64, (N + 63) / 64, BH);
  hipLaunchKernelGGL(scores_kernel, grid, dim3(256), 0, st, qbar, kbar, N, D, S);
  return hipGetLastError();
}

hipError_t launch_route_rows(const double* S, int64_t rows, int N, float top_p, int k_floor, uint32_t* mask,
                             int32_t* kv_cnt, uint32_t* status, hipStream_t st) {
  const int words = (N + 31) / 32;
  dim3 grid((unsigned)rows);
#define FVA_ROUTE_CASE(SL, TH)                                                                                 \
  if (N <= SL) {                                                                                               \
    hipLaunchKernelGGL((route_rows_kernel<SL, TH>), grid, dim3(TH), 0, st, S, N, words, top_p, k_floor, mask, \
                       kv_cnt, status);                                                                        \
    return hipGetLastError();                                                                                  \
  }
  FVA_ROUTE_CASE(64, 64)
  FVA_ROUTE_CASE(128, 64)
  FVA_ROUTE_CASE(256, 64)
  FVA_ROUTE_CASE(512, 64)
#undef FVA_ROUTE_CASE
  if (N <= 8192) {
    const int threads = 64 * ((words + 63) / 64);
    hipLaunchKernelGGL(route_select_kernel, grid, dim3(threads), 0, st, S, N, words, top_p, k_floor, mask, kv_cnt,
                       status);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace fva
