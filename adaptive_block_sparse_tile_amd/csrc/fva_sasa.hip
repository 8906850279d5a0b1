// fva_sasa.hip -- slack-aware sparse augmentation, one-GPU form.
//
// FVAttn abstract and its summary (key modules 2 and 3): after runtime load
// balancing the non-critical ranks still have slack, which is filled with
// extra high-value attention blocks chosen from the attention scores, so that
// the critical path does not grow.  On one GPU the ranks are the 8 XCDs:
//   1. every row's cost is the time the attention kernel spends on it, in
//      steps of one 32-key half on its busiest SIMD: a query block of c_i
//      tokens (t_i = ceil(c_i / 32) row tiles on 8 wavefronts, two per SIMD;
//      a ragged block's tiles split their key halves over two wavefronts)
//      takes r_i = ceil(t_i / 2) steps per 64-key chunk, and a key block of
//      c_j tokens is ceil(c_j / 64) chunks, so row cost =
//      r_i * sum_{kept j} ceil(c_j / 64); a head's cost is the sum over its
//      rows;
//   2. heads go longest first (ties: lower head) to the XCD with the least
//      load so far (ties: lower XCD) -- the LPT rule of the attention
//      schedule; the heaviest XCD's load is the makespan M;
//   3. every other XCD x offers, in rounds r = 1..R, each of its rows (heads
//      in the order they were assigned to x, rows in block order) the r-th
//      block the router dropped from that row, in the router's order (score
//      descending, lower index first); the longest prefix of these offers
//      whose summed cost r_i * ceil(c_j / 64) fits M - load_x is added to the
//      mask.
// The attention then runs with each XCD serving only its own heads.
//
// The XCDs of one MI355X need not run at one speed (measured per-XCD time per
// unit of this cost differs by up to 9% on one box), so each XCD x may carry a
// relative speed w_x (per mille of the mean, measured from a trace): a head
// then goes to the XCD where it would finish first, (load_x + c) / w_x, the
// critical XCD m is the one with the largest load_m / w_m, and XCD x's slack is
// floor(load_m * w_x / w_m) - load_x.  All w_x equal is the unweighted rule.
#include <algorithm>

#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

constexpr int SASA_NXCD = 8;

// Register exchange between lanes (DPP; CTRL 0xB1: lane ^ 1, 0x4E: lane ^ 2,
// 0x141: lane 7 - i within each 8 lanes), 32 or 64 bits.
template <int CTRL>
__device__ inline int sasa_dpp(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline int64_t sasa_dpp(int64_t x) {
  const uint32_t lo = (uint32_t)sasa_dpp<CTRL>((int)(uint32_t)x), hi = (uint32_t)sasa_dpp<CTRL>((int)(x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ inline bool mask_bit(const uint32_t* row, int j) { return (row[j >> 5] >> (j & 31)) & 1u; }

__device__ inline int block_count(const Geo& g, int j) { return block_box(g, j).count; }
// steps of a query block per 64-key chunk on the busiest SIMD, and the chunks of a key block
__device__ inline int row_rate(const Geo& g, int i) { return ((block_count(g, i) + 31) / 32 + 1) / 2; }
__device__ inline int key_chunks(const Geo& g, int j) { return (block_count(g, j) + 63) / 64; }

// Per row (one wavefront), for the rows of one slab of score tiles (tiles
// of 64 query blocks of one head, scored by the router's own scores kernel,
// so the scores are bit-equal to what the router ranked): the row cost, the
// kept count, and the first R dropped blocks in the router's order (-1 past
// the last one), and a copy of the row's mask words into mask_out (null:
// augmented in place).  Workgroup r of the launch is slab row r (rows past N
// in a head's last tile do nothing).
__global__ __launch_bounds__(64) void sasa_cand_kernel(const double* __restrict__ S, int t0, int nIT,
                                                       const uint32_t* __restrict__ mask, Geo g, int words, int R,
                                                       int32_t* __restrict__ cand, int64_t* __restrict__ row_cost,
                                                       int32_t* __restrict__ kv_cnt, uint32_t* __restrict__ mask_out) {
  const int N = g.N;
  const int64_t tile = t0 + blockIdx.x / 64;
  const int i = (int)((tile % nIT) * 64 + blockIdx.x % 64);
  if (i >= N) return;
  const int64_t row = (tile / nIT) * N + i;
  const int lane = threadIdx.x;
  const uint32_t* m = mask + row * words;
  if (mask_out)
    for (int w = lane; w < words; w += 64) mask_out[row * words + w] = m[w];
  const double* s = S + (int64_t)blockIdx.x * N;
  int64_t kept_chunks = 0;
  int kept = 0;
  for (int j = lane; j < N; j += 64)
    if (mask_bit(m, j)) {
      kept_chunks += key_chunks(g, j);
      ++kept;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kept_chunks += __shfl_xor(kept_chunks, off);
    kept += __shfl_xor(kept, off);
  }
  if (lane == 0) {
    row_cost[row] = (int64_t)row_rate(g, (int)(row % N)) * kept_chunks;
    if (kv_cnt) kv_cnt[row] = kept;
  }
  // the previous pick (ps, pj); the next pick is the best dropped block that
  // comes after it in the order (s descending, j ascending)
  double ps = 0.0;
  int pj = -1;
  bool more = true;
  for (int r = 0; r < R; ++r) {
    double bs = 0.0;
    int bj = N;  // N: none
    if (more)
      for (int j = lane; j < N; j += 64) {
        if (mask_bit(m, j)) continue;
        const double x = s[j];
        if (!isfinite(x)) continue;  // (a row with a non-finite score keeps every block anyway)
        if (pj >= 0 && !(x < ps || (x == ps && j > pj))) continue;
        if (bj == N || x > bs || (x == bs && j < bj)) {
          bs = x;
          bj = j;
        }
      }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int oj = __shfl_xor(bj, off);
      if (oj != N && (bj == N || os > bs || (os == bs && oj < bj))) {
        bs = os;
        bj = oj;
      }
    }
    if (lane == 0) cand[row * R + r] = bj == N ? -1 : bj;
    if (bj == N) more = false;
    ps = bs;
    pj = bj;
  }
}

// Heads to XCDs, longest first (one workgroup of 1024), each to the XCD where
// it would finish first (ties: lower XCD).  Writes head_xcd, the heads of
// each XCD in assignment order (slot_head[x * BH + k]), their number (nh[x])
// and the XCD loads (load[x]).  Head costs: each head's rows are summed by a
// group of lanes (in a fixed order), the heads are ranked, and the costs are
// stored in rank order; the assignment runs on wavefront 0.
__global__ __launch_bounds__(1024) void sasa_lpt_kernel(const int64_t* __restrict__ row_cost, int N, int BH, XcdWeights w,
                                                        int32_t* __restrict__ head_xcd, int32_t* __restrict__ slot_head,
                                                        int32_t* __restrict__ nh, int64_t* __restrict__ load) {
  extern __shared__ int64_t hs[];  // [BH] head costs, [BH] costs in rank order, then [BH] int32 heads in rank order
  int64_t* hcost = hs;
  int64_t* rcost = hs + BH;
  int32_t* horder = (int32_t*)(hs + 2 * BH);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // lanes per head: a power of two up to 64, so that every head's group fits in one wavefront
  int per = 64;
  while (per > 1 && per * BH > (int)blockDim.x) per >>= 1;
  const int heads_per_pass = (int)blockDim.x / per;
  for (int x0 = 0; x0 < BH; x0 += heads_per_pass) {
    const int x = x0 + tid / per, sub = tid % per;
    int64_t c = 0;
    if (x < BH)
      for (int i = sub; i < N; i += per) c += row_cost[(int64_t)x * N + i];
    for (int off = per / 2; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (x < BH && sub == 0) hcost[x] = c;
  }
  __syncthreads();
  for (int x = tid; x < BH; x += blockDim.x) {
    int r = 0;
    for (int y = 0; y < BH; ++y)
      if (hcost[y] > hcost[x] || (hcost[y] == hcost[x] && y < x)) ++r;
    horder[r] = x;
    rcost[r] = hcost[x];
  }
  __syncthreads();
  if (wave != 0) return;
  // The assignment on wavefront 0: lane x (mod 8) holds XCD x's load, head
  // count and weight; the XCD of the earliest finish comes from three
  // register exchanges inside each group of 8 lanes (lane i with i ^ 1, then
  // i ^ 2, then 7 - i), every group computing the same thing.  The ranked
  // heads and costs are read 64 at a time into the lanes and taken from
  // there one by one.  Loads stay below 2^43 and weights below 2^20 (the
  // host's limits), so load x weight is exact in 64 bits.
  const int xl = lane & (SASA_NXCD - 1);
  uint32_t wx = (uint32_t)w.w[0];
#pragma unroll
  for (int x = 1; x < SASA_NXCD; ++x)
    if (xl == x) wx = (uint32_t)w.w[x];
  auto mul = [](uint64_t a, uint32_t b) -> uint64_t {  // a < 2^43, b < 2^20
    return (uint64_t)(uint32_t)a * b + ((uint64_t)((uint32_t)(a >> 32) * b) << 32);
  };
  int64_t ld = 0;
  int cnt = 0;
  for (int r0 = 0; r0 < BH; r0 += 64) {
    const int rr = r0 + lane;
    const int my_hd = rr < BH ? horder[rr] : 0;
    const int64_t my_c = rr < BH ? rcost[rr] : 0;
    const int n = min(64, BH - r0);
    for (int i = 0; i < n; ++i) {
      const int hd = __builtin_amdgcn_readlane(my_hd, i);
      const int64_t c = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(my_c >> 32), i) << 32) |
                                  (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)my_c, i));
      // earliest finish (ld + c) / w, ties to the lower XCD
      int64_t a = ld + c;
      uint32_t aw = wx;
      int bx = xl;
      auto take = [&](int64_t pa, uint32_t pw, int px) {
        const uint64_t lhs = mul((uint64_t)pa, aw), rhs = mul((uint64_t)a, pw);  // pa / pw vs a / aw
        if (lhs < rhs || (lhs == rhs && px < bx)) {
          a = pa;
          aw = pw;
          bx = px;
        }
      };
      take(sasa_dpp<0xB1>(a), (uint32_t)sasa_dpp<0xB1>((int)aw), sasa_dpp<0xB1>(bx));     // lane ^ 1
      take(sasa_dpp<0x4E>(a), (uint32_t)sasa_dpp<0x4E>((int)aw), sasa_dpp<0x4E>(bx));     // lane ^ 2
      take(sasa_dpp<0x141>(a), (uint32_t)sasa_dpp<0x141>((int)aw), sasa_dpp<0x141>(bx));  // 7 - lane, within 8
      const int best = __builtin_amdgcn_readfirstlane(bx);
      const int slot = __builtin_amdgcn_readlane(cnt, best);
      if (lane == 0) {
        slot_head[best * BH + slot] = hd;
        head_xcd[hd] = best;
      }
      if (xl == best) {
        ld += c;
        ++cnt;
      }
    }
  }
  if (lane < SASA_NXCD) {
    nh[lane] = cnt;
    load[lane] = ld;
  }
}

// One workgroup per XCD: the offers in (round, head slot, row) order, an
// inclusive prefix sum of their costs, and every offer whose prefix fits the
// slack is added (offers without a block cost 0 and add nothing).  added[x]
// receives the added cost.
__global__ __launch_bounds__(1024) void sasa_take_kernel(Geo g, int words, int R, int BH, XcdWeights w,
                                                         const int32_t* __restrict__ cand,
                                                         const int32_t* __restrict__ slot_head,
                                                         const int32_t* __restrict__ nh,
                                                         const int64_t* __restrict__ load, uint32_t* __restrict__ mask,
                                                         int32_t* __restrict__ kv_cnt, int64_t* __restrict__ added) {
  __shared__ int64_t wsum[16];
  __shared__ int64_t base_s, taken_s;
  const int x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = g.N;
  // the critical XCD: largest load / weight (ties: lower XCD)
  int m = 0;
  for (int y = 1; y < SASA_NXCD; ++y)
    if (load[y] * w.w[m] > load[m] * w.w[y]) m = y;
  const int64_t slack = load[m] * w.w[x] / w.w[m] - load[x];
  const int64_t Q = (int64_t)nh[x] * N;
  const int64_t total = Q * R;
  if (tid == 0) {
    base_s = 0;
    taken_s = 0;
  }
  __syncthreads();
  for (int64_t t0 = 0; t0 < total; t0 += 1024) {
    const int64_t base = base_s;
    if (base > slack) break;  // (uniform: read after the barrier that ended the previous tile)
    const int64_t o = t0 + tid;
    int64_t cost = 0;
    int64_t row = -1;
    int j = -1;
    if (o < total) {
      const int r = (int)(o / Q);
      const int64_t rem = o % Q;
      const int k = (int)(rem / N), i = (int)(rem % N);
      row = (int64_t)slot_head[x * BH + k] * N + i;
      j = cand[row * R + r];
      if (j >= 0) cost = (int64_t)row_rate(g, i) * key_chunks(g, j);
    }
    // inclusive scan over the workgroup
    int64_t v = cost;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(v, off);
      if (lane >= off) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int64_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int64_t incl = base + before + v;
    if (j >= 0 && incl <= slack) {
      atomicOr(&mask[row * words + (j >> 5)], 1u << (j & 31));
      if (kv_cnt) atomicAdd(&kv_cnt[row], 1);
      atomicAdd((unsigned long long*)&taken_s, (unsigned long long)cost);
    }
    __syncthreads();
    if (tid == 1023) base_s = incl;
    __syncthreads();
  }
  if (tid == 0) added[x] = taken_s;
}

hipError_t launch_sasa(const double* qbar, const double* kbar, int D, const uint32_t* mask_in, const Geo& g, int BH,
                       int R, const XcdWeights& w, const double* S_ready, double* S, int64_t slab_tiles,
                       uint32_t* mask_out, int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, int32_t* cand,
                       int64_t* row_cost, int32_t* slot_head, int32_t* nh, hipStream_t st) {
  const int words = (g.N + 31) / 32;
  uint32_t* copy_to = mask_out != mask_in ? mask_out : nullptr;
  const int nIT = (g.N + 63) / 64;
  const int64_t tiles = (int64_t)BH * nIT;
  if (S_ready) slab_tiles = tiles;  // the router's one slab holds every tile
  for (int64_t t0 = 0; t0 < tiles; t0 += slab_tiles) {
    const int nt = (int)std::min<int64_t>(slab_tiles, tiles - t0);
    const double* slab = S_ready;
    if (!slab) {
      hipError_t e = launch_scores_slab(qbar, kbar, g.N, D, (int)t0, nt, S, st);
      if (e != hipSuccess) return e;
      slab = S;
    }
    hipLaunchKernelGGL(sasa_cand_kernel, dim3((unsigned)nt * 64), dim3(64), 0, st, slab, (int)t0, nIT, mask_in, g,
                       words, R, cand, row_cost, kv_cnt, copy_to);
  }
  hipLaunchKernelGGL(sasa_lpt_kernel, dim3(1), dim3(1024), (size_t)BH * 20, st, row_cost, g.N, BH, w, head_xcd,
                     slot_head, nh, xcd_load);
  hipLaunchKernelGGL(sasa_take_kernel, dim3(SASA_NXCD), dim3(1024), 0, st, g, words, R, BH, w, cand, slot_head, nh,
                     xcd_load, mask_out, kv_cnt, xcd_load + SASA_NXCD);
  return hipGetLastError();
}

}  // namespace fva
