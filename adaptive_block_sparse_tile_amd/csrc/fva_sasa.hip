// fva_sasa.hip -- slack-aware sparse augmentation, one-GPU form.
//
// FVAttn abstract and its summary (key modules 2 and 3): after runtime load
// balancing the non-critical ranks still have slack, which is filled with
// extra high-value attention blocks chosen from the attention scores, so that
// the critical path does not grow.  On one GPU the ranks are the 8 XCDs:
//   1. every row's cost is its real token pairs, c_i * sum_{kept j} c_j, and
//      a head's cost is the sum over its rows;
//   2. heads go longest first (ties: lower head) to the XCD with the least
//      load so far (ties: lower XCD) -- the LPT rule of the attention
//      schedule; the heaviest XCD's load is the makespan M;
//   3. every other XCD x offers, in rounds r = 1..R, each of its rows (heads
//      in the order they were assigned to x, rows in block order) the r-th
//      block the router dropped from that row, in the router's order (score
//      descending, lower index first); the longest prefix of these offers
//      whose summed cost c_i * c_j fits M - load_x is added to the mask.
// The attention then runs with each XCD serving only its own heads.
#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

constexpr int SASA_NXCD = 8;

__device__ inline bool mask_bit(const uint32_t* row, int j) { return (row[j >> 5] >> (j & 31)) & 1u; }

__device__ inline int block_count(const Geo& g, int j) { return block_box(g, j).count; }

// Per row (one wavefront): the row cost, the kept count, and the first R
// dropped blocks in the router's order (-1 past the last one).
__global__ __launch_bounds__(64) void sasa_cand_kernel(const double* __restrict__ S, const uint32_t* __restrict__ mask,
                                                       Geo g, int words, int R, int32_t* __restrict__ cand,
                                                       int64_t* __restrict__ row_cost,
                                                       int32_t* __restrict__ kv_cnt) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = g.N;
  const uint32_t* m = mask + row * words;
  const double* s = S + row * N;
  int64_t kept_tok = 0;
  int kept = 0;
  for (int j = lane; j < N; j += 64)
    if (mask_bit(m, j)) {
      kept_tok += block_count(g, j);
      ++kept;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    kept_tok += __shfl_xor(kept_tok, off);
    kept += __shfl_xor(kept, off);
  }
  if (lane == 0) {
    row_cost[row] = (int64_t)block_count(g, (int)(row % N)) * kept_tok;
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

// Heads to XCDs, longest first (one workgroup).  Writes head_xcd, the heads
// of each XCD in assignment order (slot_head[x * BH + k]), their number
// (nh[x]) and the XCD loads (load[x]); makespan = max load.
__global__ __launch_bounds__(256) void sasa_lpt_kernel(const int64_t* __restrict__ row_cost, int N, int BH,
                                                       int32_t* __restrict__ head_xcd, int32_t* __restrict__ slot_head,
                                                       int32_t* __restrict__ nh, int64_t* __restrict__ load) {
  extern __shared__ int64_t hs[];  // [BH] head costs, then [BH] int32 order
  int64_t* hcost = hs;
  int32_t* horder = (int32_t*)(hs + BH);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  for (int x = wave; x < BH; x += nwaves) {
    int64_t c = 0;
    for (int i = lane; i < N; i += 64) c += row_cost[(int64_t)x * N + i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if (lane == 0) hcost[x] = c;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < BH; x += blockDim.x) {
    int r = 0;
    for (int y = 0; y < BH; ++y)
      if (hcost[y] > hcost[x] || (hcost[y] == hcost[x] && y < x)) ++r;
    horder[r] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t ld[SASA_NXCD];
    int cnt[SASA_NXCD];
    for (int x = 0; x < SASA_NXCD; ++x) ld[x] = 0, cnt[x] = 0;
    for (int r = 0; r < BH; ++r) {
      const int hd = horder[r];
      int best = 0;
      for (int x = 1; x < SASA_NXCD; ++x)
        if (ld[x] < ld[best]) best = x;
      ld[best] += hcost[hd];
      head_xcd[hd] = best;
      slot_head[best * BH + cnt[best]] = hd;
      ++cnt[best];
    }
    for (int x = 0; x < SASA_NXCD; ++x) {
      nh[x] = cnt[x];
      load[x] = ld[x];
    }
  }
}

// One workgroup per XCD: the offers in (round, head slot, row) order, an
// inclusive prefix sum of their costs, and every offer whose prefix fits the
// slack is added (offers without a block cost 0 and add nothing).  added[x]
// receives the added cost.
__global__ __launch_bounds__(1024) void sasa_take_kernel(Geo g, int words, int R, int BH,
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
  int64_t M = 0;
  for (int y = 0; y < SASA_NXCD; ++y) M = max(M, load[y]);
  const int64_t slack = M - load[x];
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
      if (j >= 0) cost = (int64_t)block_count(g, i) * block_count(g, j);
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

hipError_t launch_sasa(const double* S, const uint32_t* mask_in, const Geo& g, int BH, int R, uint32_t* mask_out,
                       int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, int32_t* cand, int64_t* row_cost,
                       int32_t* slot_head, int32_t* nh, hipStream_t st) {
  const int words = (g.N + 31) / 32;
  const int64_t rows = (int64_t)BH * g.N;
  if (mask_out != mask_in) {
    hipError_t e = hipMemcpyAsync(mask_out, mask_in, (size_t)rows * words * sizeof(uint32_t),
                                  hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sasa_cand_kernel, dim3((unsigned)rows), dim3(64), 0, st, S, mask_in, g, words, R, cand, row_cost,
                     kv_cnt);
  hipLaunchKernelGGL(sasa_lpt_kernel, dim3(1), dim3(256), (size_t)BH * 12, st, row_cost, g.N, BH, head_xcd, slot_head,
                     nh, xcd_load);
  hipLaunchKernelGGL(sasa_take_kernel, dim3(SASA_NXCD), dim3(1024), 0, st, g, words, R, BH, cand, slot_head, nh,
                     xcd_load, mask_out, kv_cnt, xcd_load + SASA_NXCD);
  return hipGetLastError();
}

}  // namespace fva
