// fva_static.hip -- static block masks (local partitions plus anchor slabs).
//
// Sol-Attn article (bjdmk.com.cn), section 3: tokens of one local window
// attend to each other in full, and anchor tokens connect every window: a
// query-key pair is kept when both sit in the same local window or when
// either one is an anchor.  Here the same rule acts on the (t, y, x)
// coordinates of the video blocks instead of on token positions: the local
// windows are boxes of lt x lh x lw blocks (a partition of the block grid),
// and the anchors are the block slabs whose temporal index is a multiple of
// anchor_t (0: no anchors).  On a one-dimensional grid of one-token blocks
// this is the article's token mask with block_size = lt and
// anchor_stride = anchor_t.
#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

// One workgroup per (b, h, query block); lanes walk the mask words.
__global__ __launch_bounds__(64) void static_mask_kernel(Geo g, int lt, int lh, int lw, int anchor_t, int words,
                                                         uint32_t* __restrict__ mask, int32_t* __restrict__ kv_cnt) {
  const int64_t row = blockIdx.x;  // (b*heads + h)*N + i
  const int i = (int)(row % g.N);
  const int it = i / (g.nH * g.nW), ih = (i / g.nW) % g.nH, iw = i % g.nW;
  const bool q_anchor = anchor_t > 0 && it % anchor_t == 0;
  __shared__ int total;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  int mine = 0;
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    uint32_t bits = 0u;
    for (int b = 0; b < 32; ++b) {
      const int j = w * 32 + b;
      if (j >= g.N) break;
      const int jt = j / (g.nH * g.nW), jh = (j / g.nW) % g.nH, jw = j % g.nW;
      const bool local = it / lt == jt / lt && ih / lh == jh / lh && iw / lw == jw / lw;
      const bool anchor = q_anchor || (anchor_t > 0 && jt % anchor_t == 0);
      if (local || anchor) bits |= 1u << b;
    }
    mask[row * words + w] = bits;
    mine += __builtin_popcount(bits);
  }
  atomicAdd(&total, mine);
  __syncthreads();
  if (threadIdx.x == 0 && kv_cnt) kv_cnt[row] = total;
}

hipError_t launch_static_mask(const Geo& g, int64_t rows, int lt, int lh, int lw, int anchor_t, uint32_t* mask,
                              int32_t* kv_cnt, hipStream_t st) {
  const int words = (g.N + 31) / 32;
  hipLaunchKernelGGL(static_mask_kernel, dim3((unsigned)rows), dim3(64), 0, st, g, lt, lh, lw, anchor_t, words, mask,
                     kv_cnt);
  return hipGetLastError();
}

}  // namespace fva
