// fva_dev.h -- device-side shared definitions of libfva (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fva {

typedef uint16_t bf16_bits;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Geometry of the tiled token grid, passed by value to kernels.
// Blocks are numbered n = (it*nH + ih)*nW + iw; the tokens of a block are laid
// out row-major over (t, y, x) inside it.  A block's first position in the
// block-ordered token sequence has the closed form
//   start(n) = it*bt*H*W + et*(ih*bh)*W + et*eh*(iw*bw)
// (all earlier block rows along t cover bt*H*W tokens each, and so on).
struct Geo {
  int T, H, W, bt, bh, bw;
  int nT, nH, nW, N;
};

// The heads a launch works on: heads h0 .. h0 + n - 1 of tensors with
// `stride` heads per token, and the matching rows of [B, stride, N, ...]
// masks and counts.  A whole-tensor launch has h0 = 0 and stride = n.
struct Heads {
  int n, h0, stride;
  // the tensor-wide (b*stride + h0 + h) of the launch's (b*n + h)
  __host__ __device__ int64_t global(int64_t bh) const { return (bh / n) * stride + h0 + bh % n; }
};

struct Box {
  int t0, y0, x0, et, eh, ew, count, start;
};

__host__ __device__ inline Box block_box(const Geo& g, int n) {
  Box b;
  int iw = n % g.nW;
  int ih = (n / g.nW) % g.nH;
  int it = n / (g.nW * g.nH);
  b.t0 = it * g.bt;
  b.y0 = ih * g.bh;
  b.x0 = iw * g.bw;
  b.et = min(g.bt, g.T - b.t0);
  b.eh = min(g.bh, g.H - b.y0);
  b.ew = min(g.bw, g.W - b.x0);
  b.count = b.et * b.eh * b.ew;
  b.start = b.t0 * g.H * g.W + b.et * b.y0 * g.W + b.et * b.eh * b.x0;
  return b;
}

__device__ inline float bf16_to_f32(bf16_bits h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline double bf16_to_f64(bf16_bits h) { return (double)__uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even.
__device__ inline bf16_bits f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (bf16_bits)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_bits)(u >> 16);
}

}  // namespace fva
