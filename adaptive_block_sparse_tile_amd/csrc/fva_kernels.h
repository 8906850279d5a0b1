// fva_kernels.h -- launch helpers of libfva's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fva_dev.h"

namespace fva {

// Router (fva_route.hip)
hipError_t launch_pool(const void* q, const void* k, const Geo& g, int B, int L, int heads, int D, double* qbar,
                       double* kbar, uint32_t* status, hipStream_t st);
hipError_t launch_scores(const double* qbar, const double* kbar, int BH, int N, int D, double* S, hipStream_t st);
hipError_t launch_route_rows(const double* S, int64_t rows, int N, float top_p, int k_floor, uint32_t* mask,
                             int32_t* kv_cnt, uint32_t* status, hipStream_t st);

// Attention (fva_attn.hip)
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, L, heads, D;
  Geo g;
  const uint32_t* mask;
  float scale;
  uint64_t* trace;
  // workspace views
  int32_t* tok;
  int32_t* blk_cnt;
  uint64_t* keys;
  uint32_t* rank;
  int32_t* order;
  uint32_t* queue;
};

// Query rows per work item for a block volume (32, 64, 128 or 256 rows).
int attn_waves_for_block(int block_volume);
// Persistent workgroups for a (D, waves) variant on the current device.
int attn_persistent_workgroups(int D, int waves, int* err);
hipError_t launch_sparse_attn(const AttnLaunch& a, bool lpt, hipStream_t st);
hipError_t launch_dense_attn(const void* q, const void* k, const void* v, void* o, int B, int L, int heads, int D,
                             float scale, hipStream_t st);

}  // namespace fva
