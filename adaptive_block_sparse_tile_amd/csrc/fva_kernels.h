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
// Slack-aware augmentation over the router's scores S (fp64 [BH, N, N]).
hipError_t launch_sasa(const double* S, const uint32_t* mask_in, const Geo& g, int BH, int R, uint32_t* mask_out,
                       int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, int32_t* cand, int64_t* row_cost,
                       int32_t* slot_head, int32_t* nh, hipStream_t st);

// Static block mask of every (b, h): rows = B*heads*N.
hipError_t launch_static_mask(const Geo& g, int64_t rows, int lt, int lh, int lw, int anchor_t, uint32_t* mask,
                              int32_t* kv_cnt, hipStream_t st);
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
  int32_t* tok;        // [L] block-ordered token ids
  int32_t* blk_cnt;    // [N] real tokens per block
  uint16_t* tiles;     // [B*heads*N*chunks_per_block] chunk images of K and V
  uint64_t* keys;      // [items] cost << 32 | ~item
  uint32_t* rank;      // [items] rank inside the item's head
  int32_t* order;      // [items] queue contents
  int32_t* head_pos;   // [B*heads] first order slot of each head
  uint64_t* head_cost; // [B*heads] summed item costs of each head
  int32_t* qoff;       // [9] queue segments (one per XCD)
  uint32_t* qctr;      // [8] queue pop counters
};

// 64-key chunk slots reserved per block.
int attn_chunks_per_block(int block_volume);
// Bytes of the chunk images for a number of slots.
size_t attn_tile_bytes(int D, int64_t slots);
// Persistent workgroups of the sparse kernel for (D, block volume) on the
// current device.
int attn_persistent_workgroups(int D, int block_volume, int* err);
// Work items per (b, h): query blocks, or groups of them for small blocks.
int attn_items_per_head(const Geo& g);
// cost[i] = keys[i] >> 32 for i < n (the item costs of a plan)
hipError_t launch_item_costs(const uint64_t* keys, int64_t n, uint32_t* cost, hipStream_t st);
// plan: token table, chunk images, item costs and the LPT (or naive) queues
// in the workspace; exec: the persistent attention kernel over that plan
// sched: 0 LPT with stealing, 1 naive, 2 per-XCD without stealing (heads by
// head_xcd if not null, else by the LPT rule)
hipError_t launch_sparse_plan(const AttnLaunch& a, int sched, const int32_t* head_xcd, hipStream_t st);
hipError_t launch_sparse_exec(const AttnLaunch& a, int sched, hipStream_t st);
// dense reference: natural-order chunk images (dense_tile_bytes) in tiles,
// then query tiles of 256 tokens over every key
size_t dense_tile_bytes(int B, int L, int heads, int D);
hipError_t launch_dense_attn(const void* q, const void* k, const void* v, void* o, int B, int L, int heads, int D,
                             float scale, void* tiles, hipStream_t st);

}  // namespace fva
