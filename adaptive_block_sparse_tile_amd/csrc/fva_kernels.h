// fva_kernels.h -- launch helpers of libfva's kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fva_dev.h"

namespace fva {

// Router (fva_route.hip)
// Pooled means of the heads hd selects (written compactly, [B, hd.n, N, D]);
// clear_status: zero *status first (the router's row kernels OR into it).
hipError_t launch_pool(const void* q, const void* k, const Geo& g, int B, int L, const Heads& hd, int D, double* qbar,
                       double* kbar, uint32_t* status, bool clear_status, hipStream_t st);
// Bytes of the router's static scratch on each GPU, and its device address
// on the current device (looked up on the first call per device).
constexpr size_t kRouteScratchBytes = (size_t)128 << 20;
hipError_t route_scratch(void** ptr);
// Scores and row routing slab by slab: the query rows of every head are cut
// into tiles of 64 query blocks, and slab_tiles tiles at a time get their
// fp64 scores in S ([slab_tiles * 64][N]) and are routed from there.
// Mask and count rows are those of the heads hd selects in [B, hd.stride, N, ...].
hipError_t launch_route_slabs(const double* qbar, const double* kbar, int B, const Heads& hd, int N, int D,
                              float top_p, int k_floor, double* S, int64_t slab_tiles, uint32_t* mask,
                              int32_t* kv_cnt, uint32_t* status, hipStream_t st);
// Scores of the tiles t0 .. t0 + nt - 1 (64 query blocks of one head each)
// into S [nt * 64][N], as the router computes them.
hipError_t launch_scores_slab(const double* qbar, const double* kbar, int N, int D, int t0, int nt, double* S,
                              hipStream_t st);
// Slack-aware augmentation; the scores are recomputed slab by slab from the
// router's pooled means (fp64 [BH, N, D]) with the router's scores kernel, in
// S (slab_tiles tiles of 64 rows).
// Relative speeds of the 8 XCDs (per mille of the mean; all equal: unweighted).
struct XcdWeights {
  int64_t w[8];
};
hipError_t launch_sasa(const double* qbar, const double* kbar, int D, const uint32_t* mask_in, const Geo& g, int BH,
                       int R, const XcdWeights& w, const double* S_ready, double* S, int64_t slab_tiles,
                       uint32_t* mask_out, int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, int32_t* cand,
                       int64_t* row_cost, int32_t* slot_head, int32_t* nh, hipStream_t st);

// Static block mask of every (b, h): rows = B*heads*N.
hipError_t launch_static_mask(const Geo& g, int64_t rows, int lt, int lh, int lw, int anchor_t, uint32_t* mask,
                              int32_t* kv_cnt, hipStream_t st);


// Attention (fva_attn.hip)
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, L, heads, D;  // heads: this launch's heads (hd.n)
  Heads hd;            // which heads of q, k, v, o, the mask and the counts
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
  uint64_t* plan_tag;  // [1] shape tag written by the plan, checked by the exec
};

// Shape tag of a plan (nonzero hash of the tensor shape and the grid).
uint64_t plan_tag_of(int B, int L, int heads, int D, const Geo& g);

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
