/*
 * fva.h -- C ABI of libfva: routed block-sparse attention for video DiTs on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, on the GPU, the data-parallel hot path of
 * training-free adaptive sparse attention as the FVAttn abstract describes
 * its sparse-routing frontend (Top-p routing, a Top-k safety floor,
 * video-aware block organisation, a mask repaired at runtime) followed by
 * attention restricted to the routed blocks:
 *   1. the (T,H,W) latent token grid is tiled into (bt,bh,bw) blocks; the
 *      number of blocks is prod ceil(dim/block) and the blocks on the far
 *      edges are ragged (vLLM-Omni FastVideo VSA guide, sections 1, 3, 6);
 *   2. fva_route: per (batch, head, query block), block-mean pooled Q and K,
 *      scores scaled by 1/sqrt(D), row softmax over all blocks, a descending
 *      order, the smallest prefix whose cumulative probability reaches top_p,
 *      at least k_floor blocks, materialised as a bit mask;
 *   3. fva_sparse_attn: exact softmax attention of every real query token
 *      over the real tokens of the kept key blocks only, scheduled across the
 *      compute units longest-item-first from the routed per-row work (the
 *      one-GPU share of the FVAttn abstract's runtime load balancing).
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V, O are bf16, contiguous BSHD: element (b, l, h, d) at
 *     ((b*L + l)*heads + h)*D + d.  Token l = (t*H + y)*W + x.
 *   - Every tensor, mask and workspace pointer is a DEVICE pointer owned by
 *     the caller.  The library never allocates, frees or caches device memory
 *     at run time and keeps no state between calls; the one exception is the
 *     static per-GPU scratch array of fva_route_noalloc, part of the loaded
 *     module, whose contents the last such call leaves behind.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue their kernels on it and return without synchronising.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is launched, the status says which rule failed
 *     and fva_last_error() gives the detail.  There is no fallback path: the
 *     library never silently runs something else.
 *   - FVA_ERR_DEVICE means a HIP call failed while enqueueing; the HIP
 *     context may be unusable and the caller must not continue on it.
 *   - Calls that share a workspace buffer must not overlap in time.
 */
#ifndef FVA_H
#define FVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FVA_OK = 0,
  FVA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, NaN top_p, unknown schedule */
  FVA_ERR_SHAPE = 2,       /* T*H*W != L */
  FVA_ERR_TOPK = 3,        /* k_floor < 1 or k_floor > num_blocks */
  FVA_ERR_SCALE = 4,       /* |scale - 1/sqrt(D)| > 1e-6 */
  FVA_ERR_WORKSPACE = 5,   /* workspace null, smaller than required or not 256-byte aligned */
  FVA_ERR_UNSUPPORTED = 6, /* D not in {64,128}; block volume > 256; num_blocks > 8192; B*heads > 4096;
                              a kernel grid past 2^32 threads for this shape */
  FVA_ERR_DEVICE = 7       /* a HIP runtime call failed */
} fva_status;

/* Latent token grid (T, H, W) and block shape (bt, bh, bw), all >= 1. */
typedef struct {
  int32_t T, H, W;
  int32_t bt, bh, bw;
} fva_grid;

/* Shape of the contiguous BSHD bf16 tensors Q, K, V and O. */
typedef struct {
  int32_t B, L, heads, D;
} fva_desc;

/* Routing knobs.  0 < top_p < 1: Top-p with a floor of k_floor blocks;
 * top_p >= 1: every block is kept; top_p <= 0: Top-p is off and exactly
 * k_floor blocks are kept (fixed top-k, as the VSA backend does).
 * 1 <= k_floor <= num_blocks; k_floor == num_blocks gives dense rows. */
typedef struct {
  float top_p;
  int32_t k_floor;
} fva_route_cfg;

/* Schedules of the persistent attention kernel. */
/* LPT: heads go longest-first (summed real token pairs) to one queue per XCD;
 * each queue holds its heads' items in descending real token pairs; an idle
 * workgroup takes from its own XCD's queue first, then from the others.
 * NAIVE: one queue in (batch, head, query block) order. */
#define FVA_SCHED_LPT 0
#define FVA_SCHED_NAIVE 1
/* XCD: the ranks of the FVAttn abstract's load balancing played by the 8 XCDs:
 * heads are assigned as for LPT (or as fva_sasa assigned them, see
 * fva_attn_plan) and each XCD serves only its own queue, without taking
 * items from the others.  The launch puts 32 workgroups on each XCD. */
#define FVA_SCHED_XCD 2

/* Number of blocks prod ceil(dim/block) (VSA guide, section 3), or -1 when a
 * dimension is not positive.  Host only. */
int32_t fva_num_blocks(const fva_grid* grid);

/* Device workspace fva_route needs, or 0 for invalid arguments: the pooled
 * Q and K (fp64 [B*heads, N, D] each) and one slab of fp64 block scores.
 * The scores are computed and routed in tiles of 64 query blocks of one
 * head, as many tiles at a time as fit 512 MiB (at least one), so the whole
 * [B*heads, N, N] score matrix is never held.  Host only. */
size_t fva_route_workspace_bytes(const fva_desc* desc, const fva_grid* grid);

/* Device workspace fva_sparse_attn needs, or 0 for invalid arguments: the
 * block-ordered token table, the K and V of every (b, h, block) re-tiled into
 * 64-key chunk images (about 2*B*L*heads*D*2 bytes plus ragged-block padding),
 * work item costs, ranks, order and the per-XCD queues. */
size_t fva_attn_workspace_bytes(const fva_desc* desc, const fva_grid* grid);

/* Number of persistent workgroups fva_sparse_attn launches on the current
 * device for this shape; the trace buffer holds 4 uint64 per workgroup.
 * Returns -1 on invalid arguments or a HIP error. */
int32_t fva_attn_workgroups(const fva_desc* desc, const fva_grid* grid);

/* Block router (FVAttn abstract: Top-p routing, Top-k safety floor,
 * video-aware blocks, runtime mask repair; VSA guide section 5: scores use
 * head_dim^-0.5).  Pooling, scores, softmax, order, cumulative mass and the
 * count are taken in fp64; ties in score go to the lower block index.
 *   q, k     bf16 [B, L, heads, D] (device)
 *   mask     out, uint32 [B, heads, N, ceil(N/32)]: bit (j % 32) of word
 *            j / 32 of row (b, h, i) is set iff key block j is kept for
 *            query block i.  Rows are written whole.
 *   kv_cnt   out, int32 [B, heads, N]: kept blocks per row (nullable).
 *   status   out, uint32 [1]: bit 0 set if some row had a non-finite score
 *            and was repaired to keep every block (nullable).
 *   ws       device workspace of at least fva_route_workspace_bytes(),
 *            256-byte aligned; contents on entry are ignored.
 * Errors: INVALID_ARG, SHAPE, TOPK ("k_floor K > num_blocks N"),
 * UNSUPPORTED, WORKSPACE, DEVICE. */
fva_status fva_route(const void* q, const void* k, const fva_desc* desc, const fva_grid* grid,
                     const fva_route_cfg* cfg, uint32_t* mask, int32_t* kv_cnt, uint32_t* status, void* ws,
                     size_t ws_bytes, void* stream);

/* fva_route for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  It
 * takes no workspace: the pooled Q and K and the score slab live in a static
 * scratch array of FVA_ROUTE_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call makes no allocation (the
 * scratch's device address is looked up once per device, on the first call
 * there).  Same arguments, results and errors as fva_route, plus
 * FVA_ERR_UNSUPPORTED when the pooled means of this shape,
 * 2 * B*heads*N*D*8 bytes, leave no room in the scratch for one tile of 64
 * score rows (64*N*8 bytes); the long-video shape (5 heads, 6144 blocks,
 * D = 128) takes 60 MiB of pooled means.  Calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Nothing in the
 * scratch needs clearing between calls: every value read is written first
 * by the same call. */
#define FVA_ROUTE_SCRATCH_BYTES ((size_t)128 << 20)
fva_status fva_route_noalloc(const void* q, const void* k, const fva_desc* desc, const fva_grid* grid,
                             const fva_route_cfg* cfg, uint32_t* mask, int32_t* kv_cnt, uint32_t* status,
                             void* stream);

/* Static block mask: a second source of masks for fva_sparse_attn besides
 * the router (Sol-Attn article, section 3: tokens attend in full inside
 * their local window, and anchors link every window; here both rules act on
 * block coordinates).  With (t, y, x) the block coordinates of query block i
 * and key block j:
 *   kept(i, j) = (t_i/lt == t_j/lt && y_i/lh == y_j/lh && x_i/lw == x_j/lw)
 *             || (anchor_t > 0 && (t_i % anchor_t == 0 || t_j % anchor_t == 0))
 * (integer division): local boxes of lt x lh x lw blocks partition the block
 * grid, and the block slabs at temporal indices that are multiples of
 * anchor_t are anchors, kept by every row and keeping every block.  Every
 * row keeps at least its own block.  On a (T, 1, 1) grid of (1, 1, 1)
 * blocks this is the article's token mask with block_size = lt and
 * anchor_stride = anchor_t. */
typedef struct {
  int32_t lt, lh, lw;  /* local box, in blocks; each >= 1 */
  int32_t anchor_t;    /* anchor period along t, in blocks; 0 = no anchors */
} fva_static_cfg;

/* Writes the static mask of every (b, h) (the same pattern each time) and
 * its kept counts, in the layout fva_route writes.
 *   mask    out, uint32 [B, heads, N, ceil(N/32)] (device)
 *   kv_cnt  out, int32 [B, heads, N] (device, nullable)
 * Errors: INVALID_ARG (null mask, lt/lh/lw < 1, anchor_t < 0), SHAPE,
 * UNSUPPORTED, DEVICE.  No workspace. */
fva_status fva_static_mask(const fva_desc* desc, const fva_grid* grid, const fva_static_cfg* cfg, uint32_t* mask,
                           int32_t* kv_cnt, void* stream);

/* Block-sparse attention (VSA guide sections 1 and 6: each query block
 * attends only to its selected key/value blocks; ragged edge blocks run on
 * their real prefix and padding never acts as a key).  For every real token
 * l of query block i of (b, h):
 *   O[b,l,h,:] = sum_{l' in kept(i)} softmax_l'(scale * Q[b,l,h,:].K[b,l',h,:]) V[b,l',h,:]
 * with bf16 MFMA products, fp32 accumulation and online softmax, and the
 * result rounded to bf16.  Every token of the grid is written.
 *   q, k, v  bf16 [B, L, heads, D] (device); o out, same shape
 *   mask     uint32 [B, heads, N, ceil(N/32)] as fva_route writes it; a row
 *            with no bit set is an error the caller must avoid (its O rows
 *            are written as zeros)
 *   scale    softmax scale; must be within 1e-6 of 1/sqrt(D)
 *   sched    FVA_SCHED_LPT, FVA_SCHED_NAIVE or FVA_SCHED_XCD; all give bitwise
 *            equal O
 *   trace    nullable device uint64 [fva_attn_workgroups()][4]: per
 *            workgroup first-item start, last-item end, summed item time
 *            (100 MHz ticks) and (items << 40 | xcc_id << 32 | hw_id)
 *   ws       device workspace of at least fva_attn_workspace_bytes()
 * Errors: INVALID_ARG, SHAPE, SCALE, UNSUPPORTED, WORKSPACE, DEVICE. */
fva_status fva_sparse_attn(const void* q, const void* k, const void* v, void* o, const fva_desc* desc,
                           const fva_grid* grid, const uint32_t* mask, float scale, int32_t sched, uint64_t* trace,
                           void* ws, size_t ws_bytes, void* stream);

/* fva_sparse_attn in two calls, for callers that time or overlap the two
 * parts.  fva_attn_plan enqueues the preparation: the block-ordered token
 * table, the 64-key chunk images of K and V, the work item costs (from mask)
 * and the schedule, all written into ws.  fva_attn_exec enqueues the
 * attention kernel that reads them (the K and V the plan read, the Q it is
 * given), and may run any number of times on one plan.  exec must run after
 * the plan (same stream, or ordered after it), with ws untouched in between
 * and with the same desc and grid; it attends over the kept blocks of the
 * mask it is given, and the plan's mask only orders the work, so any mask
 * gives the same O.  The plan leaves a tag of desc and grid in ws: an exec
 * whose ws holds no plan for its desc and grid writes NaN (bf16 0x7FC0) to
 * every element of O instead of computing it.  Arguments and errors as for
 * fva_sparse_attn; plan does not read q, exec does not read k or v.  head_xcd (nullable device int32 [B*heads],
 * used with FVA_SCHED_XCD only): the XCD (0..7) of each (b, h), as fva_sasa
 * writes it; null assigns heads by the LPT rule.  exec must be given the
 * same sched as plan. */
fva_status fva_attn_plan(const void* k, const void* v, const fva_desc* desc, const fva_grid* grid,
                         const uint32_t* mask, int32_t sched, const int32_t* head_xcd, void* ws, size_t ws_bytes,
                         void* stream);
fva_status fva_attn_exec(const void* q, void* o, const fva_desc* desc, const fva_grid* grid, const uint32_t* mask,
                         float scale, int32_t sched, uint64_t* trace, void* ws, size_t ws_bytes, void* stream);

/* The whole layer in one call: fva_route, then fva_sparse_attn (LPT
 * schedule) on its mask, optionally pipelined over head groups (FVAttn
 * abstract, "Overlap/Opt.": the overhead of scheduling hidden behind the
 * attention; summary, key module 4).
 *   groups = 1: route, plan and attention of all heads in order on stream,
 *     the same work as fva_route followed by fva_sparse_attn.
 *   groups = G > 1: the heads are cut into G contiguous groups (group g:
 *     heads g*heads/G .. (g+1)*heads/G - 1), each routed, planned and
 *     attended on its own, the groups alternating between stream (even g)
 *     and side_stream (odd g).  One group's routing, planning and attention
 *     then start while the previous group's attention still runs: they take
 *     the compute units that attention frees in its tail, so consecutive
 *     attention launches overlap instead of each ending in its own tail.
 *     side_stream NULL or equal to stream runs the groups in order on
 *     stream.  side_stream waits for the work enqueued on stream before the
 *     call (and for group 0's pooling), and stream waits for everything the
 *     call enqueued on side_stream, so to the caller the call is one ordered
 *     operation on stream.
 * Outputs are those of fva_route (mask, kv_cnt, status) and fva_sparse_attn
 * (o), bit for bit the same for every `groups` and stream choice.
 *   ws   device workspace of at least fva_routed_attn_workspace_bytes():
 *        one router and one attention workspace (for the largest group) per
 *        stream used; with G > 1 the size covers two streams.
 * Measured on one MI355X, the pipeline pays when a head's share of the layer
 * is long (the 393,216-token video, one head per group) and costs more than
 * it hides on short layers (the 27,280-token Wan layer), where groups = 1 is
 * the right choice.
 * Errors: those of fva_route and fva_sparse_attn, and INVALID_ARG for groups
 * outside 1..heads. */
size_t fva_routed_attn_workspace_bytes(const fva_desc* desc, const fva_grid* grid, int32_t groups);
fva_status fva_routed_attn(const void* q, const void* k, const void* v, void* o, const fva_desc* desc,
                           const fva_grid* grid, const fva_route_cfg* cfg, float scale, int32_t groups,
                           uint32_t* mask, int32_t* kv_cnt, uint32_t* status, void* ws, size_t ws_bytes,
                           void* stream, void* side_stream);

/* Number of work items of the sparse attention for this shape, or -1 for
 * invalid arguments.  A work item is one query block; blocks of at most 64
 * tokens are grouped 2x1x2 (t, y, x) per item and blocks of 65..128 tokens
 * 1x1x2, so that an item still fills the kernel's 8 wavefronts.  Item id =
 * (b*heads + h)*G + g, with G groups per (b, h) numbered in (t, y, x) order
 * over the grid of groups.  Host only. */
int32_t fva_attn_items(const fva_desc* desc, const fva_grid* grid);

/* The schedule fva_attn_plan wrote into ws (FVAttn abstract, key module 1:
 * runtime load balancing of head and block work; here, LPT list scheduling
 * over the 8 XCD queues).  The cost of an item is its real query rows times
 * the real key tokens of the union of its members' kept blocks.  Heads go,
 * in descending summed cost (ties: lower head), to the XCD with the least
 * assigned cost (ties: lower XCD), or where head_xcd put them; an XCD's
 * queue holds its heads in that order, each head's items in descending cost
 * (ties: lower item id; FVA_SCHED_NAIVE: item order, every head on queue 0).
 * Enqueues copies on the stream:
 *   order  out, device int32 [fva_attn_items()]: item ids in queue order;
 *          queue x is order[qoff[x] .. qoff[x+1])
 *   qoff   out, device int32 [9]
 *   cost   out, device uint32 [fva_attn_items()] (nullable): each item's
 *          cost, by item id
 * ws must hold a plan (fva_attn_plan) for desc and grid; the exec does not
 * change these arrays.  Errors: FVA_ERR_INVALID_ARG (null order or qoff),
 * shape errors as for fva_attn_plan, FVA_ERR_WORKSPACE, FVA_ERR_DEVICE. */
fva_status fva_attn_schedule(const fva_desc* desc, const fva_grid* grid, const void* ws, size_t ws_bytes,
                             int32_t* order, int32_t* qoff, uint32_t* cost, void* stream);

/* Slack-aware sparse augmentation, one-GPU form (FVAttn abstract and
 * summary, key modules 2 and 3: after load balancing, the slack left on the
 * non-critical ranks is filled with extra high-value blocks chosen from the
 * attention scores, without lengthening the critical path).  The ranks are
 * the 8 XCDs.  Row cost = the attention kernel's time on the row, in steps
 * of one 32-key half on its busiest SIMD: r_i = ceil(ceil(c_i/32)/2) steps
 * per 64-key chunk (32-row tiles on 8 wavefronts, two per SIMD; a ragged
 * block's tiles split their key halves over two wavefronts) times
 * ceil(c_j/64) chunks summed over the kept key blocks j; head cost = the sum
 * over its rows; heads go longest first (ties: lower head) to the least
 * loaded XCD (ties: lower XCD); the heaviest XCD's load is the makespan M.  Every other XCD x offers, in rounds r = 1..rounds, each of its
 * rows (heads in the order they were assigned to x, rows in block order) the
 * r-th block the router dropped from that row, in the router's order (block
 * score descending, lower index first); the longest prefix of these offers
 * whose summed cost r_i * ceil(c_j/64) fits M - load_x is added.  Run the attention
 * with FVA_SCHED_XCD and this head_xcd so that each XCD serves its own heads.
 *   mask_in    uint32 [B, heads, N, ceil(N/32)] from fva_route
 *   route_ws   the workspace of that fva_route call, untouched since: its
 *              pooled Q and K, and its score slab when that held every tile
 *              (the scores are then read from it; otherwise they are
 *              recomputed slab by slab with the router's own scores kernel,
 *              bit-equal to what it routed on)
 *   rounds     0..8 (0 copies the mask)
 *   xcd_weight nullable host int32 [8]: relative speed of each XCD (per
 *              mille; 1..1000000), e.g. from fva_trace_xcd_speed.  A head
 *              goes to the XCD where it would finish first, (load_x + c) /
 *              w_x; the critical XCD m has the largest load_m / w_m; XCD x
 *              may add up to floor(load_m * w_x / w_m) - load_x.  NULL: all
 *              XCDs equal (the rule above).
 *   mask_out   out, same layout (may equal mask_in)
 *   kv_cnt     out, int32 [B, heads, N] kept counts after augmentation (nullable)
 *   head_xcd   out, int32 [B*heads]
 *   xcd_load   out, int64 [16]: load of each XCD before (0..7) and the cost
 *              added to it (8..15), in the steps of the row cost
 *   ws         device workspace of at least fva_sasa_workspace_bytes() (a
 *              score slab like the router's, candidates, costs, placement)
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, WORKSPACE, DEVICE. */
size_t fva_sasa_workspace_bytes(const fva_desc* desc, const fva_grid* grid, int32_t rounds);
fva_status fva_sasa(const fva_desc* desc, const fva_grid* grid, const uint32_t* mask_in, const void* route_ws,
                    size_t route_ws_bytes, int32_t rounds, const int32_t* xcd_weight, uint32_t* mask_out,
                    int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, void* ws, size_t ws_bytes, void* stream);

/* Host helper: relative speeds of the 8 XCDs for fva_sasa's xcd_weight, from
 * a trace (copied to host memory) of the per-XCD schedule (FVA_SCHED_XCD,
 * placed as fva_sasa placed the heads) and the cost fva_sasa assigned each
 * XCD (xcd_load[0..7]): speed_x = xcd_load[x] / (summed item time of the
 * workgroups on XCD x), weight_x = round(1000 * speed_x / mean speed).
 * The traces of several launches of one plan may be passed back to back
 * (n_wg = launches * workgroups): their item times add up per XCD, which
 * averages out launch-to-launch variation.
 * Returns INVALID_ARG for null pointers, n_wg < 1 or an XCD with no work. */
fva_status fva_trace_xcd_speed(const uint64_t* host_trace, int32_t n_wg, const int64_t* xcd_load,
                               int32_t* xcd_weight);

/* Dense softmax attention over all L tokens (the FlashAttention baseline the
 * FVAttn abstract measures against), on the same kernel as fva_sparse_attn:
 * the sequence is one block of L tokens whose K and V are re-tiled in natural
 * order into the workspace (64-token chunks), and every 256-token query tile
 * attends to every chunk.  q, k, v, o as for fva_sparse_attn.
 *   ws   device workspace of at least fva_dense_workspace_bytes(), 256-byte
 *        aligned, caller-owned; its contents on return are unspecified
 * Errors: INVALID_ARG, SCALE, UNSUPPORTED, WORKSPACE, DEVICE. */
size_t fva_dense_workspace_bytes(const fva_desc* desc);
fva_status fva_dense_attn_ref(const void* q, const void* k, const void* v, void* o, const fva_desc* desc, float scale,
                              void* ws, size_t ws_bytes, void* stream);

/* Host helper: CU imbalance from a trace copied to host memory.  Groups the
 * workgroups by compute unit (xcc, shader engine, CU) and returns max/mean of
 * summed busy time and of finish time (last end - earliest start) over the
 * CUs that ran work.  Returns INVALID_ARG for null pointers or n_wg < 1. */
fva_status fva_trace_imbalance(const uint64_t* host_trace, int32_t n_wg, double* busy_max_over_mean,
                               double* finish_max_over_mean, int32_t* n_cu);

/* Detail of the last error on the calling thread ("" if none). */
const char* fva_last_error(void);

/* Short name of a status code. */
const char* fva_status_name(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* FVA_H */
