// fva_api.cpp -- the C ABI of libfva: host-side validation, workspace layout
// and kernel launches.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/fva.h"
#include "fva_kernels.h"

namespace {

thread_local std::string g_last_error;

fva_status fail(fva_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fva_status ok() {
  g_last_error.clear();
  return FVA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool make_geo(const fva_grid* g, fva::Geo* out) {
  if (!g || g->T < 1 || g->H < 1 || g->W < 1 || g->bt < 1 || g->bh < 1 || g->bw < 1) return false;
  fva::Geo geo;
  geo.T = g->T; geo.H = g->H; geo.W = g->W;
  geo.bt = g->bt; geo.bh = g->bh; geo.bw = g->bw;
  geo.nT = (g->T + g->bt - 1) / g->bt;
  geo.nH = (g->H + g->bh - 1) / g->bh;
  geo.nW = (g->W + g->bw - 1) / g->bw;
  const int64_t n = (int64_t)geo.nT * geo.nH * geo.nW;
  if (n > (1 << 30)) return false;
  geo.N = (int)n;
  *out = geo;
  return true;
}

constexpr int kMaxBlocks = 8192;  // largest row the router selects in one workgroup; the attention kernel's LDS mask
constexpr int64_t kMaxTokens = 1 << 24;
constexpr int kMaxHeads = 4096;  // B*heads planned by one workgroup's LDS

fva_status check_desc(const fva_desc* d) {
  if (!d) return fail(FVA_ERR_INVALID_ARG, "desc is null");
  if (d->B < 1 || d->L < 1 || d->heads < 1 || d->D < 1)
    return fail(FVA_ERR_INVALID_ARG, "desc sizes must be positive (B %d, L %d, heads %d, D %d)", d->B, d->L,
                d->heads, d->D);
  if (d->D != 64 && d->D != 128) return fail(FVA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->D);
  if ((int64_t)d->L >= kMaxTokens) return fail(FVA_ERR_UNSUPPORTED, "L %d >= 2^24 not supported", d->L);
  const int64_t elems = (int64_t)d->B * d->L * d->heads * d->D;
  if (elems >= ((int64_t)1 << 40)) return fail(FVA_ERR_UNSUPPORTED, "tensor too large");
  return FVA_OK;
}

fva_status check_grid(const fva_desc* d, const fva_grid* g, fva::Geo* geo) {
  if (!g) return fail(FVA_ERR_INVALID_ARG, "grid is null");
  if (!make_geo(g, geo))
    return fail(FVA_ERR_INVALID_ARG, "grid and block dims must be positive (T %d H %d W %d, block %d %d %d)", g->T,
                g->H, g->W, g->bt, g->bh, g->bw);
  const int64_t thw = (int64_t)g->T * g->H * g->W;
  if (thw != d->L)
    return fail(FVA_ERR_SHAPE, "grid T*H*W = %lld does not equal sequence length %d", (long long)thw, d->L);
  const int64_t vol = (int64_t)g->bt * g->bh * g->bw;
  if (vol > 256) return fail(FVA_ERR_UNSUPPORTED, "block volume %lld > 256 not supported", (long long)vol);
  return FVA_OK;
}

fva_status check_scale(int D, float scale) {
  const double want = 1.0 / std::sqrt((double)D);
  if (!(std::fabs((double)scale - want) <= 1e-6))
    return fail(FVA_ERR_SCALE, "scale %.9g is not head_dim^-0.5 = %.9g within 1e-6", (double)scale, want);
  return FVA_OK;
}

// The router's workspace: pooled means (fp64 [B*heads, N, D], Q and K) and
// one slab of fp64 scores.  The scores are produced and consumed tile by
// tile (64 query blocks of one head per tile), so the slab holds at most
// kScoreSlabBytes of them, never the whole [B*heads, N, N] matrix.  Each slab
// costs one scores and one routing launch with their tails (about 90 us on
// the long video's 6144-block rows), hence a slab of a few hundred MiB.
#ifndef FVA_SCORE_SLAB_MIB
#define FVA_SCORE_SLAB_MIB 512
#endif
constexpr size_t kScoreSlabBytes = (size_t)FVA_SCORE_SLAB_MIB << 20;
constexpr int64_t kMaxSlabTiles = 65535;  // grid.y of the scores kernel

struct RouteWs {
  size_t qbar, kbar, s, total;
  int64_t slab_tiles;
};

RouteWs route_ws_layout(const fva_desc* d, const fva::Geo& g, size_t slab_bytes = kScoreSlabBytes) {
  RouteWs w;
  const size_t rows = (size_t)d->B * d->heads * g.N;
  const int64_t tiles = (int64_t)d->B * d->heads * ((g.N + 63) / 64);
  const size_t tile_bytes = (size_t)64 * g.N * sizeof(double);
  w.slab_tiles = std::min<int64_t>(std::min<int64_t>(tiles, kMaxSlabTiles),
                                   std::max<int64_t>(1, (int64_t)(slab_bytes / tile_bytes)));
  size_t off = 0;
  w.qbar = off; off += align_up(rows * d->D * sizeof(double));
  w.kbar = off; off += align_up(rows * d->D * sizeof(double));
  w.s = off; off += align_up((size_t)w.slab_tiles * tile_bytes);
  w.total = off;
  return w;
}

struct AttnWs {
  size_t tok, cnt, tiles, keys, rank, order, head_pos, head_cost, qoff, qctr, tag, total;
};

AttnWs attn_ws_layout(const fva_desc* d, const fva::Geo& g) {
  AttnWs w;
  const size_t bh = (size_t)d->B * d->heads;
  const size_t items = bh * g.N;
  const int cpb = fva::attn_chunks_per_block(g.bt * g.bh * g.bw);
  size_t off = 0;
  w.tok = off; off += align_up((size_t)d->L * sizeof(int32_t));
  w.cnt = off; off += align_up((size_t)g.N * sizeof(int32_t));
  w.tiles = off; off += align_up(fva::attn_tile_bytes(d->D, (int64_t)items * cpb));
  w.keys = off; off += align_up(items * sizeof(uint64_t));
  w.rank = off; off += align_up(items * sizeof(uint32_t));
  w.order = off; off += align_up(items * sizeof(int32_t));
  w.head_pos = off; off += align_up(bh * sizeof(int32_t));
  w.head_cost = off; off += align_up(bh * sizeof(uint64_t));
  w.qoff = off; off += align_up(16 * sizeof(int32_t));
  w.qctr = off; off += align_up(16 * sizeof(uint32_t));
  w.tag = off; off += align_up(sizeof(uint64_t));
  w.total = off;
  return w;
}

fva_status check_ws(const void* ws, size_t have, size_t need) {
  if (!ws) return fail(FVA_ERR_WORKSPACE, "workspace is null (%zu bytes needed)", need);
  if (((uintptr_t)ws) % kAlign) return fail(FVA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (have < need) return fail(FVA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
  return FVA_OK;
}

fva_status device_error(hipError_t e, const char* what) {
  return fail(FVA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// A launch's grid must fit one dispatch: fewer than 2^32 work-items along x.
fva_status check_launch(int64_t workgroups, int threads, const char* what) {
  if (workgroups < 1 || workgroups * threads < ((int64_t)1 << 32)) return FVA_OK;
  return fail(FVA_ERR_UNSUPPORTED, "%s needs %lld workgroups of %d threads, more than one launch holds (2^32 threads)",
              what, (long long)workgroups, threads);
}

// B*heads is bounded for every entry point (the schedule's per-head LDS
// tables and the per-head grid dimension of its ranking kernel).
fva_status check_heads(const fva_desc* d) {
  if ((int64_t)d->B * d->heads > kMaxHeads)
    return fail(FVA_ERR_UNSUPPORTED, "B*heads = %lld > %d not supported", (long long)d->B * d->heads, kMaxHeads);
  return FVA_OK;
}

// Launch sizes of the router for this shape (rows are routed one slab of
// score tiles per launch).
fva_status check_route_launches(const fva_desc* d, const fva::Geo& g, int64_t slab_tiles) {
  const int64_t chunks = ((int64_t)d->heads * d->D / 8 + 63) / 64;
  const int words = (g.N + 31) / 32;
  const int threads = g.N <= 512 ? 64 : 64 * ((words + 63) / 64);
  fva_status st = check_launch((int64_t)g.N * chunks, 256, "pooling");
  if (st == FVA_OK) st = check_launch(slab_tiles * 64, threads, "row routing");
  return st;
}

}  // namespace

extern "C" {

int32_t fva_num_blocks(const fva_grid* grid) {
  fva::Geo g;
  if (!make_geo(grid, &g)) return -1;
  return g.N;
}

size_t fva_route_workspace_bytes(const fva_desc* desc, const fva_grid* grid) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK) return 0;
  return route_ws_layout(desc, g).total;
}

size_t fva_attn_workspace_bytes(const fva_desc* desc, const fva_grid* grid) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK) return 0;
  return attn_ws_layout(desc, g).total;
}

int32_t fva_attn_workgroups(const fva_desc* desc, const fva_grid* grid) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK) return -1;
  int err = 0;
  const int n = fva::attn_persistent_workgroups(desc->D, g.bt * g.bh * g.bw, &err);
  return err ? -1 : n;
}

// Host validation of a router call whose score slab may hold slab_bytes;
// on success *lay is its workspace layout.
static fva_status route_check(const void* q, const void* k, const fva_desc* desc, const fva_grid* grid,
                              const fva_route_cfg* cfg, const uint32_t* mask, size_t slab_bytes, fva::Geo* g,
                              RouteWs* lay) {
  if (!q || !k || !mask || !cfg) return fail(FVA_ERR_INVALID_ARG, "q, k, mask and cfg must not be null");
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  if ((st = check_grid(desc, grid, g)) != FVA_OK) return st;
  if (std::isnan(cfg->top_p)) return fail(FVA_ERR_INVALID_ARG, "top_p is NaN");
  if (cfg->k_floor < 1) return fail(FVA_ERR_TOPK, "k_floor %d must be a positive integer", cfg->k_floor);
  if (cfg->k_floor > g->N) return fail(FVA_ERR_TOPK, "k_floor %d > num_blocks %d", cfg->k_floor, g->N);
  if (g->N > kMaxBlocks) return fail(FVA_ERR_UNSUPPORTED, "num_blocks %d > %d not supported", g->N, kMaxBlocks);
  *lay = route_ws_layout(desc, *g, slab_bytes);
  if ((st = check_heads(desc)) != FVA_OK || (st = check_route_launches(desc, *g, lay->slab_tiles)) != FVA_OK)
    return st;
  return FVA_OK;
}

// The router's launches on a validated call for the heads hd selects, its
// workspace at ws: the pooling (which zeroes *status first if clear_status)
// and then the slabs of scores and row routing (route_slabs false: only the
// pooling).
static fva_status route_launch(const void* q, const void* k, const fva_desc* desc, const fva::Geo& g,
                               const fva_route_cfg* cfg, const RouteWs& lay, uint32_t* mask, int32_t* kv_cnt,
                               uint32_t* status, void* ws, void* stream, const fva::Heads& hd,
                               bool clear_status = true, bool pool = true, bool route_slabs = true) {
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  double* qbar = (double*)(w + lay.qbar);
  double* kbar = (double*)(w + lay.kbar);
  double* S = (double*)(w + lay.s);
  hipError_t e = hipSuccess;
  if (pool) {
    e = fva::launch_pool(q, k, g, desc->B, desc->L, hd, desc->D, qbar, kbar, status, clear_status, s);
    if (e != hipSuccess) return device_error(e, "pool kernel launch");
  }
  if (route_slabs) {
    e = fva::launch_route_slabs(qbar, kbar, desc->B, hd, g.N, desc->D, cfg->top_p, cfg->k_floor, S, lay.slab_tiles,
                                mask, kv_cnt, status, s);
    if (e != hipSuccess) return device_error(e, "router launch");
  }
  return ok();
}

fva_status fva_route(const void* q, const void* k, const fva_desc* desc, const fva_grid* grid,
                     const fva_route_cfg* cfg, uint32_t* mask, int32_t* kv_cnt, uint32_t* status, void* ws,
                     size_t ws_bytes, void* stream) {
  fva::Geo g;
  RouteWs lay;
  fva_status st = route_check(q, k, desc, grid, cfg, mask, kScoreSlabBytes, &g, &lay);
  if (st != FVA_OK) return st;
  if ((st = check_ws(ws, ws_bytes, lay.total)) != FVA_OK) return st;
  return route_launch(q, k, desc, g, cfg, lay, mask, kv_cnt, status, ws, stream,
                      fva::Heads{desc->heads, 0, desc->heads});
}

fva_status fva_route_noalloc(const void* q, const void* k, const fva_desc* desc, const fva_grid* grid,
                             const fva_route_cfg* cfg, uint32_t* mask, int32_t* kv_cnt, uint32_t* status,
                             void* stream) {
  fva::Geo g;
  RouteWs one;
  fva_status st = route_check(q, k, desc, grid, cfg, mask, 0, &g, &one);
  if (st != FVA_OK) return st;
  // the pooled means must fit with room for at least one tile of scores
  if (one.total > fva::kRouteScratchBytes)
    return fail(FVA_ERR_UNSUPPORTED, "the router needs %zu bytes of scratch for this shape, more than the %zu of "
                "the static scratch (use fva_route with a workspace)", one.total, fva::kRouteScratchBytes);
  RouteWs lay;
  if ((st = route_check(q, k, desc, grid, cfg, mask, fva::kRouteScratchBytes - one.s, &g, &lay)) != FVA_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = fva::route_scratch(&scratch);
  if (e != hipSuccess) return device_error(e, "static scratch lookup");
  return route_launch(q, k, desc, g, cfg, lay, mask, kv_cnt, status, scratch, stream,
                      fva::Heads{desc->heads, 0, desc->heads});
}

// Shared validation and workspace views of the sparse attention calls.
static fva_status sparse_setup(const void* q, const void* k, const void* v, void* o, bool need_q, bool need_kv,
                               const fva_desc* desc, const fva_grid* grid, const uint32_t* mask, float scale,
                               bool check_scale_arg, int32_t sched, void* ws, size_t ws_bytes, fva::AttnLaunch* a) {
  if ((need_q && (!q || !o)) || (need_kv && (!k || !v)) || !mask)
    return fail(FVA_ERR_INVALID_ARG, "tensor and mask pointers must not be null");
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  fva::Geo g;
  if ((st = check_grid(desc, grid, &g)) != FVA_OK) return st;
  if (check_scale_arg && (st = check_scale(desc->D, scale)) != FVA_OK) return st;
  if (sched != FVA_SCHED_LPT && sched != FVA_SCHED_NAIVE && sched != FVA_SCHED_XCD)
    return fail(FVA_ERR_INVALID_ARG, "unknown schedule %d", sched);
  // an item's mask rows are staged in LDS (kMaxBlocks / 32 words)
  if (g.N > kMaxBlocks) return fail(FVA_ERR_UNSUPPORTED, "num_blocks %d > %d not supported", g.N, kMaxBlocks);
  const int64_t items = (int64_t)desc->B * desc->heads * g.N;
  const int64_t slots = items * fva::attn_chunks_per_block(g.bt * g.bh * g.bw);
  if (slots >= ((int64_t)1 << 31)) return fail(FVA_ERR_UNSUPPORTED, "too many work items");
  if ((st = check_heads(desc)) != FVA_OK) return st;
  if ((st = check_launch(slots, 256, "chunk tiling")) != FVA_OK) return st;
  const AttnWs lay = attn_ws_layout(desc, g);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != FVA_OK) return st;
  char* w = (char*)ws;
  a->q = q; a->k = k; a->v = v; a->o = o;
  a->B = desc->B; a->L = desc->L; a->heads = desc->heads; a->D = desc->D;
  a->hd = fva::Heads{desc->heads, 0, desc->heads};
  a->g = g;
  a->mask = mask;
  a->scale = scale;
  a->trace = nullptr;
  a->tok = (int32_t*)(w + lay.tok);
  a->blk_cnt = (int32_t*)(w + lay.cnt);
  a->tiles = (uint16_t*)(w + lay.tiles);
  a->keys = (uint64_t*)(w + lay.keys);
  a->rank = (uint32_t*)(w + lay.rank);
  a->order = (int32_t*)(w + lay.order);
  a->head_pos = (int32_t*)(w + lay.head_pos);
  a->head_cost = (uint64_t*)(w + lay.head_cost);
  a->qoff = (int32_t*)(w + lay.qoff);
  a->qctr = (uint32_t*)(w + lay.qctr);
  a->plan_tag = (uint64_t*)(w + lay.tag);
  return FVA_OK;
}

// SASA workspace: per-row candidates int32 [rows][rounds], per-row costs
// int64 [rows], heads per XCD int32 [8][BH], head counts int32 [8].
struct SasaWs {
  size_t s, cand, cost, slot, nh, total;
  int64_t slab_tiles;
};
static SasaWs sasa_ws_layout(const fva_desc* d, const fva::Geo& g, int rounds) {
  SasaWs w;
  const size_t BH = (size_t)d->B * d->heads;
  const size_t rows = BH * g.N;
  const RouteWs rl = route_ws_layout(d, g);  // the same slab of scores as the router's
  w.slab_tiles = rl.slab_tiles;
  size_t off = 0;
  w.s = off; off += rl.total - rl.s;
  w.cand = off; off += align_up(rows * (size_t)std::max(rounds, 1) * sizeof(int32_t));
  w.cost = off; off += align_up(rows * sizeof(int64_t));
  w.slot = off; off += align_up(8 * BH * sizeof(int32_t));
  w.nh = off; off += align_up(8 * sizeof(int32_t));
  w.total = off;
  return w;
}

size_t fva_sasa_workspace_bytes(const fva_desc* desc, const fva_grid* grid, int32_t rounds) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK || rounds < 0 || rounds > 8) return 0;
  return sasa_ws_layout(desc, g, rounds).total;
}

fva_status fva_sasa(const fva_desc* desc, const fva_grid* grid, const uint32_t* mask_in, const void* route_ws,
                    size_t route_ws_bytes, int32_t rounds, const int32_t* xcd_weight, uint32_t* mask_out,
                    int32_t* kv_cnt, int32_t* head_xcd, int64_t* xcd_load, void* ws, size_t ws_bytes, void* stream) {
  if (!mask_in || !route_ws || !mask_out || !head_xcd || !xcd_load)
    return fail(FVA_ERR_INVALID_ARG, "mask_in, route_ws, mask_out, head_xcd and xcd_load must not be null");
  if (rounds < 0 || rounds > 8) return fail(FVA_ERR_INVALID_ARG, "rounds %d outside 0..8", rounds);
  fva::XcdWeights w;
  for (int x = 0; x < 8; ++x) {
    w.w[x] = xcd_weight ? xcd_weight[x] : 1000;
    if (w.w[x] < 1 || w.w[x] > 1000000)
      return fail(FVA_ERR_INVALID_ARG, "xcd_weight[%d] = %lld outside 1..1000000", x, (long long)w.w[x]);
  }
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  fva::Geo g;
  if ((st = check_grid(desc, grid, &g)) != FVA_OK) return st;
  if ((st = check_heads(desc)) != FVA_OK) return st;
  if (g.N > kMaxBlocks) return fail(FVA_ERR_UNSUPPORTED, "num_blocks %d > %d not supported", g.N, kMaxBlocks);
  if ((st = check_launch((int64_t)desc->B * desc->heads * g.N, 64, "augmentation candidates")) != FVA_OK) return st;
  const RouteWs rl = route_ws_layout(desc, g);
  if (route_ws_bytes < rl.total)
    return fail(FVA_ERR_WORKSPACE, "route workspace holds %zu bytes, the router's is %zu", route_ws_bytes, rl.total);
  const SasaWs lay = sasa_ws_layout(desc, g, rounds);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != FVA_OK) return st;
  char* base = (char*)ws;
  const double* qbar = (const double*)((const char*)route_ws + rl.qbar);
  const double* kbar = (const double*)((const char*)route_ws + rl.kbar);
  // the router's scores, when its one slab held every tile
  const int64_t tiles = (int64_t)desc->B * desc->heads * ((g.N + 63) / 64);
  const double* s_ready = rl.slab_tiles >= tiles ? (const double*)((const char*)route_ws + rl.s) : nullptr;
  hipError_t e = fva::launch_sasa(qbar, kbar, desc->D, mask_in, g, desc->B * desc->heads, rounds, w, s_ready,
                                  (double*)(base + lay.s), lay.slab_tiles, mask_out, kv_cnt, head_xcd, xcd_load,
                                  (int32_t*)(base + lay.cand), (int64_t*)(base + lay.cost),
                                  (int32_t*)(base + lay.slot), (int32_t*)(base + lay.nh), (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "sasa launch");
  return ok();
}

fva_status fva_static_mask(const fva_desc* desc, const fva_grid* grid, const fva_static_cfg* cfg, uint32_t* mask,
                           int32_t* kv_cnt, void* stream) {
  if (!mask || !cfg) return fail(FVA_ERR_INVALID_ARG, "mask and cfg must not be null");
  if (cfg->lt < 1 || cfg->lh < 1 || cfg->lw < 1)
    return fail(FVA_ERR_INVALID_ARG, "local box %d x %d x %d must be at least 1 block", cfg->lt, cfg->lh, cfg->lw);
  if (cfg->anchor_t < 0) return fail(FVA_ERR_INVALID_ARG, "anchor_t %d < 0", cfg->anchor_t);
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  fva::Geo g;
  if ((st = check_grid(desc, grid, &g)) != FVA_OK) return st;
  if (g.N > kMaxBlocks) return fail(FVA_ERR_UNSUPPORTED, "num_blocks %d > %d not supported", g.N, kMaxBlocks);
  if ((st = check_heads(desc)) != FVA_OK) return st;
  const int64_t rows = (int64_t)desc->B * desc->heads * g.N;
  if ((st = check_launch(rows, 64, "static mask")) != FVA_OK) return st;
  hipError_t e = fva::launch_static_mask(g, rows, cfg->lt, cfg->lh, cfg->lw, cfg->anchor_t, mask, kv_cnt,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "static mask launch");
  return ok();
}

fva_status fva_sparse_attn(const void* q, const void* k, const void* v, void* o, const fva_desc* desc,
                           const fva_grid* grid, const uint32_t* mask, float scale, int32_t sched, uint64_t* trace,
                           void* ws, size_t ws_bytes, void* stream) {
  fva::AttnLaunch a;
  fva_status st = sparse_setup(q, k, v, o, true, true, desc, grid, mask, scale, true, sched, ws, ws_bytes, &a);
  if (st != FVA_OK) return st;
  a.trace = trace;
  hipError_t e = fva::launch_sparse_plan(a, sched, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "sparse attention plan launch");
  e = fva::launch_sparse_exec(a, sched, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "sparse attention launch");
  return ok();
}

fva_status fva_attn_plan(const void* k, const void* v, const fva_desc* desc, const fva_grid* grid,
                         const uint32_t* mask, int32_t sched, const int32_t* head_xcd, void* ws, size_t ws_bytes,
                         void* stream) {
  fva::AttnLaunch a;
  fva_status st = sparse_setup(nullptr, k, v, nullptr, false, true, desc, grid, mask, 0.f, false, sched, ws, ws_bytes,
                               &a);
  if (st != FVA_OK) return st;
  hipError_t e = fva::launch_sparse_plan(a, sched, head_xcd, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "sparse attention plan launch");
  return ok();
}

fva_status fva_attn_exec(const void* q, void* o, const fva_desc* desc, const fva_grid* grid, const uint32_t* mask,
                         float scale, int32_t sched, uint64_t* trace, void* ws, size_t ws_bytes, void* stream) {
  fva::AttnLaunch a;
  fva_status st = sparse_setup(q, nullptr, nullptr, o, true, false, desc, grid, mask, scale, true, sched, ws,
                               ws_bytes, &a);
  if (st != FVA_OK) return st;
  a.trace = trace;
  hipError_t e = fva::launch_sparse_exec(a, sched, (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "sparse attention launch");
  return ok();
}

// Whole layer over head groups: group g holds heads [g*heads/G, (g+1)*heads/G).
static int group_first_head(int heads, int groups, int g) { return (int)((int64_t)g * heads / groups); }

// Workspace of one stream of fva_routed_attn: a router and an attention
// workspace sized for the largest group, back to back.
struct LayerWs {
  RouteWs route;
  AttnWs attn;
  size_t one;  // bytes of one stream's set
};
static LayerWs layer_ws_layout(const fva_desc* desc, const fva::Geo& g, int groups) {
  fva_desc dmax = *desc;
  dmax.heads = (desc->heads + groups - 1) / groups;
  LayerWs w;
  w.route = route_ws_layout(&dmax, g);
  w.attn = attn_ws_layout(&dmax, g);
  w.one = w.route.total + w.attn.total;
  return w;
}

size_t fva_routed_attn_workspace_bytes(const fva_desc* desc, const fva_grid* grid, int32_t groups) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK || groups < 1 || groups > desc->heads)
    return 0;
  return (groups > 1 ? 2 : 1) * layer_ws_layout(desc, g, groups).one;
}

fva_status fva_routed_attn(const void* q, const void* k, const void* v, void* o, const fva_desc* desc,
                           const fva_grid* grid, const fva_route_cfg* cfg, float scale, int32_t groups,
                           uint32_t* mask, int32_t* kv_cnt, uint32_t* status, void* ws, size_t ws_bytes,
                           void* stream, void* side_stream) {
  if (!v || !o) return fail(FVA_ERR_INVALID_ARG, "tensor pointers must not be null");
  fva::Geo g;
  RouteWs whole;
  fva_status st = route_check(q, k, desc, grid, cfg, mask, kScoreSlabBytes, &g, &whole);
  if (st != FVA_OK) return st;
  if ((st = check_scale(desc->D, scale)) != FVA_OK) return st;
  if (groups < 1 || groups > desc->heads)
    return fail(FVA_ERR_INVALID_ARG, "groups %d outside 1..heads (%d)", groups, desc->heads);
  const LayerWs lay = layer_ws_layout(desc, g, groups);
  const hipStream_t s0 = (hipStream_t)stream;
  const hipStream_t s1 = (groups > 1 && side_stream && side_stream != stream) ? (hipStream_t)side_stream : s0;
  const int sets = s1 != s0 ? 2 : 1;
  if ((st = check_ws(ws, ws_bytes, (size_t)sets * lay.one)) != FVA_OK) return st;
  // every group is validated before anything is enqueued
  std::vector<fva::AttnLaunch> al(groups);
  std::vector<fva_desc> dg(groups, *desc);
  for (int gi = 0; gi < groups; ++gi) {
    const int hb = group_first_head(desc->heads, groups, gi), he = group_first_head(desc->heads, groups, gi + 1);
    dg[gi].heads = he - hb;
    char* base = (char*)ws + (size_t)(sets == 2 ? gi % 2 : 0) * lay.one;
    if ((st = check_route_launches(&dg[gi], g, lay.route.slab_tiles)) != FVA_OK) return st;
    if ((st = sparse_setup(q, k, v, o, true, true, &dg[gi], grid, mask, scale, true, FVA_SCHED_LPT,
                           base + lay.route.total, lay.attn.total, &al[gi])) != FVA_OK)
      return st;
    al[gi].hd = fva::Heads{he - hb, hb, desc->heads};
  }
  hipError_t e = hipSuccess;
  for (int gi = 0; gi < groups; ++gi) {
    const hipStream_t s = gi % 2 ? s1 : s0;
    char* base = (char*)ws + (size_t)(sets == 2 ? gi % 2 : 0) * lay.one;
    const fva::Heads hd = al[gi].hd;
    // group 0's pooling zeroes the status word, before the side stream joins
    if ((st = route_launch(q, k, &dg[gi], g, cfg, lay.route, mask, kv_cnt, status, base, s, hd, gi == 0, true,
                           false)) != FVA_OK)
      return st;
    if (gi == 0 && s1 != s0) {
      // the side stream starts after the caller's earlier work on stream and this clear
      hipEvent_t ev;
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return device_error(e, "event");
      e = hipEventRecord(ev, s0);
      if (e == hipSuccess) e = hipStreamWaitEvent(s1, ev, 0);
      hipEventDestroy(ev);
      if (e != hipSuccess) return device_error(e, "stream fork");
    }
    if ((st = route_launch(q, k, &dg[gi], g, cfg, lay.route, mask, kv_cnt, status, base, s, hd, false, false,
                           true)) != FVA_OK)
      return st;
    if ((e = fva::launch_sparse_plan(al[gi], FVA_SCHED_LPT, nullptr, s)) != hipSuccess)
      return device_error(e, "sparse attention plan launch");
    if ((e = fva::launch_sparse_exec(al[gi], FVA_SCHED_LPT, s)) != hipSuccess)
      return device_error(e, "sparse attention launch");
  }
  if (s1 != s0) {
    // stream resumes after everything enqueued on the side stream
    hipEvent_t ev;
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return device_error(e, "event");
    e = hipEventRecord(ev, s1);
    if (e == hipSuccess) e = hipStreamWaitEvent(s0, ev, 0);
    hipEventDestroy(ev);
    if (e != hipSuccess) return device_error(e, "stream join");
  }
  return ok();
}

int32_t fva_attn_items(const fva_desc* desc, const fva_grid* grid) {
  fva::Geo g;
  if (check_desc(desc) != FVA_OK || check_grid(desc, grid, &g) != FVA_OK) return -1;
  const int64_t n = (int64_t)desc->B * desc->heads * fva::attn_items_per_head(g);
  return n > INT32_MAX ? -1 : (int32_t)n;
}

fva_status fva_attn_schedule(const fva_desc* desc, const fva_grid* grid, const void* ws, size_t ws_bytes,
                             int32_t* order, int32_t* qoff, uint32_t* cost, void* stream) {
  if (!order || !qoff) return fail(FVA_ERR_INVALID_ARG, "order and qoff must not be null");
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  fva::Geo g;
  if ((st = check_grid(desc, grid, &g)) != FVA_OK) return st;
  const AttnWs lay = attn_ws_layout(desc, g);
  if ((st = check_ws(ws, ws_bytes, lay.total)) != FVA_OK) return st;
  const int64_t items = (int64_t)desc->B * desc->heads * fva::attn_items_per_head(g);
  const char* w = (const char*)ws;
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(order, w + lay.order, (size_t)items * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(qoff, w + lay.qoff, 9 * sizeof(int32_t), hipMemcpyDeviceToDevice, s);  // 8 queues + end
  if (e == hipSuccess && cost) e = fva::launch_item_costs((const uint64_t*)(w + lay.keys), items, cost, s);
  if (e != hipSuccess) return device_error(e, "schedule copy");
  return ok();
}

size_t fva_dense_workspace_bytes(const fva_desc* desc) {
  if (check_desc(desc) != FVA_OK) return 0;
  return align_up(fva::dense_tile_bytes(desc->B, desc->L, desc->heads, desc->D));
}

fva_status fva_dense_attn_ref(const void* q, const void* k, const void* v, void* o, const fva_desc* desc, float scale,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!q || !k || !v || !o) return fail(FVA_ERR_INVALID_ARG, "q, k, v and o must not be null");
  fva_status st = check_desc(desc);
  if (st != FVA_OK) return st;
  if ((st = check_scale(desc->D, scale)) != FVA_OK) return st;
  if ((st = check_heads(desc)) != FVA_OK) return st;
  const int64_t bh = (int64_t)desc->B * desc->heads;
  if ((st = check_launch(bh * ((desc->L + 63) / 64), 256, "chunk tiling")) != FVA_OK ||
      (st = check_launch(8 * ((bh * ((desc->L + 255) / 256) + 7) / 8), 512, "dense attention")) != FVA_OK)
    return st;
  if ((st = check_ws(ws, ws_bytes, fva_dense_workspace_bytes(desc))) != FVA_OK) return st;
  hipError_t e = fva::launch_dense_attn(q, k, v, o, desc->B, desc->L, desc->heads, desc->D, scale, ws,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return device_error(e, "dense attention launch");
  return ok();
}

fva_status fva_trace_imbalance(const uint64_t* t, int32_t n_wg, double* busy_ratio, double* finish_ratio,
                               int32_t* n_cu) {
  if (!t || n_wg < 1 || !busy_ratio || !finish_ratio) return fail(FVA_ERR_INVALID_ARG, "bad trace arguments");
  // CU identity: XCC id plus the HW_ID fields se_id [15:13], sh_id [12], cu_id [11:8]
  std::map<uint64_t, std::pair<double, uint64_t>> cu;  // key -> (busy, last end)
  uint64_t t0 = ~0ull;
  for (int i = 0; i < n_wg; ++i) {
    const uint64_t* r = t + (size_t)i * 4;
    const uint64_t items = r[3] >> 40;
    if (!items) continue;
    if (r[0] < t0) t0 = r[0];
  }
  if (t0 == ~0ull) return fail(FVA_ERR_INVALID_ARG, "trace holds no work");
  for (int i = 0; i < n_wg; ++i) {
    const uint64_t* r = t + (size_t)i * 4;
    const uint64_t items = r[3] >> 40;
    if (!items) continue;
    const uint32_t hw = (uint32_t)r[3];
    const uint64_t xcc = (r[3] >> 32) & 0xff;
    const uint64_t key = (xcc << 16) | (((hw >> 13) & 7u) << 5) | (((hw >> 12) & 1u) << 4) | ((hw >> 8) & 15u);
    auto& e = cu[key];
    e.first += (double)r[2];
    if (r[1] > e.second) e.second = r[1];
  }
  double bmax = 0, bsum = 0, fmax_ = 0, fsum = 0;
  for (auto& kv : cu) {
    const double b = kv.second.first, f = (double)(kv.second.second - t0);
    bmax = std::max(bmax, b);
    bsum += b;
    fmax_ = std::max(fmax_, f);
    fsum += f;
  }
  const double n = (double)cu.size();
  *busy_ratio = bsum > 0 ? bmax / (bsum / n) : 0.0;
  *finish_ratio = fsum > 0 ? fmax_ / (fsum / n) : 0.0;
  if (n_cu) *n_cu = (int32_t)cu.size();
  return ok();
}

fva_status fva_trace_xcd_speed(const uint64_t* t, int32_t n_wg, const int64_t* xcd_load, int32_t* xcd_weight) {
  if (!t || n_wg < 1 || !xcd_load || !xcd_weight) return fail(FVA_ERR_INVALID_ARG, "bad trace arguments");
  double busy[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = 0; i < n_wg; ++i) {
    const uint64_t* r = t + (size_t)i * 4;
    if (!(r[3] >> 40)) continue;
    busy[(r[3] >> 32) & 7] += (double)r[2];
  }
  double speed[8], mean = 0.0;
  for (int x = 0; x < 8; ++x) {
    if (busy[x] <= 0.0 || xcd_load[x] <= 0)
      return fail(FVA_ERR_INVALID_ARG, "XCD %d has no measured work (load %lld, busy %.0f ticks)", x,
                  (long long)xcd_load[x], busy[x]);
    speed[x] = (double)xcd_load[x] / busy[x];
    mean += speed[x] / 8.0;
  }
  for (int x = 0; x < 8; ++x) xcd_weight[x] = (int32_t)std::lround(1000.0 * speed[x] / mean);
  return ok();
}

const char* fva_last_error(void) { return g_last_error.c_str(); }

const char* fva_status_name(int32_t s) {
  switch (s) {
    case FVA_OK: return "FVA_OK";
    case FVA_ERR_INVALID_ARG: return "FVA_ERR_INVALID_ARG";
    case FVA_ERR_SHAPE: return "FVA_ERR_SHAPE";
    case FVA_ERR_TOPK: return "FVA_ERR_TOPK";
    case FVA_ERR_SCALE: return "FVA_ERR_SCALE";
    case FVA_ERR_WORKSPACE: return "FVA_ERR_WORKSPACE";
    case FVA_ERR_UNSUPPORTED: return "FVA_ERR_UNSUPPORTED";
    case FVA_ERR_DEVICE: return "FVA_ERR_DEVICE";
    default: return "unknown";
  }
}

}  // extern "C"
