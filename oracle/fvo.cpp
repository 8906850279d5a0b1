// fvo.cpp -- fp64 CPU oracle for routed block-sparse video attention.
//
// TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
// benchmark's CPU-baseline leg load this library.  The product path (the HIP
// library) never links, loads or calls it, and the two share no code, header,
// table or helper.
//
// What it computes, step by step, in the order the method states it:
//   1. video-aware 3D block organisation of the (T,H,W) token grid
//      [vLLM-Omni FastVideo VSA guide, sections 1, 3 and 6;
//       FVAttn abstract: video-aware organisation of the blocks]
//   2. block-mean pooling of Q and K over the real tokens of each block
//   3. pooled block scores scaled by 1/sqrt(D)          [VSA guide, section 5]
//   4. row softmax over all N key blocks
//   5. descending order of the blocks (ties: lower block index first)
//   6. cumulative probability in that order; the smallest prefix whose mass
//      reaches top_p                                    [FVAttn summary, key
//      module 1: Top-p routing by cumulative-probability threshold]
//   7. Top-k safety floor: keep max(k_floor, count) blocks  [FVAttn abstract]
//   8. mask materialisation and validity repair          [FVAttn abstract]
//   9. exact softmax attention of every real query token over the real tokens
//      of its row's kept key blocks; pad tokens are never keys
//                                                        [VSA guide, sections 1, 6]
// Everything is fp64; bf16 inputs are widened exactly.  Plain loops, no
// blocking or fusion beyond these definitions.
//
// Readings where the pages are silent:
//   - pooling is the mean over real tokens (divide by the real count);
//   - blocks are numbered row-major over (block-t, block-h, block-w), and the
//     tokens of a block are visited row-major over (t, y, x);
//   - the crossing block is kept (smallest prefix with mass >= p);
//   - top_p >= 1 keeps every block; top_p <= 0 disables Top-p (fixed top-k);
//   - a row with a non-finite score is repaired to all N blocks (status bit 0).
//
// Ambiguity flags (rows that finite-precision arithmetic may legitimately
// route differently, excluded from bit-exact comparison), for a margin eps
// (1e-5 by default):
//   bit0 E1: moving the threshold p by +-eps changes the kept count;
//   bit1 E2: the last kept and first dropped scores differ by less than
//            eps*max(1,|s|) but are not equal;
//   bit2    : non-finite row (repaired to dense).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

struct Block {
  int t0, y0, x0;  // origin on the token grid
  int et, eh, ew;  // extents (ragged at the far edges)
  int count;       // real tokens = et*eh*ew
};

struct Geometry {
  int T = 0, H = 0, W = 0, bt = 0, bh = 0, bw = 0;
  int nT = 0, nH = 0, nW = 0, N = 0;
  std::vector<Block> blocks;
  std::vector<std::vector<int64_t>> tokens;  // tokens[n] = real token ids of block n, row-major (t,y,x)
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Step 1 -- video-aware block organisation.  N = prod ceil(dim / block); the
// last block along each axis keeps only the real rows (the rest is padding).
bool make_geometry(const int32_t* g, Geometry& geo) {
  geo.T = g[0]; geo.H = g[1]; geo.W = g[2]; geo.bt = g[3]; geo.bh = g[4]; geo.bw = g[5];
  if (geo.T <= 0 || geo.H <= 0 || geo.W <= 0 || geo.bt <= 0 || geo.bh <= 0 || geo.bw <= 0) return false;
  geo.nT = ceil_div(geo.T, geo.bt);
  geo.nH = ceil_div(geo.H, geo.bh);
  geo.nW = ceil_div(geo.W, geo.bw);
  geo.N = geo.nT * geo.nH * geo.nW;
  geo.blocks.resize(geo.N);
  geo.tokens.assign(geo.N, {});
  for (int it = 0; it < geo.nT; ++it)
    for (int ih = 0; ih < geo.nH; ++ih)
      for (int iw = 0; iw < geo.nW; ++iw) {
        int n = (it * geo.nH + ih) * geo.nW + iw;
        Block b;
        b.t0 = it * geo.bt; b.y0 = ih * geo.bh; b.x0 = iw * geo.bw;
        b.et = std::min(geo.bt, geo.T - b.t0);
        b.eh = std::min(geo.bh, geo.H - b.y0);
        b.ew = std::min(geo.bw, geo.W - b.x0);
        b.count = b.et * b.eh * b.ew;
        geo.blocks[n] = b;
        for (int t = b.t0; t < b.t0 + b.et; ++t)
          for (int y = b.y0; y < b.y0 + b.eh; ++y)
            for (int x = b.x0; x < b.x0 + b.ew; ++x)
              geo.tokens[n].push_back(((int64_t)t * geo.H + y) * geo.W + x);
      }
  return true;
}

double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Run fn(item) for item in [0, n) on up to nthreads host threads.
void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& fn) {
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n) nthreads = (int)std::max<int64_t>(1, n);
  std::atomic<int64_t> next(0);
  auto work = [&]() {
    for (;;) {
      int64_t i = next.fetch_add(1);
      if (i >= n) break;
      fn(i);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();
}

// Step 2 -- block mean of one (b, h) over the real tokens of block n.
void pool_block(const uint16_t* x, int64_t L, int heads, int D, const Geometry& geo, int b, int h, int n,
                double* out /*[D]*/) {
  const auto& toks = geo.tokens[n];
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t l : toks) {
    const uint16_t* row = x + (((int64_t)b * L + l) * heads + h) * D;
    for (int d = 0; d < D; ++d) out[d] += bf16_to_double(row[d]);
  }
  for (int d = 0; d < D; ++d) out[d] /= (double)toks.size();
}


// Steps 4-8 on one row of block scores s[0..N).  Writes the mask words, the
// kept count and the ambiguity flags of the row; returns true if the row had a
// non-finite score.
bool route_row(const double* s, int N, float top_p, int k_floor, double margin, uint32_t* mask_row, int32_t* cnt,
               uint8_t* flags) {
  const int words = (N + 31) / 32;
  for (int w = 0; w < words; ++w) mask_row[w] = 0;
  *flags = 0;
  bool finite = true;
  for (int j = 0; j < N; ++j)
    if (!std::isfinite(s[j])) finite = false;
  if (!finite) {
    // repair: a row whose scores cannot be ranked attends to every block
    for (int j = 0; j < N; ++j) mask_row[j >> 5] |= 1u << (j & 31);
    *cnt = N;
    *flags = 4;
    return true;
  }
  // step 4: softmax over all N blocks (max subtracted)
  double smax = s[0];
  for (int j = 1; j < N; ++j) smax = std::max(smax, s[j]);
  std::vector<double> e(N), P(N);
  double Z = 0.0;
  for (int j = 0; j < N; ++j) {
    e[j] = std::exp(s[j] - smax);
    Z += e[j];
  }
  for (int j = 0; j < N; ++j) P[j] = e[j] / Z;
  // step 5: descending order, ties to the lower block index
  std::vector<int> order(N);
  for (int j = 0; j < N; ++j) order[j] = j;
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    if (s[a] != s[b]) return s[a] > s[b];
    return a < b;
  });
  // step 6: cumulative mass C[m] of the first m blocks in that order
  std::vector<double> C(N + 1);
  C[0] = 0.0;
  for (int m = 1; m <= N; ++m) C[m] = C[m - 1] + P[order[m - 1]];
  const double p = (double)top_p;
  auto count_for = [&](double thr) -> int {
    for (int m = 1; m <= N; ++m)
      if (C[m] >= thr) return m;
    return N;
  };
  int nstar;
  if (p >= 1.0) nstar = N;
  else if (p <= 0.0) nstar = 0;
  else nstar = count_for(p);
  // step 7: Top-k safety floor
  int keep = std::min(N, std::max(k_floor, nstar));
  // step 8: materialise (the repair of the count to [1, N] is implied by the
  // validated 1 <= k_floor <= N); kept blocks are a prefix of the order
  for (int m = 0; m < keep; ++m) mask_row[order[m] >> 5] |= 1u << (order[m] & 31);
  *cnt = keep;
  // ambiguity flags
  if (p > 0.0 && p < 1.0) {
    int lo = count_for(p - margin), hi = count_for(p + margin);
    if (std::min(N, std::max(k_floor, lo)) != std::min(N, std::max(k_floor, hi))) *flags |= 1;
  }
  if (keep < N) {
    double a = s[order[keep - 1]], b = s[order[keep]];
    double gap = a - b;
    if (gap > 0.0 && gap < margin * std::max(1.0, std::fabs(a))) *flags |= 2;
  }
  return false;
}

}  // namespace

extern "C" {

// Number of blocks for grid (T,H,W) and block (bt,bh,bw); -1 if invalid.
int fvo_num_blocks(const int32_t* grid6) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  return geo.N;
}

// Block table: out[n*7 + {0..6}] = t0, y0, x0, et, eh, ew, count.
int fvo_block_table(const int32_t* grid6, int32_t* out) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  for (int n = 0; n < geo.N; ++n) {
    const Block& b = geo.blocks[n];
    int32_t* o = out + (int64_t)n * 7;
    o[0] = b.t0; o[1] = b.y0; o[2] = b.x0; o[3] = b.et; o[4] = b.eh; o[5] = b.ew; o[6] = b.count;
  }
  return geo.N;
}

// Token -> block id map, blk[l] for l in [0, T*H*W).
int fvo_token_block(const int32_t* grid6, int32_t* blk) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  for (int n = 0; n < geo.N; ++n)
    for (int64_t l : geo.tokens[n]) blk[l] = n;
  return geo.N;
}

// Step 2: pooled means out[((b*heads + h)*N + n)*D + d] for x bf16 [B, L, heads, D].
int fvo_pool(const uint16_t* x, int B, int64_t L, int heads, int D, const int32_t* grid6, double* out, int nthreads) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  if ((int64_t)geo.T * geo.H * geo.W != L) return -2;
  const int N = geo.N;
  parallel_for((int64_t)B * heads * N, nthreads, [&](int64_t it) {
    int n = (int)(it % N);
    int h = (int)((it / N) % heads);
    int b = (int)(it / ((int64_t)N * heads));
    pool_block(x, L, heads, D, geo, b, h, n, out + it * D);
  });
  return N;
}

// Step 3: block scores s[((b*heads + h)*N + i)*N + j] = (qbar_i . kbar_j) / sqrt(D).
int fvo_scores(const double* qbar, const double* kbar, int B, int heads, int N, int D, double* s, int nthreads) {
  const double rs = std::sqrt((double)D);
  parallel_for((int64_t)B * heads * N, nthreads, [&](int64_t row) {
    int64_t bh = row / N;
    const double* qi = qbar + row * D;
    for (int j = 0; j < N; ++j) {
      const double* kj = kbar + (bh * N + j) * D;
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
      s[row * N + j] = dot / rs;
    }
  });
  return 0;
}

// Steps 4-8 on R rows of given scores.  mask [R, ceil(N/32)], cnt [R], flags [R].
// status bit0 is set if any row was non-finite.
int fvo_route_scores(const double* s, int64_t R, int N, float top_p, int k_floor, double margin, uint32_t* mask,
                     int32_t* cnt, uint8_t* flags, uint32_t* status, int nthreads) {
  if (N <= 0 || k_floor < 1 || k_floor > N || std::isnan(top_p)) return -1;
  const int words = (N + 31) / 32;
  std::atomic<uint32_t> st(0);
  parallel_for(R, nthreads, [&](int64_t r) {
    if (route_row(s + r * N, N, top_p, k_floor, margin, mask + r * words, cnt + r, flags + r)) st.fetch_or(1u);
  });
  if (status) *status = st.load();
  return 0;
}

// The whole router (steps 1-8) from bf16 Q and K [B, L, heads, D].
int fvo_route(const uint16_t* q, const uint16_t* k, int B, int64_t L, int heads, int D, const int32_t* grid6,
              float top_p, int k_floor, double margin, uint32_t* mask, int32_t* cnt, uint8_t* flags, uint32_t* status,
              int nthreads) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  if ((int64_t)geo.T * geo.H * geo.W != L) return -2;
  const int N = geo.N;
  const int64_t R = (int64_t)B * heads * N;
  std::vector<double> qbar(R * D), kbar(R * D), s(R * N);
  fvo_pool(q, B, L, heads, D, grid6, qbar.data(), nthreads);
  fvo_pool(k, B, L, heads, D, grid6, kbar.data(), nthreads);
  fvo_scores(qbar.data(), kbar.data(), B, heads, N, D, s.data(), nthreads);
  return fvo_route_scores(s.data(), R, N, top_p, k_floor, margin, mask, cnt, flags, status, nthreads);
}

// Step 9: block-sparse attention for the listed work items.  An item is
// (b*heads + h)*N + i: every real query token of block i attends, with an
// exact fp64 softmax, to the real tokens of the key blocks set in mask row
// (b, h, i).  out is [B, L, heads, D] fp64; only the items' rows are written.
// items == nullptr means all B*heads*N items.
int fvo_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int64_t L, int heads, int D,
             const int32_t* grid6, const uint32_t* mask, double scale, const int64_t* items, int64_t n_items,
             double* out, int nthreads) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  if ((int64_t)geo.T * geo.H * geo.W != L) return -2;
  const int N = geo.N;
  const int words = (N + 31) / 32;
  const int64_t total = (int64_t)B * heads * N;
  if (!items) n_items = total;
  parallel_for(n_items, nthreads, [&](int64_t idx) {
    int64_t item = items ? items[idx] : idx;
    int i = (int)(item % N);
    int h = (int)((item / N) % heads);
    int b = (int)(item / ((int64_t)N * heads));
    const uint32_t* mrow = mask + item * words;
    // key set: real tokens of the kept blocks, ascending block order
    std::vector<int64_t> keys;
    for (int j = 0; j < N; ++j)
      if (mrow[j >> 5] >> (j & 31) & 1u)
        for (int64_t l : geo.tokens[j]) keys.push_back(l);
    std::vector<double> qv(D), sc(keys.size()), acc(D);
    for (int64_t lq : geo.tokens[i]) {
      const uint16_t* qr = q + (((int64_t)b * L + lq) * heads + h) * D;
      for (int d = 0; d < D; ++d) qv[d] = bf16_to_double(qr[d]);
      double m = -INFINITY;
      for (size_t r = 0; r < keys.size(); ++r) {
        const uint16_t* kr = k + (((int64_t)b * L + keys[r]) * heads + h) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[d] * bf16_to_double(kr[d]);
        sc[r] = dot * scale;
        m = std::max(m, sc[r]);
      }
      double z = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (size_t r = 0; r < keys.size(); ++r) {
        double w = std::exp(sc[r] - m);
        z += w;
        const uint16_t* vr = v + (((int64_t)b * L + keys[r]) * heads + h) * D;
        for (int d = 0; d < D; ++d) acc[d] += w * bf16_to_double(vr[d]);
      }
      double* o = out + (((int64_t)b * L + lq) * heads + h) * D;
      for (int d = 0; d < D; ++d) o[d] = acc[d] / z;
    }
  });
  return 0;
}

// Effective attention work of a mask: sum over rows of c_i * sum_{j kept} c_j
// (real query-key token pairs).  FLOPs = 4 * D * pairs.
int64_t fvo_real_pairs(const int32_t* grid6, const uint32_t* mask, int64_t rows_per_n /* B*heads */) {
  Geometry geo;
  if (!make_geometry(grid6, geo)) return -1;
  const int N = geo.N, words = (N + 31) / 32;
  int64_t total = 0;
  for (int64_t r = 0; r < rows_per_n * N; ++r) {
    int i = (int)(r % N);
    int64_t kv = 0;
    for (int j = 0; j < N; ++j)
      if (mask[r * words + (j >> 5)] >> (j & 31) & 1u) kv += geo.blocks[j].count;
    total += kv * geo.blocks[i].count;
  }
  return total;
}

int fvo_hardware_threads(void) { return (int)std::thread::hardware_concurrency(); }

}  // extern "C"
