// fva_attn.hip -- block-sparse flash attention and its work schedule, gfx950.
//
// VSA guide (sections 1 and 6): each query block attends only to its selected
// key/value blocks; the far-edge blocks are ragged and run on their real
// prefix, and padding never acts as a key.  FVAttn abstract: per-head work is
// uneven after Top-p routing and is balanced at runtime from the current
// routing; on one GPU this becomes longest-item-first list scheduling of
// (batch, head, query block) items over the compute units.
//
// Kernel shape (one work item = the real rows of one query block):
//   - WAVES wavefronts, each owning 32 query rows held in registers as the
//     B operand of v_mfma_f32_32x32x16_bf16;
//   - key/value rows stream through LDS in chunks of 64 keys, double
//     buffered: K row-major [key][d], V transposed [d][key] so both MFMA A
//     operands are single 16-byte LDS reads;
//   - S^T = K Q^T puts one query per lane column, so the online softmax row
//     statistics need only one cross-lane exchange (lane ^ 32) per chunk, and
//     the probabilities feed O^T += V^T P^T straight from registers;
//   - the running max is raised lazily (only when it grows by more than 8 in
//     log2 units), which skips most rescales of the O accumulators.
// A persistent grid pops items from a queue in the schedule's order; the
// dense reference runs the same core over consecutive 32*WAVES-token tiles.
#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

constexpr int KCH = 64;  // keys per chunk

struct AttnParams {
  const bf16_bits* q;
  const bf16_bits* k;
  const bf16_bits* v;
  bf16_bits* o;
  int B, L, heads;
  Geo g;
  int words;
  const uint32_t* mask;
  const int32_t* tok;    // block-ordered token ids (sparse)
  const int32_t* order;  // item order (sparse)
  uint32_t* queue;       // work counter (sparse)
  int n_items;
  int q_tiles;  // dense: query tiles per (b, h)
  float scale_log2;
  uint64_t* trace;
};

// Walks the key positions of one work item chunk by chunk: the set bits of
// the item's mask row in ascending block order (sparse) or the whole
// sequence (dense).  All threads of the workgroup hold the same state.
struct KvIter {
  const uint32_t* mrow;
  int words;
  int w;
  uint32_t bits;
  int start, count, c, nch;
  bool done;

  template <bool DENSE>
  __device__ void first(const Geo& g, const uint32_t* row, int nwords, int L) {
    c = 0;
    done = false;
    if (DENSE) {
      start = 0;
      count = L;
      nch = (L + KCH - 1) / KCH;
      return;
    }
    mrow = row;
    words = nwords;
    w = 0;
    bits = load_word(g, 0);
    next_block(g);
  }

  // mask word w with the bits of blocks >= N cleared
  __device__ uint32_t load_word(const Geo& g, int wi) const {
    uint32_t x = mrow[wi];
    const int rem = g.N - wi * 32;
    if (rem < 32) x &= (1u << rem) - 1u;
    return x;
  }

  __device__ void next_block(const Geo& g) {
    while (bits == 0u) {
      if (++w >= words) {
        done = true;
        return;
      }
      bits = load_word(g, w);
    }
    const int bit = __builtin_ctz(bits);
    bits &= bits - 1u;
    const Box bx = block_box(g, w * 32 + bit);
    start = bx.start;
    count = bx.count;
    nch = (count + KCH - 1) / KCH;
    c = 0;
  }

  template <bool DENSE>
  __device__ void advance(const Geo& g) {
    if (c + 1 < nch) {
      ++c;
      return;
    }
    if (DENSE) {
      done = true;
      return;
    }
    next_block(g);
  }

  __device__ int base() const { return start + c * KCH; }
  __device__ int valid() const { return min(KCH, count - c * KCH); }
};

template <int D, int THREADS>
struct Prefetch {
  static constexpr int KSLOTS = 4 * D;  // (row, 16-element piece) pairs of a 64-key K chunk
  static constexpr int KREG = (KSLOTS + THREADS - 1) / THREADS;
  static constexpr int VSLOTS = 4 * D;  // (d pair, 8-key group) pairs of a 64-key V chunk
  static constexpr int VREG = (VSLOTS + THREADS - 1) / THREADS;
  u32x4 kv[KREG][2];
  uint32_t vv[VREG][8];
};

template <bool DENSE>
__device__ inline int pos_to_token(const AttnParams& p, int pos) {
  return DENSE ? pos : p.tok[pos];
}

template <int D, int THREADS, bool DENSE>
__device__ inline void load_chunk(const AttnParams& p, int64_t head_off, int base, int valid,
                                  Prefetch<D, THREADS>& pf) {
  using PF = Prefetch<D, THREADS>;
  const int tid = threadIdx.x;
  const int64_t rs = (int64_t)p.heads * D;  // token row stride (elements)
#pragma unroll
  for (int u = 0; u < PF::KREG; ++u) {
    const int s = tid + u * THREADS;
    const int r = s / (D / 16), piece = s % (D / 16);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (s < PF::KSLOTS && r < valid) {
      const int64_t tok = pos_to_token<DENSE>(p, base + r);
      const u32x4* src = (const u32x4*)(p.k + head_off + tok * rs + piece * 16);
      a = src[0];
      b = src[1];
    }
    pf.kv[u][0] = a;
    pf.kv[u][1] = b;
  }
#pragma unroll
  for (int u = 0; u < PF::VREG; ++u) {
    const int s = tid + u * THREADS;
    const int dp = s % (D / 2), kg = s / (D / 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = kg * 8 + e;
      uint32_t x = 0u;
      if (s < PF::VSLOTS && r < valid) {
        const int64_t tok = pos_to_token<DENSE>(p, base + r);
        x = *(const uint32_t*)(p.v + head_off + tok * rs + dp * 2);
      }
      pf.vv[u][e] = x;
    }
  }
}

// LDS row strides (elements): 16 bytes of padding per row keeps the 16-byte
// operand reads of 32 consecutive rows on distinct bank groups.
template <int D>
struct alignas(16) Lds {
  static constexpr int KST = D + 8;
  static constexpr int VST = KCH + 8;
  bf16_bits k[2][KCH][KST];
  bf16_bits vt[2][D][VST];
};

// Key k of a chunk is stored in V^T at position pi(k): inside each group of
// 16 keys, bits 2 and 3 of the key index trade places, so the eight keys one
// lane contributes to a 16-key MFMA step are contiguous.
template <int D, int THREADS>
__device__ inline void store_chunk(Lds<D>& lds, int buf, const Prefetch<D, THREADS>& pf) {
  using PF = Prefetch<D, THREADS>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < PF::KREG; ++u) {
    const int s = tid + u * THREADS;
    if (s < PF::KSLOTS) {
      const int r = s / (D / 16), piece = s % (D / 16);
      u32x4* dst = (u32x4*)&lds.k[buf][r][piece * 16];
      dst[0] = pf.kv[u][0];
      dst[1] = pf.kv[u][1];
    }
  }
#pragma unroll
  for (int u = 0; u < PF::VREG; ++u) {
    const int s = tid + u * THREADS;
    if (s < PF::VSLOTS) {
      const int dp = s % (D / 2), kg = s / (D / 2);
      const uint32_t* w = pf.vv[u];
      // keys 8kg+0..3 -> positions 16(kg/2) + 4(kg%2) + 0..3 ; keys 8kg+4..7 -> +8
      const int p0 = 16 * (kg >> 1) + 4 * (kg & 1);
      u32x2 lo0, lo1, hi0, hi1;
      lo0[0] = (w[0] & 0xffffu) | (w[1] << 16);
      lo0[1] = (w[2] & 0xffffu) | (w[3] << 16);
      lo1[0] = (w[4] & 0xffffu) | (w[5] << 16);
      lo1[1] = (w[6] & 0xffffu) | (w[7] << 16);
      hi0[0] = (w[0] >> 16) | (w[1] & 0xffff0000u);
      hi0[1] = (w[2] >> 16) | (w[3] & 0xffff0000u);
      hi1[0] = (w[4] >> 16) | (w[5] & 0xffff0000u);
      hi1[1] = (w[6] >> 16) | (w[7] & 0xffff0000u);
      *(u32x2*)&lds.vt[buf][2 * dp][p0] = lo0;
      *(u32x2*)&lds.vt[buf][2 * dp][p0 + 8] = lo1;
      *(u32x2*)&lds.vt[buf][2 * dp + 1][p0] = hi0;
      *(u32x2*)&lds.vt[buf][2 * dp + 1][p0 + 8] = hi1;
    }
  }
}

__device__ inline uint64_t wall_ticks() { return __builtin_amdgcn_s_memrealtime(); }

template <int D, int WAVES, bool DENSE>
__global__ __launch_bounds__(WAVES * 64) void attn_kernel(AttnParams p) {
  constexpr int THREADS = WAVES * 64;
  constexpr int QROWS = WAVES * 32;
  constexpr int DS = D / 16;  // 16-wide d steps of Q K^T
  constexpr int DT = D / 32;  // 32-row d tiles of O^T
  __shared__ Lds<D> lds;
  __shared__ int item_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, hi = lane >> 5;

  uint64_t t_first = 0, t_last = 0, busy = 0, nitems = 0;

  for (int iter = 0;; ++iter) {
    // ---- fetch a work item
    int item;
    if (DENSE) {
      if (iter > 0) break;
      const int per = (p.n_items + 7) / 8;  // consecutive items share an XCD (blockIdx % 8)
      item = (blockIdx.x % 8) * per + blockIdx.x / 8;
      if (item >= p.n_items) break;
    } else {
      if (tid == 0) {
        const uint32_t slot = atomicAdd(p.queue, 1u);
        item_s = slot < (uint32_t)p.n_items ? p.order[slot] : -1;
      }
      __syncthreads();
      item = item_s;
      if (item < 0) break;
    }
    const uint64_t t_start = wall_ticks();

    int b, h, qbase, qcount;
    const uint32_t* mrow = nullptr;
    if (DENSE) {
      const int tile = item % p.q_tiles;
      const int bh = item / p.q_tiles;
      h = bh % p.heads;
      b = bh / p.heads;
      qbase = tile * QROWS;
      qcount = min(QROWS, p.L - qbase);
    } else {
      const int i = item % p.g.N;
      const int bh = item / p.g.N;
      h = bh % p.heads;
      b = bh / p.heads;
      const Box bx = block_box(p.g, i);
      qbase = bx.start;
      qcount = bx.count;
      mrow = p.mask + (int64_t)item * p.words;
    }
    const int64_t head_off = (int64_t)b * p.L * p.heads * D + (int64_t)h * D;
    const int64_t rs = (int64_t)p.heads * D;

    // ---- Q fragment: row 32*wave + lr, d = 16s + 8hi .. +7
    const int qrow = wave * 32 + lr;
    const bool wave_active = wave * 32 < qcount;
    bf16x8 qf[DS];
    {
      int64_t qtok = 0;
      const bool ok = qrow < qcount;
      if (ok) qtok = pos_to_token<DENSE>(p, qbase + qrow);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = *(const u32x4*)(p.q + head_off + qtok * rs + 16 * s + 8 * hi);
        qf[s] = __builtin_bit_cast(bf16x8, x);
      }
    }

    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    float m_used = -INFINITY, lsum = 0.f;

    KvIter it;
    it.template first<DENSE>(p.g, mrow, p.words, p.L);
    Prefetch<D, THREADS> pf;
    int buf = 0;
    if (!it.done) {
      load_chunk<D, THREADS, DENSE>(p, head_off, it.base(), it.valid(), pf);
      store_chunk<D, THREADS>(lds, 0, pf);
    }
    __syncthreads();

    while (!it.done) {
      const int valid = it.valid();
      KvIter nx = it;
      nx.template advance<DENSE>(p.g);
      if (!nx.done) load_chunk<D, THREADS, DENSE>(p, head_off, nx.base(), nx.valid(), pf);

      if (wave_active) {
        // S^T (keys x queries) for 64 keys: two 32x32 tiles
        f32x16 s[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const bf16x8 a = *(const bf16x8*)&lds.k[buf][32 * kt + lr][16 * ds + 8 * hi];
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], s[kt], 0, 0, 0);
          }
        }
        // online softmax in log2 units; lane holds keys 32kt + 8(r/4) + 4hi + r%4
        float mloc = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = s[kt][r] * p.scale_log2;
            if (valid < KCH) {
              const int key = 32 * kt + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key >= valid) x = -INFINITY;
            }
            s[kt][r] = x;
            mloc = fmaxf(mloc, x);
          }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_used, mloc);
        if (__any(m_new > m_used + 8.0f)) {
          const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
          lsum *= alpha;
          m_used = m_new;
        }
        bf16x8 pb[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pe = __builtin_amdgcn_exp2f(s[kt][8 * qh + e] - m_used);
              lsum += pe;
              pb[kt][qh][e] = (__bf16)pe;
            }
        // O^T (d x queries) += V^T P^T
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qh = 0; qh < 2; ++qh)
#pragma unroll
            for (int t = 0; t < DT; ++t) {
              const bf16x8 a = *(const bf16x8*)&lds.vt[buf][32 * t + lr][32 * kt + 16 * qh + 8 * hi];
              acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][qh], acc[t], 0, 0, 0);
            }
      }

      if (!nx.done) store_chunk<D, THREADS>(lds, buf ^ 1, pf);
      __syncthreads();
      buf ^= 1;
      it = nx;
    }

    // ---- normalise and store the real rows (lane and lane ^ 32 share a row)
    float lt = 0.f;
    if (wave_active) lt = lsum + __shfl_xor(lsum, 32);
    if (wave_active && qrow < qcount) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int64_t otok = pos_to_token<DENSE>(p, qbase + qrow);
      bf16_bits* dst = p.o + head_off + otok * rs;
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 w;
          w[0] = (uint32_t)f32_to_bf16(acc[t][4 * g4 + 0] * inv) | ((uint32_t)f32_to_bf16(acc[t][4 * g4 + 1] * inv) << 16);
          w[1] = (uint32_t)f32_to_bf16(acc[t][4 * g4 + 2] * inv) | ((uint32_t)f32_to_bf16(acc[t][4 * g4 + 3] * inv) << 16);
          *(u32x2*)(dst + 32 * t + 8 * g4 + 4 * hi) = w;
        }
    }
    const uint64_t t_end = wall_ticks();
    if (nitems == 0) t_first = t_start;
    t_last = t_end;
    busy += t_end - t_start;
    ++nitems;
    __syncthreads();
  }

  if (p.trace && tid == 0) {
    const uint32_t hwid = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID
    const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20);  // HW_REG_XCC_ID
    uint64_t* t = p.trace + (int64_t)blockIdx.x * 4;
    t[0] = t_first;
    t[1] = t_last;
    t[2] = busy;
    t[3] = (nitems << 40) | ((uint64_t)(xcc & 0xffu) << 32) | hwid;
  }
}

// ---------------------------------------------------------------------------
// Schedule kernels
// ---------------------------------------------------------------------------

// Block-ordered token table and real counts: one workgroup per block.
__global__ __launch_bounds__(256) void layout_kernel(Geo g, int32_t* __restrict__ tok, int32_t* __restrict__ cnt) {
  const int n = blockIdx.x;
  const Box bx = block_box(g, n);
  if (threadIdx.x == 0) cnt[n] = bx.count;
  const int plane = bx.eh * bx.ew;
  for (int r = threadIdx.x; r < bx.count; r += blockDim.x) {
    const int dt = r / plane, rem = r % plane;
    const int dy = rem / bx.ew, dx = rem % bx.ew;
    tok[bx.start + r] = ((bx.t0 + dt) * g.H + (bx.y0 + dy)) * g.W + bx.x0 + dx;
  }
}

// Work of every item (real query-key token pairs) and its sort key; resets
// the queue.  cost < 2^32 because a block holds at most 256 tokens and
// L < 2^24.  key = cost << 32 | (~item): descending keys give descending cost,
// ties to the lower item id.
__global__ __launch_bounds__(256) void cost_kernel(const uint32_t* __restrict__ mask, const int32_t* __restrict__ cnt,
                                                   int N, int words, int n_items, bool lpt,
                                                   uint64_t* __restrict__ keys, uint32_t* __restrict__ rank,
                                                   int32_t* __restrict__ order, uint32_t* __restrict__ queue) {
  const int item = blockIdx.x * blockDim.x + threadIdx.x;
  if (item == 0) *queue = 0u;
  if (item >= n_items) return;
  if (!lpt) {
    order[item] = item;
    return;
  }
  const uint32_t* row = mask + (int64_t)item * words;
  uint32_t kv = 0;
  for (int w = 0; w < words; ++w) {
    uint32_t bits = row[w];
    const int rem = N - w * 32;
    if (rem < 32) bits &= (1u << rem) - 1u;  // ignore bits of blocks >= N
    while (bits) {
      const int j = w * 32 + __builtin_ctz(bits);
      bits &= bits - 1u;
      kv += (uint32_t)cnt[j];
    }
  }
  const uint32_t cost = (uint32_t)cnt[item % N] * kv;
  keys[item] = ((uint64_t)cost << 32) | (uint64_t)(~(uint32_t)item);
  rank[item] = 0u;
}

// rank[a] += #{b in this tile : key[b] > key[a]}  (keys are distinct)
__global__ __launch_bounds__(256) void rank_kernel(const uint64_t* __restrict__ keys, int n_items,
                                                   uint32_t* __restrict__ rank) {
  __shared__ uint64_t tile[2048];
  const int a = blockIdx.x * 256 + threadIdx.x;
  const int b0 = blockIdx.y * 2048;
  const int nb = min(2048, n_items - b0);
  for (int t = threadIdx.x; t < nb; t += 256) tile[t] = keys[b0 + t];
  __syncthreads();
  if (a >= n_items) return;
  const uint64_t ka = keys[a];
  uint32_t c = 0;
  for (int t = 0; t < nb; ++t) c += tile[t] > ka ? 1u : 0u;
  if (c) atomicAdd(&rank[a], c);
}

__global__ __launch_bounds__(256) void scatter_kernel(const uint32_t* __restrict__ rank, int n_items,
                                                      int32_t* __restrict__ order) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a < n_items) order[rank[a]] = a;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
int attn_waves_for_block(int vol) {
  if (vol <= 64) return 2;
  if (vol <= 128) return 4;
  return 8;
}

template <int D, int WAVES, bool DENSE>
static const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&attn_kernel<D, WAVES, DENSE>);
}

static const void* sparse_kernel(int D, int waves) {
  if (D == 128) {
    if (waves == 2) return kernel_ptr<128, 2, false>();
    if (waves == 4) return kernel_ptr<128, 4, false>();
    return kernel_ptr<128, 8, false>();
  }
  if (waves == 2) return kernel_ptr<64, 2, false>();
  if (waves == 4) return kernel_ptr<64, 4, false>();
  return kernel_ptr<64, 8, false>();
}

int attn_persistent_workgroups(int D, int waves, int* err) {
  int dev = 0, cus = 0, occ = 0;
  *err = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, sparse_kernel(D, waves), waves * 64, 0) != hipSuccess) {
    *err = 1;
    return 0;
  }
  if (occ < 1) occ = 1;
  return cus * occ;
}

template <int D, int WAVES>
static void launch_sparse_t(const AttnParams& prm, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_kernel<D, WAVES, false>), dim3(grid), dim3(WAVES * 64), 0, st, prm);
}

hipError_t launch_sparse_attn(const AttnLaunch& a, bool lpt, hipStream_t st) {
  const int n_items = a.B * a.heads * a.g.N;
  const int words = (a.g.N + 31) / 32;
  hipLaunchKernelGGL(layout_kernel, dim3(a.g.N), dim3(256), 0, st, a.g, a.tok, a.blk_cnt);
  hipLaunchKernelGGL(cost_kernel, dim3((n_items + 255) / 256), dim3(256), 0, st, a.mask, a.blk_cnt, a.g.N, words,
                     n_items, lpt, a.keys, a.rank, a.order, a.queue);
  if (lpt) {
    hipLaunchKernelGGL(rank_kernel, dim3((n_items + 255) / 256, (n_items + 2047) / 2048), dim3(256), 0, st, a.keys,
                       n_items, a.rank);
    hipLaunchKernelGGL(scatter_kernel, dim3((n_items + 255) / 256), dim3(256), 0, st, a.rank, n_items, a.order);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  AttnParams prm;
  prm.q = (const bf16_bits*)a.q;
  prm.k = (const bf16_bits*)a.k;
  prm.v = (const bf16_bits*)a.v;
  prm.o = (bf16_bits*)a.o;
  prm.B = a.B;
  prm.L = a.L;
  prm.heads = a.heads;
  prm.g = a.g;
  prm.words = words;
  prm.mask = a.mask;
  prm.tok = a.tok;
  prm.order = a.order;
  prm.queue = a.queue;
  prm.n_items = n_items;
  prm.q_tiles = 0;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  prm.trace = a.trace;

  const int waves = attn_waves_for_block(a.g.bt * a.g.bh * a.g.bw);
  int err = 0;
  const int grid = attn_persistent_workgroups(a.D, waves, &err);
  if (err) return hipErrorInvalidValue;
  if (a.D == 128) {
    if (waves == 2) launch_sparse_t<128, 2>(prm, grid, st);
    else if (waves == 4) launch_sparse_t<128, 4>(prm, grid, st);
    else launch_sparse_t<128, 8>(prm, grid, st);
  } else {
    if (waves == 2) launch_sparse_t<64, 2>(prm, grid, st);
    else if (waves == 4) launch_sparse_t<64, 4>(prm, grid, st);
    else launch_sparse_t<64, 8>(prm, grid, st);
  }
  return hipGetLastError();
}

hipError_t launch_dense_attn(const void* q, const void* k, const void* v, void* o, int B, int L, int heads, int D,
                             float scale, hipStream_t st) {
  constexpr int WAVES = 8;
  AttnParams prm = {};
  prm.q = (const bf16_bits*)q;
  prm.k = (const bf16_bits*)k;
  prm.v = (const bf16_bits*)v;
  prm.o = (bf16_bits*)o;
  prm.B = B;
  prm.L = L;
  prm.heads = heads;
  prm.q_tiles = (L + WAVES * 32 - 1) / (WAVES * 32);
  prm.n_items = B * heads * prm.q_tiles;
  prm.scale_log2 = scale * 1.4426950408889634f;
  prm.trace = nullptr;
  const int grid = 8 * ((prm.n_items + 7) / 8);
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, WAVES, true>), dim3(grid), dim3(WAVES * 64), 0, st, prm);
  else
    hipLaunchKernelGGL((attn_kernel<64, WAVES, true>), dim3(grid), dim3(WAVES * 64), 0, st, prm);
  return hipGetLastError();
}

}  // namespace fva
