// fva_attn.hip -- block-sparse flash attention and its work schedule, gfx950.
//
// VSA guide (sections 1 and 6): each query block attends only to its selected
// key/value blocks; the far-edge blocks are ragged and run on their real
// prefix, and padding never acts as a key.  The guide's backend reorders the
// sequence into a block-ordered tiled layout before its kernel; here the keys
// and values are likewise re-tiled once per call, directly into the byte
// image each 64-key chunk has in LDS.
//
// FVAttn abstract: Top-p routing leaves uneven per-head work, which runtime
// load balancing moves between ranks by whole heads, from the current
// routing.  The one-GPU share: heads are assigned longest-first to the eight
// XCDs (each XCD has its own L2, so the keys and values of a head stay in one
// cache), each XCD's queue runs its heads' (query block) items longest-first,
// and a workgroup whose queue is empty takes items from the other XCDs (the
// per-XCD schedule turns that off, so that each XCD plays one rank).
//
// Attention kernel (one work item = the real rows of one query block, or of a
// small group of small blocks):
//   - WAVES wavefronts, each owning QT sub-tiles of 32 query rows held in
//     registers as B operands of v_mfma_f32_32x32x16_bf16, so each K or V^T
//     operand read from LDS feeds QT MFMAs;
//   - chunks of 64 keys move from HBM straight into a 4-stage LDS ring, three
//     chunks ahead of the one being computed; a chunk is K [64][D] followed by
//     V^T [D][64], both in 16-byte pieces stored piece-major, so the MFMA
//     operand reads of 16-lane groups hit distinct banks without padding;
//   - S^T = K Q^T gives each lane one query column, so the softmax row
//     statistics need one cross-half lane swap per 32 keys, and the bf16
//     probabilities feed O^T += V^T P^T from registers;
//   - per 32 keys, Q K^T of the next 32 keys, P V of the current ones and the
//     exponentials are interleaved so the matrix cores and the vector ALUs
//     work at the same time;
//   - Q is pre-multiplied by the score scale in log2 units and the Q K^T
//     accumulator starts at minus the row's running max, so each exponent
//     argument comes straight out of the MFMA;
//   - the running max is raised lazily (only when it grows by more than 8 in
//     log2 units), which skips most rescales of the O accumulators.
#include "fva_dev.h"
#include "fva_kernels.h"

namespace fva {

constexpr int KCH = 64;     // keys per chunk
constexpr int STAGES = 4;   // LDS ring depth
constexpr int NXCD = 8;     // XCDs of an MI355X

// A chunk of 64 keys, in LDS and in the tiled copy in HBM alike (the copy
// is byte-identical to the LDS image, so it moves by direct global-to-LDS
// loads), stored as 16-byte pieces (8 bf16) in piece-major order:
//   K:   piece c (d = 8c .. 8c+7) of key row r at piece index c*64 + r;
//   V^T: piece g (positions 8g .. 8g+7, key k at position pi(k)) of row d at
//        index D*8 + g*D + d.
// An MFMA operand read by 16 consecutive lanes (16 consecutive K rows, or 16
// consecutive d) then covers 256 contiguous bytes, one piece per bank group,
// so there are no bank conflicts without any row padding; the image is
// exactly 2*64*D*2 bytes (a whole number of 1 KB DMA pieces, 4 per
// wavefront for D = 128), and each operand address is a per-lane base plus
// a compile-time offset.
template <int D>
struct Lds {
  static constexpr int VBASE = KCH * D;
  static constexpr int ELEMS = 2 * KCH * D;
  __host__ __device__ static constexpr int k_off(int row, int col) { return ((col >> 3) * KCH + row) * 8 + (col & 7); }
  __host__ __device__ static constexpr int v_off(int d, int pos) { return VBASE + ((pos >> 3) * D + d) * 8 + (pos & 7); }
};

// Key k of a chunk sits at V^T position pi(k): inside each group of 16 keys,
// bits 2 and 3 of the index trade places, so the eight keys a lane feeds one
// 16-key MFMA step are contiguous.  pi is its own inverse.
__host__ __device__ inline int pi_key(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

struct AttnParams {
  const bf16_bits* q;
  const bf16_bits* k;
  const bf16_bits* v;
  bf16_bits* o;
  int B, L, heads;  // heads: the launch's own heads (hd.n)
  Heads hd;         // which heads of the tensors, masks and counts they are
  Geo g;
  int words, cpb;          // mask words per row; chunk slots per block
  const uint32_t* mask;
  const int32_t* tok;      // block-ordered token ids (sparse)
  const int32_t* cnt;      // real tokens per block (sparse)
  const bf16_bits* tiles;  // chunk images (sparse)
  const int32_t* order;    // item order (sparse)
  const int32_t* qoff;     // [NXCD + 1] queue segments in order (sparse)
  uint32_t* qctr;          // [NXCD] pop counters (sparse)
  int steal;               // sparse: an idle workgroup takes items from the other XCDs' queues
  int n_items;
  int q_tiles;  // dense: query tiles per (b, h)
  // sparse work items are groups of up to 4 query blocks: a (gt, gh, gw) box
  // of blocks on the block grid, gT x gH x gW groups per (b, h); each member
  // block gets wpb wavefronts
  int gt, gh, gw, gT, gH, gW, n_groups, wpb;
  float scale_log2;
  uint64_t* trace;
  // sparse: the shape tag the plan wrote into the workspace, and the value
  // this launch expects there (a mismatch: the workspace holds no plan for
  // this shape, and O is filled with NaN instead)
  const uint64_t* plan_tag;
  uint64_t want_tag;
};

// Block index of member k of group gid, or -1 past the grid's edge.
__device__ inline int group_member(const AttnParams& p, int gid, int k) {
  const int gwi = gid % p.gW, ghi = (gid / p.gW) % p.gH, gti = gid / (p.gW * p.gH);
  const int c = k % p.gw, b = (k / p.gw) % p.gh, a = k / (p.gw * p.gh);
  const int it = gti * p.gt + a, ih = ghi * p.gh + b, iw = gwi * p.gw + c;
  if (it >= p.g.nT || ih >= p.g.nH || iw >= p.g.nW) return -1;
  return (it * p.g.nH + ih) * p.g.nW + iw;
}

// One chunk of a work item's key sequence.
struct Chunk {
  int slot;   // chunk image index
  int valid;  // real keys in the chunk (1..64)
  int blk;    // sparse: key block of the chunk
};

// Walks the chunks of one work item: the set bits of the union of its member
// blocks' mask rows (staged in LDS, bits >= N cleared) in ascending block
// order (sparse) or the whole sequence (dense).  Every thread of the
// workgroup holds the same state.
struct KvIter {
  const uint32_t* umask;  // LDS
  const uint16_t* cnt;    // LDS: real tokens per block
  int w, words, c, nch, count, slot0, blk;
  uint32_t bits;
  bool done;

  __device__ void next_block(const Geo& g, int bh, int cpb) {
    while (bits == 0u) {
      if (++w >= words) {
        done = true;
        return;
      }
      bits = umask[w];
    }
    blk = w * 32 + __builtin_ctz(bits);
    bits &= bits - 1u;
    count = cnt[blk];
    nch = (count + KCH - 1) / KCH;
    slot0 = (bh * g.N + blk) * cpb;
    c = 0;
  }

  template <bool DENSE>
  __device__ void first(const Geo& g, int nwords, int L, int bh, int cpb) {
    done = false;
    c = 0;
    blk = -1;
    if (DENSE) {
      count = L;
      nch = (L + KCH - 1) / KCH;
      slot0 = bh * cpb;
      return;
    }
    words = nwords;
    w = 0;
    bits = umask[0];
    next_block(g, bh, cpb);
  }

  template <bool DENSE>
  __device__ void advance(const Geo& g, int bh, int cpb) {
    if (c + 1 < nch) {
      ++c;
      return;
    }
    if (DENSE) {
      done = true;
      return;
    }
    next_block(g, bh, cpb);
  }

  __device__ Chunk chunk() const {
    Chunk ck;
    ck.slot = slot0 + c;
    ck.valid = min(KCH, count - c * KCH);
    ck.blk = blk;
    return ck;
  }
};

// A chunk image moves from HBM straight into LDS, 1 KB per wavefront
// instruction (global_load_lds_dwordx4: lane l's 16 bytes land at the LDS
// address in M0 + 16 l).  It is written as inline assembly so that the
// compiler's wait counting stays blind to these loads: its LDS waits inside
// the attention loop then stay fine-grained.  The instruction has no
// register result; completion is tracked here, by the explicit vmcnt waits
// before each barrier (wait_vmem), and the barrier (barrier_lds) orders
// every LDS read of a stage after the wait for the loads into it.
// Every wavefront issues the same number (PER_WAVE) of instructions per
// chunk, so that a wait for "all but the newest chunk" is one vmcnt
// immediate.  Wavefront w loads the PER_WAVE consecutive pieces from piece
// PER_WAVE * w on: one scalar base for the chunk, the wavefront's offset in
// a VGPR fixed for the kernel, and the piece in the instruction's immediate
// offset, which moves the global and the LDS address alike (M0 holds the
// wavefront's first LDS piece).  So a chunk costs a few scalar instructions
// besides the loads.
template <int D, int WAVES>
struct ChunkDma {
  static constexpr int BYTES = Lds<D>::ELEMS * 2;
  static constexpr int PIECES = BYTES / 1024;
  static constexpr int PER_WAVE = PIECES / WAVES;
  static_assert(BYTES % 1024 == 0 && PIECES == PER_WAVE * WAVES, "whole 1 KB pieces, the same count per wavefront");
  static_assert(PER_WAVE == 2 || PER_WAVE == 4, "pieces per wavefront: immediate offsets below 4 KB");
  // voff: this lane's byte offset in the chunk image (wavefront's first piece + 16 * lane)
  __device__ static uint32_t lane_offset(int wave, int lane) {
    return (uint32_t)wave * (PER_WAVE * 1024u) + (uint32_t)lane * 16u;
  }
  __device__ static void issue(const bf16_bits* tiles, int slot, bf16_bits* lds, int wave, uint32_t voff) {
    // (the slot is the same in every lane; say so, so that it stays scalar)
    const uint32_t us = (uint32_t)__builtin_amdgcn_readfirstlane(slot);
    const uint64_t gbase = (uint64_t)(uintptr_t)tiles + (uint64_t)us * (uint64_t)BYTES;
    const uint32_t lbase = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)((char*)lds) +
                           (uint32_t)wave * (PER_WAVE * 1024u);
    if constexpr (PER_WAVE == 4)
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "global_load_lds_dwordx4 %1, %2\n\t"
          "global_load_lds_dwordx4 %1, %2 offset:1024\n\t"
          "global_load_lds_dwordx4 %1, %2 offset:2048\n\t"
          "global_load_lds_dwordx4 %1, %2 offset:3072"
          :
          : "s"(lbase), "v"(voff), "s"(gbase)
          : "memory", "m0");
    else
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "global_load_lds_dwordx4 %1, %2\n\t"
          "global_load_lds_dwordx4 %1, %2 offset:1024"
          :
          : "s"(lbase), "v"(voff), "s"(gbase)
          : "memory", "m0");
  }
};

// Workgroup barrier for LDS data: waits for this wavefront's LDS operations
// and meets the other wavefronts, but leaves global loads in flight (a
// __syncthreads() would wait for all of them, including the chunk loads
// issued ahead; callers wait for the loads they need with wait_vmem).  The
// empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ inline void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// wait until at most N of this wavefront's global loads (including those
// into LDS) are outstanding; expcnt and lgkmcnt are not waited for
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N <= 15, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

template <bool DENSE>
__device__ inline int pos_to_token(const AttnParams& p, int pos) {
  return DENSE ? pos : p.tok[pos];
}

__device__ inline uint64_t wall_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// max and sum of the values of lanes l and l ^ 32.  permlane32_swap on two
// copies of x leaves the low half of x in every lane of one result and the
// high half in every lane of the other.
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Running max of a row before it has seen a real key: finite, so the
// exponent argument needs no special case, and far enough below any real
// score (in log2 units) that the first real key raises it and scales the
// empty accumulators by exp2(-huge) = 0.
constexpr float M_NONE = -1.0e30f;
// lazy raise: the running max moves only when a new score exceeds it by more
// than this many log2 units, so probabilities stay <= 2^RAISE_SLACK
constexpr float RAISE_SLACK = 8.0f;

// The attention kernel.  A work item is processed by WAVES wavefronts; each
// owns QT sub-tiles of 32 query rows (rows 32*(QT*wave + qt) + lr of the
// item) and therefore reuses every K and V^T operand it reads from LDS for QT
// MFMAs.  Per 64-key chunk and wavefront: 2*D/16 K reads feeding QT MFMAs each
// (S^T), and 4*D/32 V^T reads feeding QT MFMAs each (O^T).
//
// GRP: work items are groups of query blocks (p.wpb wavefronts per block).
template <int D, int WAVES, int QT, bool DENSE, bool GRP>
__global__ __launch_bounds__(WAVES * 64) void attn_kernel(AttnParams p) {
  static_assert(!(DENSE && GRP), "dense items are query tiles");
  constexpr int THREADS = WAVES * 64;
  constexpr int QROWS = WAVES * QT * 32;
  constexpr int DS = D / 16;  // 16-wide d steps of Q K^T
  constexpr int DT = D / 32;  // 32-row d tiles of O^T
  // the LDS ring: one array per stage, so that the compiler sees that the
  // loads in flight into one stage do not touch the stages being read
  __shared__ __attribute__((aligned(16))) bf16_bits ring0[Lds<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring1[Lds<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring2[Lds<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_bits ring3[Lds<D>::ELEMS];
  __shared__ int item_s;
  // Tables sized by the launch (dynamic LDS, sparse_lds_bytes): the item's
  // mask, i.e. the union of its members' rows (umask, `words` words) and,
  // for groups, each member's own row (gmask, 4 x `words`), and the real
  // tokens of every block (cnt_s, N entries), read by the chunk walk at each
  // block change (a table lookup instead of the three integer divisions of
  // the block's geometry, which cost the walk some 80 scalar instructions
  // per block).  Sized by N rather than by the largest grid, they leave the
  // rest of the CU's LDS to kernels of other streams.
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn_lds[];
  uint32_t* umask = dyn_lds;
  uint32_t* gmask = dyn_lds + p.words;  // member k's row at gmask + k * words
  uint16_t* cnt_s = (uint16_t*)(dyn_lds + (GRP ? 5 : 1) * p.words);
  static_assert(STAGES == 4, "four ring stages");
  auto stage = [&](int sidx) -> bf16_bits* {
    return sidx == 0 ? ring0 : (sidx == 1 ? ring1 : (sidx == 2 ? ring2 : ring3));
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wavefront
  const int lr = lane & 31, hi = lane >> 5;
  const float cl2 = p.scale_log2;

  if (!DENSE && *p.plan_tag != p.want_tag) {
    // no plan for this shape in the workspace: every element of O becomes
    // NaN (grid-stride over the persistent workgroups) rather than output
    // computed from mismatched tables
    const int64_t n = (int64_t)p.B * p.L * p.heads * D;
    for (int64_t e = (int64_t)blockIdx.x * THREADS + tid; e < n; e += (int64_t)gridDim.x * THREADS) {
      const int64_t row = e / D;  // (b*L + l)*heads + h
      p.o[((row / p.heads) * p.hd.stride + p.hd.h0 + row % p.heads) * D + e % D] = (bf16_bits)0x7FC0;
    }
    return;
  }
  if (!DENSE)  // ordered before any read by the barrier after the first item fetch
    for (int j = tid; j < p.g.N; j += THREADS) cnt_s[j] = (uint16_t)p.cnt[j];
  uint64_t t_first = 0, t_last = 0, busy = 0, nitems = 0;

  // Work items come from the XCD queues (thread 0 pops them).  The next item
  // is popped when the current one's chunk loop ends and its mask rows are
  // staged in LDS while the current item's output is written, so an item
  // starts with a single round trip to memory (Q and its first chunks
  // together).  (Popping it earlier, while the current item runs, reserves
  // it too soon: the kernel's tail grew and wan14b ran 1.7% slower.)
  // take a slot of this XCD's queue (thread 0; its queue's segment is read
  // from memory each time, so that nothing of it stays live in registers
  // across the chunk loop)
  auto take_own_slot = [&]() -> uint32_t {
    const int x = (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 7);  // HW_REG_XCC_ID
    const int n = p.qoff[x + 1] - p.qoff[x];
    return n > 0 ? atomicAdd(&p.qctr[x], 1u) : ~0u;
  };
  // the item of a taken slot, or (stealing) one from another queue, or -1
  auto item_of_slot = [&](uint32_t s) -> int {
    const int my_xcd = (int)(__builtin_amdgcn_s_getreg((15 << 11) | 20) & 7);
    const int n0 = p.qoff[my_xcd + 1] - p.qoff[my_xcd];
    if (s < (uint32_t)n0) return p.order[p.qoff[my_xcd] + s];
    for (int t = 1; t < (p.steal ? NXCD : 1); ++t) {
      const int x = (my_xcd + t) % NXCD;
      const int n = p.qoff[x + 1] - p.qoff[x];
      if (n <= 0 || __atomic_load_n(&p.qctr[x], __ATOMIC_RELAXED) >= (uint32_t)n) continue;
      const uint32_t u = atomicAdd(&p.qctr[x], 1u);
      if (u < (uint32_t)n) return p.order[p.qoff[x] + u];
    }
    return -1;
  };
  // the item's mask rows in LDS: the union of its members' rows (bits >= N
  // cleared) and, for groups, each member's own row
  auto stage_mask = [&](int item) {
    if (!GRP) {
      const int n = item % p.g.N;
      const uint32_t* row = p.mask + (p.hd.global(item / p.g.N) * p.g.N + n) * p.words;
      for (int wi = tid; wi < p.words; wi += THREADS) {
        const int rem = p.g.N - wi * 32;
        umask[wi] = rem < 32 ? row[wi] & ((1u << rem) - 1u) : row[wi];
      }
    } else {
      const int gid = item % p.n_groups;
      const int bhg = item / p.n_groups;
      const int ng = p.gt * p.gh * p.gw;
      for (int wi = tid; wi < p.words; wi += THREADS) {
        uint32_t u = 0u;
        for (int k = 0; k < 4; ++k) {
          const int n = k < ng ? group_member(p, gid, k) : -1;
          const uint32_t x = n >= 0 ? p.mask[(p.hd.global(bhg) * p.g.N + n) * p.words + wi] : 0u;
          gmask[k * p.words + wi] = x;
          u |= x;
        }
        const int rem = p.g.N - wi * 32;
        umask[wi] = rem < 32 ? u & ((1u << rem) - 1u) : u;
      }
    }
  };
  if (!DENSE) {
    if (tid == 0) item_s = item_of_slot(take_own_slot());
    __syncthreads();
    if (item_s >= 0) stage_mask(item_s);
    __syncthreads();
  }

  for (int iter = 0;; ++iter) {
    // ---- the work item (its mask rows are already in LDS)
    int item;
    if (DENSE) {
      if (iter > 0) break;
      const int per = (p.n_items + NXCD - 1) / NXCD;  // consecutive tiles share an XCD (blockIdx % 8)
      item = (blockIdx.x % NXCD) * per + blockIdx.x / NXCD;
      if (item >= p.n_items) break;
    } else {
      item = item_s;
      if (item < 0) break;
    }
    const uint64_t t_start = wall_ticks();

    int b, h, bh;
    int qbase, qcount;  // this wavefront's query block: first position, real rows
    int row0;           // first row of this wavefront inside that block
    int mine = -1;      // groups: this wavefront's member index, or -1
    int ksel = -1;      // -1: every key of every chunk; 0 / 1: only key half ksel of each chunk
    bool merge = false;  // some tile of the item is split over two wavefronts (uniform)
    KvIter it;
    it.umask = umask;
    it.cnt = cnt_s;
    if (DENSE) {
      const int tile = item % p.q_tiles;
      bh = item / p.q_tiles;
      qbase = tile * QROWS;
      qcount = min(QROWS, p.L - qbase);
      row0 = 32 * QT * wave;
    } else if (!GRP) {
      const int n = item % p.g.N;
      bh = item / p.g.N;
      const Box bx = block_box(p.g, n);
      qbase = bx.start;
      qcount = bx.count;
      // Ragged blocks: the per-chunk work of a 32-row tile is two key halves,
      // and the four SIMDs of the CU hold wavefronts w and w + 4.  A block of
      // 5 or 6 tiles gives its tiles 4 and 5 two wavefronts each, one per key
      // half, and a block of at most 4 tiles does so for all its tiles, so
      // every SIMD carries at most 3 (resp. 2) halves per chunk instead of 4;
      // the two partial softmax states of a tile are merged at the end.
      const int nt = (qcount + 32 * QT - 1) / (32 * QT);
      merge = QT == 1 && nt <= 6;
      int tile = wave;
      if (QT == 1 && nt <= 4) {
        tile = wave >> 1;
        ksel = wave & 1;
      } else if (QT == 1 && nt <= 6 && wave >= 4) {
        tile = 4 + ((wave - 4) >> 1);
        ksel = wave & 1;
      }
      row0 = 32 * QT * tile;
    } else {
      const int gid = item % p.n_groups;
      bh = item / p.n_groups;
      // The member block this wavefront serves.  Wavefronts w and w + 4
      // share a SIMD, so with 2 wavefronts per member the members pair up on
      // SIMDs 0-1 (wavefronts 0, 1, 4, 5) and 2-3 (2, 3, 6, 7).  Blocks that
      // are neighbours in t or in x keep many of the same key blocks, so in
      // a 2x1x2 group the diagonal members (t0, x0) + (t1, x1) share one SIMD
      // pair and (t0, x1) + (t1, x0) the other: a chunk that only two
      // neighbours keep then runs on all four SIMDs.
      int msel = wave / p.wpb, tsel = wave % p.wpb;
      if (p.wpb == 2) {
        const int pair = (wave >> 1) & 1, slot = wave >> 2;
        msel = pair == 0 ? (slot ? 3 : 0) : (slot ? 2 : 1);
        tsel = wave & 1;
      }
      const int n_mine = group_member(p, gid, msel);
      row0 = 32 * QT * tsel;
      if (n_mine >= 0) {
        mine = msel;
        const Box bx = block_box(p.g, n_mine);
        qbase = bx.start;
        qcount = bx.count;
      } else {
        qbase = 0;
        qcount = 0;
      }
    }
    h = bh % p.heads;
    b = bh / p.heads;
    const int64_t rs = (int64_t)p.hd.stride * D;
    const int64_t head_off = (int64_t)b * p.L * rs + (int64_t)(p.hd.h0 + h) * D;

    // ---- Q fragments: sub-tile qt holds row row0 + 32*qt + lr of the block, d = 16s + 8hi .. +7,
    //      times the score scale in log2 units (rounded to bf16), so that the
    //      Q K^T MFMA yields exponent arguments directly
    const bool wave_active = row0 < qcount;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x8 qf[QT][DS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int qrow = row0 + 32 * qt + lr;
      const bool ok = qrow < qcount;
      int64_t qtok = 0;
      if (ok) qtok = pos_to_token<DENSE>(p, qbase + qrow);
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = *(const u32x4*)(p.q + head_off + qtok * rs + 16 * s + 8 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2_t pr = {(__bf16)(__uint_as_float(x[e] << 16) * cl2),
                               (__bf16)(__uint_as_float(x[e] & 0xffff0000u) * cl2)};
          x[e] = __builtin_bit_cast(uint32_t, pr);
        }
        qf[qt][s] = __builtin_bit_cast(bf16x8, x);
      }
    }

    // Softmax state of each row (log2 units).  m_run: the running max the
    // O^T accumulators and the row sum are scaled by.  moff: the offset the
    // Q K^T MFMAs subtract (their accumulator starts at negm = -moff), equal
    // to m_run once the row has seen a real key and 0 before.  thr: the
    // raise threshold on those offset scores.
    f32x16 acc[QT][DT], negm[QT];
    float m_run[QT], moff[QT], lsum[QT], thr[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qt][t][r] = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) negm[qt][r] = 0.f;
      m_run[qt] = M_NONE;
      moff[qt] = 0.f;
      thr[qt] = M_NONE + RAISE_SLACK;
      lsum[qt] = 0.f;
    }

    // ---- pipeline: `it` is the next chunk to load; the ring holds `ready`
    //      chunks (loaded or in flight) starting with the one being
    //      computed, with real key counts v0, v1, v2 as this wavefront sees them
    it.template first<DENSE>(p.g, p.words, p.L, bh, p.cpb);
    // real keys of the chunks in the ring as this wavefront sees them: a key
    // block its own query block did not keep counts as 0 real keys
    auto seen = [&](const Chunk& ck) -> int {
      if (!GRP) return ck.valid;  // a single member: the union is its own row
      if (mine < 0) return 0;
      return ((gmask[mine * p.words + (ck.blk >> 5)] >> (ck.blk & 31)) & 1u) ? ck.valid : 0;
    };
    // chunks arrive by direct loads three chunks ahead of the one being computed
    constexpr int LOOK = 3;
    using Dma = ChunkDma<D, WAVES>;
    const uint32_t dma_voff = Dma::lane_offset(wave, lane);
    int ready = 0, v0 = 0, v1 = 0, v2 = 0;
#pragma unroll
    for (int sidx = 0; sidx < LOOK; ++sidx) {
      if (it.done) break;
      const Chunk ck = it.chunk();
      Dma::issue(p.tiles, ck.slot, stage(sidx), wave, dma_voff);
      const int sv = seen(ck);
      if (sidx == 0) v0 = sv;
      else if (sidx == 1) v1 = sv;
      else v2 = sv;
      ++ready;
      it.template advance<DENSE>(p.g, bh, p.cpb);
    }
    // Q and the first chunks were issued together: wait for all of them
    wait_vmem<0>();
    barrier_lds();

    // The pipeline runs on 32-key halves of the chunks (the online softmax
    // is exact at any key granularity).  A half issues, in this order:
    //   A: Q K^T steps 0..DT-1 of the next half (a dependent MFMA chain), with
    //      the probabilities of the current half's first 16 keys;
    //   B: P V of those 16 keys (one MFMA per d tile) alternating with Q K^T
    //      steps DT..2DT-1, with the probabilities of the other 16 keys;
    //   C: P V of the other 16 keys, with the statistics of the next half.
    // Independent P V MFMAs cover the latency of the Q K^T chain, and the
    // vector work is spread over the whole half rather than packed into the
    // Q K^T chain.  sA and sB hold S^T of a half for each sub-tile and trade
    // roles every half, so nothing is copied.
    constexpr int NOPS = 4 * DT;  // LDS operands per half: 2DT of K, 2DT of V^T
    constexpr int AHEAD = 4;      // operands in flight (a ring in consumption order)
    constexpr int EPS = 8 / DT;   // probabilities per sub-tile per step of A or B
    static_assert(NOPS % AHEAD == 0 && EPS % 2 == 0, "operand ring and probability pairs");
    f32x16 sA[QT], sB[QT];
    // operand bases of key half kt of a chunk image: its K rows, its V^T columns
    auto kbase = [](const bf16_bits* img, int kt) -> const bf16_bits* { return img + Lds<D>::k_off(32 * kt, 0); };
    auto vbase = [](const bf16_bits* img, int kt) -> const bf16_bits* {
      return img + (Lds<D>::v_off(0, 32 * kt) - Lds<D>::VBASE);
    };
    auto kread = [&](const bf16_bits* kb, int ds) -> bf16x8 {
      return *(const bf16x8*)(kb + Lds<D>::k_off(lr, 16 * ds + 8 * hi));
    };
    auto vread = [&](const bf16_bits* vb, int kg, int t) -> bf16x8 {
      return *(const bf16x8*)(vb + Lds<D>::v_off(32 * t + lr, 16 * kg + 8 * hi));
    };
    // operand i of a half: a K d-step (isk, a = d-step) or a V^T tile (a = key
    // group, t = d tile), in the order the MFMAs of A, B and C consume them
    struct HalfOp {
      bool isk;
      int a, t;
    };
    auto half_op = [](int i) -> HalfOp {
      if (i < DT) return {true, i, 0};
      if (i < 3 * DT) {
        const int j = i - DT;
        return (j & 1) ? HalfOp{true, DT + j / 2, 0} : HalfOp{false, 0, j / 2};
      }
      return {false, 1, i - 3 * DT};
    };

    // Row statistics of a freshly computed S^T half: the tail mask (keys past
    // the chunk's real count become -inf), the row max of the offset scores
    // and whether some row's running max must move.  Split into STAT_STEPS steps
    // so they sit between the P V MFMAs of the half before the one that uses
    // them, off the critical path.
    constexpr int STAT_STEPS = 7;
    float mxc[QT];    // this lane's max over its 16 keys of the half to be exponentiated next
    float mpart[QT];  // partial lane max
    bool rc = false;  // some row of that half needs its running max raised
    auto stat_step = [&](int step, f32x16 (&sx)[QT], int valid, int kt) __attribute__((always_inline)) {
      if (step == 0) {
        // lane holds keys 32kt + 8(r/4) + 4hi + r%4 of query lr of each sub-tile
        if (valid < 32 * kt + 32) {
          const int lim = valid - 32 * kt - 4 * hi;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (8 * (r >> 2) + (r & 3) >= lim) sx[qt][r] = -INFINITY;
        }
      } else if (step <= 4) {
        // two 3-input maxima per 4 keys
        const int r0 = 4 * (step - 1);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float m = step == 1 ? fmaxf(fmaxf(sx[qt][0], sx[qt][1]), sx[qt][2])
                                    : fmaxf(fmaxf(mpart[qt], sx[qt][r0]), sx[qt][r0 + 1]);
          mpart[qt] = step == 1 ? fmaxf(m, sx[qt][3]) : fmaxf(fmaxf(m, sx[qt][r0 + 2]), sx[qt][r0 + 3]);
          if (step == 4) mxc[qt] = mpart[qt];
        }
      } else if (step == 6) {
        // a row's two lanes share its threshold, so the lane maxima decide
        // whether some row must move without combining the lane pair (the
        // raise itself takes the row max)
        bool r = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) r = r || (mxc[qt] > thr[qt]);
        rc = __any(r);
      }
    };

    // S^T of one key half (K rows from kb; key half kt of a chunk with
    // `valid` real keys for this wavefront) and its statistics, unpipelined
    auto qk_only = [&](f32x16 (&sx)[QT], const bf16_bits* kb, int kt, int valid) __attribute__((always_inline)) {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 a = kread(kb, ds);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sx[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qt][ds], ds == 0 ? negm[qt] : sx[qt], 0, 0, 0);
      }
#pragma unroll
      for (int step = 0; step < STAT_STEPS; ++step) stat_step(step, sx, valid, kt);
    };
    const int kt0 = ksel < 0 ? 0 : ksel;  // first key half this wavefront computes
    if (wave_active && ready > 0) qk_only(sA, kbase(ring0, kt0), kt0, v0);
    // the first AHEAD operands of a half: from its V^T (vc) and the K of the
    // next half (kn)
    bf16x8 opw[AHEAD];
    auto preload = [&](const bf16_bits* vc, const bf16_bits* kn) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < AHEAD; ++i) {
        const HalfOp o = half_op(i);
        opw[i] = o.isk ? kread(kn, o.a) : vread(vc, o.a, o.t);
      }
    };
    // every wavefront's first half is key half kt0 of chunk 0; a wavefront
    // that takes both halves computes key half 1 of chunk 0 in it, one that
    // takes a single half computes its half of chunk 1 (its operands are
    // loaded before each of its halves)
    if (ksel < 0) preload(vbase(ring0, 0), kbase(ring0, 1));

    // One half: the 32 keys whose V^T starts at vc, S^T (masked, statistics
    // in mxc / rc) in sc.  S^T of the next half (K rows from kn; key half
    // kt_nxt of a chunk with valid_nxt real keys) goes to sn and its
    // statistics are taken in C.  The operand ring runs AHEAD operands into
    // the half after (its V^T from vn, its K from knn).
    constexpr int STAT_C0 = 1;  // first step of C followed by statistics (the Q K^T result has landed)
    constexpr int STAT_PER = (STAT_STEPS + DT - STAT_C0 - 1) / (DT - STAT_C0);
    auto half = [&](f32x16 (&sc)[QT], f32x16 (&sn)[QT], const bf16_bits* vc, const bf16_bits* kn, int kt_nxt,
                    int valid_nxt, const bf16_bits* vn, const bf16_bits* knn) __attribute__((always_inline)) {
      if (rc) {
        // raise: the new max (absolute) of a row is its old one or this
        // half's; scores of this half move to the new offset, and a row that
        // has still seen no real key keeps offset 0
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float m_new = fmaxf(m_run[qt], moff[qt] + max_halves(mxc[qt]));
          const float o_new = m_new > 0.5f * M_NONE ? m_new : 0.f;
          const float shift = o_new - moff[qt];
          const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
          thr[qt] = m_new - o_new + RAISE_SLACK;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sc[qt][r] -= shift;
            negm[qt][r] = -o_new;
          }
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qt][t][r] *= alpha;
          lsum[qt] *= alpha;
          m_run[qt] = m_new;
          moff[qt] = o_new;
        }
      }

      // consume operand i from the ring and read operand i + AHEAD into its slot
      auto refill = [&](int i) __attribute__((always_inline)) {
        const int j = i + AHEAD;
        const HalfOp o = half_op(j % NOPS);
        if (j < NOPS) opw[i % AHEAD] = o.isk ? kread(kn, o.a) : vread(vc, o.a, o.t);
        else opw[i % AHEAD] = o.isk ? kread(knn, o.a) : vread(vn, o.a, o.t);
      };
      const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
      u32x4 pw[2][QT];  // bf16 probability pairs: B operands of the P V MFMAs
      // probabilities r0 .. r0+EPS-1 of every sub-tile, rounded to bf16 in
      // pairs; the row sum adds the same rounded values the MFMA uses
      auto probs = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int u = 0; u < EPS; u += 2) {
            const int r = r0 + u;
            const float e0 = __builtin_amdgcn_exp2f(sc[qt][r]);
            const float e1 = __builtin_amdgcn_exp2f(sc[qt][r + 1]);
            const bf16x2_t pr = {(__bf16)e0, (__bf16)e1};
            pw[r >> 3][qt][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pr);
            lsum[qt] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsum[qt], false);
          }
      };
      auto pv = [&](int i, int kg, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc[qt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opw[i % AHEAD], __builtin_bit_cast(bf16x8, pw[kg][qt]),
                                                              acc[qt][t], 0, 0, 0);
        refill(i);
      };
      auto qk = [&](int i, int ds) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          sn[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opw[i % AHEAD], qf[qt][ds], ds == 0 ? negm[qt] : sn[qt], 0, 0,
                                                           0);
        }
        refill(i);
      };

      // ---- program order is kept by sched_barrier fences
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < DT; ++j) {  // A
        qk(j, j);
        probs(EPS * j);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < DT; ++j) {  // B
        pv(DT + 2 * j, 0, j);
        qk(DT + 2 * j + 1, DT + j);
        probs(8 + EPS * j);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Every probability of the half exists here: otherwise the compiler
      // sinks the second key group's exponentials past the tail-mask branch
      // in C, out of the MFMA gaps they are meant to fill.
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) asm volatile("" : : "v"(pw[0][qt]), "v"(pw[1][qt]), "v"(lsum[qt]));
#pragma unroll
      for (int j = 0; j < DT; ++j) {  // C
        pv(3 * DT + j, 1, j);
        if (j >= STAT_C0) {
#pragma unroll
          for (int k = (j - STAT_C0) * STAT_PER; k < (j - STAT_C0 + 1) * STAT_PER && k < STAT_STEPS; ++k)
            stat_step(k, sn, valid_nxt, kt_nxt);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // One chunk c (stage s0): the load of chunk c+LOOK is issued, the two
    // halves of c run (the second also reads K of chunk c+1), then every
    // wavefront waits until chunk c+2 has landed and the workgroup meets at
    // the barrier.  s0 is a compile-time constant
    // in each of the four unrolled copies below.
    //
    // A wavefront on one key half (ksel) runs key half ksel of chunk c and
    // (Q K^T) the same half of chunk c+1, in the first half slot of even
    // chunks and the second slot of odd ones, so that its S^T alternates
    // between sA and sB like everyone else's; its operand ring is reloaded
    // before each of its halves (what the slot before read ahead is not its
    // own).
    //
    // Grouped items: a wavefront whose own query block did not keep chunk c
    // skips both halves of c; if its block keeps chunk c+1 it computes only
    // the S^T of key half 0 of c+1 (the one result of c's second half it
    // needs), and it reloads its operand ring before its next half.
    const bool sp = !DENSE && !GRP && ksel >= 0;
    bool reload = false;
    auto chunk_step = [&](int s0) __attribute__((always_inline)) -> bool {
      const int s1 = (s0 + 1) % STAGES;
      const int sl = (s0 + LOOK) % STAGES;
      const bool more = !it.done;
      Chunk ckl = {0, 0, -1};
      if (more) {
        ckl = it.chunk();
        Dma::issue(p.tiles, ckl.slot, stage(sl), wave, dma_voff);
      }
      const bf16_bits* S0 = stage(s0);
      const bf16_bits* S1 = stage(s1);
      const bool even = (s0 & 1) == 0;
      // a one-half wavefront's half: V^T of (c, ksel), K of (c+1, ksel)
      const bf16_bits* vs = vbase(S0, sp ? ksel : 0);
      const bf16_bits* ks = kbase(S1, sp ? ksel : 0);
      const bool skip = GRP && v0 == 0;
      if (GRP && wave_active && skip) {
        if (v1 > 0) qk_only(sA, kbase(S1, 0), 0, v1);
        reload = true;
      }
      if (GRP && wave_active && !skip && reload) {
        preload(vbase(S0, 0), kbase(S0, 1));
        reload = false;
      }
      // first slot, two-half wavefronts: key half 0 of c; Q K^T of half 1 of c
      if (wave_active && !skip && (!sp || even)) {
        if (sp) preload(vs, ks);
        half(sA, sB, sp ? vs : vbase(S0, 0), sp ? ks : kbase(S0, 1), sp ? ksel : 1, sp ? v1 : v0, vbase(S0, 1),
             kbase(S1, 0));
      }
      // second slot, two-half wavefronts: key half 1 of c; Q K^T of half 0 of c+1
      if (wave_active && !skip && (!sp || !even)) {
        if (sp) preload(vs, ks);
        half(sB, sA, sp ? vs : vbase(S0, 1), sp ? ks : kbase(S1, 0), sp ? ksel : 0, v1, vbase(S1, 0),
             kbase(S1, 1));
      }
      if (more) {
        ++ready;
        it.template advance<DENSE>(p.g, bh, p.cpb);
      }
      if (more) wait_vmem<Dma::PER_WAVE>();
      else wait_vmem<0>();
      barrier_lds();
      --ready;
      const int sv = more ? seen(ckl) : 0;
      v0 = v1;
      v1 = v2;
      v2 = sv;
      return ready > 0;
    };
    while (ready > 0) {
      if (!chunk_step(0)) break;
      if (!chunk_step(1)) break;
      if (!chunk_step(2)) break;
      if (!chunk_step(3)) break;
    }

    // ---- the next item: pop it, publish its id and stage its mask rows
    //      (every wavefront is done with this item's masks) while this
    //      item's output is written; the barrier that ends the item orders
    //      both before the next item's first read
    if (!DENSE) {
      if (tid == 0) item_s = item_of_slot(take_own_slot());
      __syncthreads();
      if (item_s >= 0) stage_mask(item_s);
    }

    // ---- split tiles: the key-half-1 wavefront hands its running max, partial
    //      row sums and O^T accumulators to the key-half-0 wavefront through
    //      LDS (the ring is idle: every chunk load has landed), which rescales
    //      both to the larger max and adds them.  A side that saw no real key
    //      has the floor max and zero sums, so it contributes nothing.
    if (!DENSE && !GRP && QT == 1 && merge) {
      float* xch = (float*)stage((row0 >> 5) & 3);
      f32x4* xv = (f32x4*)xch;
      if (wave_active && ksel == 1) {
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[0][t][4 * g + e];
            xv[(t * 4 + g) * 64 + lane] = x;
          }
        xch[DT * 16 * 64 + lane] = m_run[0];
        xch[DT * 16 * 64 + 64 + lane] = lsum[0];
      }
      __syncthreads();
      if (wave_active && ksel == 0) {
        const float mb = xch[DT * 16 * 64 + lane];
        const float lb = xch[DT * 16 * 64 + 64 + lane];
        const float m = fmaxf(m_run[0], mb);
        const float ea = __builtin_amdgcn_exp2f(m_run[0] - m);
        const float eb = __builtin_amdgcn_exp2f(mb - m);
        lsum[0] = lsum[0] * ea + lb * eb;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 x = xv[(t * 4 + g) * 64 + lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[0][t][4 * g + e] = acc[0][t][4 * g + e] * ea + x[e] * eb;
          }
      }
    }

    // ---- normalise and store the real rows (lane and lane ^ 32 share a row)
    if (wave_active && ksel != 1) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float lt = sum_halves(lsum[qt]);
        const int qrow = row0 + 32 * qt + lr;
        if (qrow < qcount) {
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          const int64_t otok = pos_to_token<DENSE>(p, qbase + qrow);
          bf16_bits* dst = p.o + head_off + otok * rs;
#pragma unroll
          for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
              bf16x4_t w;
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[qt][t][4 * g4 + e] * inv);
              *(bf16x4_t*)(dst + 32 * t + 8 * g4 + 4 * hi) = w;
            }
        }
      }
    }
    const uint64_t t_end = wall_ticks();
    if (nitems == 0) t_first = t_start;
    t_last = t_end;
    busy += t_end - t_start;
    ++nitems;
    // the next item depends on this one only through LDS (its mask rows and
    // id, the ring); the output stores stay in flight and are waited for
    // with the next item's first loads
    barrier_lds();
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
// Per-call preparation kernels
// ---------------------------------------------------------------------------

// Block-ordered token table and real counts: one workgroup per block.
__global__ __launch_bounds__(256) void layout_kernel(Geo g, int32_t* __restrict__ tok, int32_t* __restrict__ cnt,
                                                     uint64_t* __restrict__ head_cost, int BH) {
  const int n = blockIdx.x;
  if (n == 0)
    for (int x = threadIdx.x; x < BH; x += blockDim.x) head_cost[x] = 0;  // summed by cost_kernel
  const Box bx = block_box(g, n);
  if (threadIdx.x == 0) cnt[n] = bx.count;
  const int plane = bx.eh * bx.ew;
  for (int r = threadIdx.x; r < bx.count; r += blockDim.x) {
    const int dt = r / plane, rem = r % plane;
    const int dy = rem / bx.ew, dx = rem % bx.ew;
    tok[bx.start + r] = ((bx.t0 + dt) * g.H + (bx.y0 + dy)) * g.W + bx.x0 + dx;
  }
}

// Chunk images of K and V in the LDS layout: one workgroup per (b, h,
// block, chunk) slot.  Rows past the block's real count are zero.  K and V
// rows are read as whole token rows (16 lanes per 256-byte row), staged in
// LDS row-major (rows padded by 16 bytes, so the column reads below hit
// distinct banks), and written out piece-major, each thread storing the next
// 16 bytes of the image.  tok = null: the tokens are in their natural order
// (the dense reference's single block of L tokens).
template <int D>
__global__ __launch_bounds__(256) void tile_kernel(const bf16_bits* __restrict__ k, const bf16_bits* __restrict__ v,
                                                   const int32_t* __restrict__ tok, Geo g, int L, Heads hd, int cpb,
                                                   bf16_bits* __restrict__ tiles) {
  __shared__ __attribute__((aligned(16))) bf16_bits ks[KCH][D + 8];
  __shared__ __attribute__((aligned(16))) bf16_bits vs[KCH][D + 8];
  const int cs = blockIdx.x;
  const int c = cs % cpb;
  const int n = (cs / cpb) % g.N;
  const int bh = cs / (cpb * g.N);
  const int h = bh % hd.n, b = bh / hd.n;
  const Box bx = block_box(g, n);
  const int valid = bx.count - c * KCH;
  if (valid <= 0) return;  // slot past the block's chunks: never read
  const int64_t rs = (int64_t)hd.stride * D;
  const int64_t head_off = (int64_t)b * L * rs + (int64_t)(hd.h0 + h) * D;
  constexpr int PIECES = KCH * D / 8;  // 16-byte pieces of K (and of V)
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s = threadIdx.x; s < PIECES; s += 256) {
    const int row = s / (D / 8), piece = s % (D / 8);
    u32x4 kx = zero, vx = zero;
    if (row < valid) {
      const int pos = bx.start + c * KCH + row;
      const int64_t t = tok ? tok[pos] : pos;
      kx = *(const u32x4*)(k + head_off + t * rs + piece * 8);
      vx = *(const u32x4*)(v + head_off + t * rs + piece * 8);
    }
    *(u32x4*)&ks[row][piece * 8] = kx;
    *(u32x4*)&vs[row][piece * 8] = vx;
  }
  __syncthreads();
  bf16_bits* dst = tiles + (int64_t)cs * Lds<D>::ELEMS;
  for (int s = threadIdx.x; s < PIECES; s += 256) {  // K piece s//64 of row s%64
    const int piece = s / KCH, row = s % KCH;
    *(u32x4*)(dst + Lds<D>::k_off(row, piece * 8)) = *(const u32x4*)&ks[row][piece * 8];
  }
  for (int s = threadIdx.x; s < D * 8; s += 256) {  // V^T piece s//D (positions 8p..8p+7) of row d = s%D
    const int piece = s / D, d = s % D;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = pi_key(piece * 8 + 2 * e), k1 = pi_key(piece * 8 + 2 * e + 1);
      w[e] = (uint32_t)vs[k0][d] | ((uint32_t)vs[k1][d] << 16);
    }
    const u32x4 x = {w[0], w[1], w[2], w[3]};
    *(u32x4*)(dst + Lds<D>::v_off(d, piece * 8)) = x;
  }
}

// Work of every item (query rows x real key tokens of the union of its
// members' kept blocks: the time the item takes), its LPT sort key, and the
// reset of the queue counters.  cost < 2^32: an item holds at most 256 query
// rows and L < 2^24.  key = cost << 32 | ~item: descending keys give
// descending cost, ties to the lower item id.  One wavefront per item, its
// lanes over the mask words; the block counts are staged in LDS (N <= 8192).
constexpr int COST_WAVES = 8;
__global__ __launch_bounds__(COST_WAVES * 64) void cost_kernel(AttnParams p, const int32_t* __restrict__ cnt,
                                                               uint64_t* __restrict__ keys, uint32_t* __restrict__ rank,
                                                               uint32_t* __restrict__ qctr,
                                                               uint64_t* __restrict__ head_cost,
                                                               uint64_t* __restrict__ tag) {
  extern __shared__ int32_t cnt_s[];  // [N]
  for (int j = threadIdx.x; j < p.g.N; j += COST_WAVES * 64) cnt_s[j] = cnt[j];
  if (blockIdx.x == 0 && threadIdx.x < NXCD) qctr[threadIdx.x] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) *tag = p.want_tag;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * COST_WAVES + wave;
  // each wavefront's cost and head, summed per head by wavefront 0 below
  __shared__ uint64_t wave_cost[COST_WAVES];
  __shared__ int wave_bh[COST_WAVES];
  if (item >= p.n_items) {
    if (lane == 0) wave_bh[wave] = -1;
    __syncthreads();
    return;
  }
  const int gid = item % p.n_groups, bh = item / p.n_groups;
  const uint32_t* rows[4];
  int nrows = 0;
  uint32_t qrows = 0;
  for (int k = 0; k < p.gt * p.gh * p.gw; ++k) {
    const int n = group_member(p, gid, k);
    if (n < 0) continue;
    rows[nrows++] = p.mask + (p.hd.global(bh) * p.g.N + n) * p.words;
    qrows += (uint32_t)cnt_s[n];
  }
  uint32_t kv = 0;
  for (int w = lane; w < p.words; w += 64) {
    uint32_t bits = 0u;
    for (int r = 0; r < nrows; ++r) bits |= rows[r][w];
    const int rem = p.g.N - w * 32;
    if (rem < 32) bits &= (1u << rem) - 1u;
    while (bits) {
      kv += (uint32_t)cnt_s[w * 32 + __builtin_ctz(bits)];
      bits &= bits - 1u;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kv += (uint32_t)__shfl_xor((int)kv, off);  // integer sum: any order
  if (lane == 0) {
    const uint32_t cost = qrows * kv;
    keys[item] = ((uint64_t)cost << 32) | (uint64_t)(~(uint32_t)item);
    rank[item] = 0u;
    wave_cost[wave] = cost;
    wave_bh[wave] = bh;
  }
  __syncthreads();
  // one atomic per run of wavefronts on the same head (a head's items are
  // consecutive): many wavefronts adding to one address serialise in L2
  if (threadIdx.x == 0) {
    uint64_t run = 0;
    int run_bh = -1;
    for (int w = 0; w < COST_WAVES; ++w) {
      const int b = wave_bh[w];
      if (b != run_bh) {
        if (run_bh >= 0) atomicAdd((unsigned long long*)&head_cost[run_bh], (unsigned long long)run);
        run = 0;
        run_bh = b;
      }
      if (b >= 0) run += wave_cost[w];
    }
    if (run_bh >= 0) atomicAdd((unsigned long long*)&head_cost[run_bh], (unsigned long long)run);
  }
}

// Heads to XCDs, longest first (single workgroup).  Head cost = sum of its
// items' costs (summed by cost_kernel); heads are taken in descending cost
// (ties: lower head) and each goes to the XCD with the least assigned cost
// (ties: lower XCD).  Writes each head's first position in the order array
// and the queue segments qoff[0..NXCD].  NAIVE puts every head on queue 0 in
// head order.  forced (nullable): each head's XCD, given by the caller
// instead of chosen.  The assignment is sequential (each choice depends on
// the loads before it) and runs on wavefront 0: lane x (mod 8) holds XCD x's
// load and head count, and the least loaded XCD comes from three register
// exchanges of the key load << 3 | x inside each group of 8 lanes; the
// ranking before it and the positions after it are spread over the workgroup.
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)x, (int)(uint32_t)x, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(x >> 32), (int)(x >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__global__ __launch_bounds__(256) void head_plan_kernel(const uint64_t* __restrict__ head_cost, int N, int BH,
                                                        bool lpt, const int32_t* __restrict__ forced,
                                                        int32_t* __restrict__ head_pos, int32_t* __restrict__ qoff) {
  // [BH] head costs, [BH] costs in rank order, then [BH] int32 head of each
  // rank, then [BH] int32 place of each rank (XCD | slot among the XCD's heads << 3)
  extern __shared__ uint64_t hsh[];
  __shared__ int32_t qoff_s[NXCD + 1];
  uint64_t* hcost = hsh;
  uint64_t* rcost = hsh + BH;
  int32_t* horder = (int32_t*)(hsh + 2 * BH);
  int32_t* place = horder + BH;
  for (int x = threadIdx.x; x < BH; x += blockDim.x) hcost[x] = lpt ? head_cost[x] : 0;
  __syncthreads();
  for (int x = threadIdx.x; x < BH; x += blockDim.x) {
    int r = 0;
    for (int y = 0; y < BH; ++y)
      if (hcost[y] > hcost[x] || (hcost[y] == hcost[x] && y < x)) ++r;
    horder[r] = x;
    rcost[r] = hcost[x];
    place[r] = forced ? min(max(forced[x], 0), NXCD - 1) : 0;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, xl = lane & (NXCD - 1);
    uint64_t ld = 0;
    int cnt = 0;
    for (int r = 0; r < BH; ++r) {
      const uint64_t c = rcost[r];
      int best;
      if (!forced && lpt) {
        uint64_t key = (ld << 3) | (uint64_t)xl;
        uint64_t o = dpp_u64<0xB1>(key);  // lane ^ 1
        key = o < key ? o : key;
        o = dpp_u64<0x4E>(key);           // lane ^ 2
        key = o < key ? o : key;
        o = dpp_u64<0x141>(key);          // 7 - lane, within 8
        key = o < key ? o : key;
        best = __builtin_amdgcn_readfirstlane((int)(key & 7));
      } else {
        best = __builtin_amdgcn_readfirstlane(place[r]);
      }
      const int slot = __builtin_amdgcn_readlane(cnt, best);
      if (lane == 0) place[r] = best | (slot << 3);
      if (xl == best) {
        ld += c;
        ++cnt;
      }
    }
    // queue segments: XCD x starts after the heads of XCDs 0 .. x-1
    int off = cnt * N;  // inclusive prefix over lanes 0..7 of each group
#pragma unroll
    for (int d = 1; d < NXCD; d <<= 1) {
      const int o = __shfl_up(off, d);
      if (xl >= d) off += o;
    }
    if (lane < NXCD) {
      qoff[lane] = off - cnt * N;
      qoff_s[lane] = off - cnt * N;
      if (lane == NXCD - 1) qoff[NXCD] = off;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < BH; r += blockDim.x)
    head_pos[horder[r]] = qoff_s[place[r] & 7] + (place[r] >> 3) * N;
}

// rank[a] += #{b in this tile of a's head : key[b] > key[a]}  (keys distinct).
// grid = (ceil(G / 256), ceil(G / 2048), heads): item tiles of one head only.
__global__ __launch_bounds__(256) void rank_kernel(const uint64_t* __restrict__ keys, int G,
                                                   uint32_t* __restrict__ rank) {
  __shared__ uint64_t tile[2048];
  const uint64_t* hk = keys + (int64_t)blockIdx.z * G;
  const int a = blockIdx.x * 256 + threadIdx.x;
  const int b0 = blockIdx.y * 2048;
  const int nb = min(2048, G - b0);
  for (int t = threadIdx.x; t < nb; t += 256) tile[t] = hk[b0 + t];
  __syncthreads();
  if (a >= G) return;
  const uint64_t ka = hk[a];
  uint32_t c = 0;
  for (int t = 0; t < nb; ++t) c += tile[t] > ka ? 1u : 0u;
  if (c) atomicAdd(&rank[(int64_t)blockIdx.z * G + a], c);
}

// The pop counters of the queues start at zero in every launch of the
// persistent kernel, so that one plan serves any number of execs.
__global__ __launch_bounds__(64) void queue_reset_kernel(uint32_t* __restrict__ qctr) {
  if (threadIdx.x < NXCD) qctr[threadIdx.x] = 0u;
}

__global__ __launch_bounds__(256) void scatter_kernel(const uint32_t* __restrict__ rank,
                                                      const int32_t* __restrict__ head_pos, int n_items, int N,
                                                      bool lpt, int32_t* __restrict__ order) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a >= n_items) return;
  const int within = lpt ? (int)rank[a] : a % N;
  order[head_pos[a / N] + within] = a;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
// Work item shape per block volume.  Every item is 8 wavefronts x 32 query
// rows; small blocks are grouped so an item still fills them:
//   volume <= 64:  2x1x2 blocks (t, y, x) per item, 2 wavefronts per block
//   volume <= 128: 1x1x2 blocks per item, 4 wavefronts per block
//   otherwise:     one block per item
// A group walks the union of its blocks' kept key blocks; each wavefront
// masks the key blocks its own query block did not keep.
constexpr int WAVES = 8;
struct GroupShape {
  int gt, gh, gw, wpb;
};
static GroupShape group_shape(int vol) {
  if (vol <= 64) return {2, 1, 2, 2};
  if (vol <= 128) return {1, 1, 2, 4};
  return {1, 1, 1, 8};
}

int attn_chunks_per_block(int vol) { return (vol + KCH - 1) / KCH; }

int attn_items_per_head(const Geo& g) {
  const GroupShape gs = group_shape(g.bt * g.bh * g.bw);
  return ((g.nT + gs.gt - 1) / gs.gt) * ((g.nH + gs.gh - 1) / gs.gh) * ((g.nW + gs.gw - 1) / gs.gw);
}

__global__ __launch_bounds__(256) void item_cost_kernel(const uint64_t* __restrict__ keys, int64_t n,
                                                        uint32_t* __restrict__ cost) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) cost[i] = (uint32_t)(keys[i] >> 32);
}

hipError_t launch_item_costs(const uint64_t* keys, int64_t n, uint32_t* cost, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(item_cost_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, keys, n, cost);
  return hipGetLastError();
}

size_t attn_tile_bytes(int D, int64_t slots) {
  return (size_t)slots * (D == 128 ? Lds<128>::ELEMS : Lds<64>::ELEMS) * sizeof(bf16_bits);
}

static const void* sparse_kernel(int D, bool grouped) {
  if (D == 128)
    return grouped ? reinterpret_cast<const void*>(&attn_kernel<128, WAVES, 1, false, true>)
                   : reinterpret_cast<const void*>(&attn_kernel<128, WAVES, 1, false, false>);
  return grouped ? reinterpret_cast<const void*>(&attn_kernel<64, WAVES, 1, false, true>)
                 : reinterpret_cast<const void*>(&attn_kernel<64, WAVES, 1, false, false>);
}

// Dynamic LDS of the sparse kernel: mask words of the item's union (and of
// its 4 members for groups), then the real token count of every block.
static size_t sparse_lds_bytes(int N, bool grouped) {
  const size_t words = (size_t)(N + 31) / 32;
  return ((grouped ? 5 : 1) * words * 4 + (size_t)N * 2 + 15) / 16 * 16;
}

int attn_persistent_workgroups(int D, int block_volume, int* err) {
  int dev = 0, cus = 0, occ = 0;
  *err = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, sparse_kernel(D, group_shape(block_volume).wpb < WAVES),
                                                   WAVES * 64, 0) != hipSuccess) {
    *err = 1;
    return 0;
  }
  if (occ < 1) occ = 1;
  return cus * occ;
}

// The tag a plan leaves in its workspace: a hash of the tensor shape and the
// token and block grid (never 0, the value of cleared memory).
uint64_t plan_tag_of(int B, int L, int heads, int D, const Geo& g) {
  const int64_t f[10] = {B, L, heads, D, g.T, g.H, g.W, g.bt, g.bh, g.bw};
  uint64_t h = 0xcbf29ce484222325ull;  // FNV-1a, 64 bit
  for (int64_t x : f)
    for (int b = 0; b < 8; ++b) h = (h ^ (uint64_t)((x >> (8 * b)) & 0xff)) * 0x100000001b3ull;
  return h | 1ull;
}

static AttnParams sparse_params(const AttnLaunch& a) {
  const int vol = a.g.bt * a.g.bh * a.g.bw;
  const GroupShape gs = group_shape(vol);
  AttnParams prm = {};
  prm.q = (const bf16_bits*)a.q;
  prm.k = (const bf16_bits*)a.k;
  prm.v = (const bf16_bits*)a.v;
  prm.o = (bf16_bits*)a.o;
  prm.B = a.B;
  prm.L = a.L;
  prm.heads = a.heads;
  prm.hd = a.hd;
  prm.g = a.g;
  prm.words = (a.g.N + 31) / 32;
  prm.cpb = attn_chunks_per_block(vol);
  prm.mask = a.mask;
  prm.tok = a.tok;
  prm.cnt = a.blk_cnt;
  prm.tiles = a.tiles;
  prm.order = a.order;
  prm.qoff = a.qoff;
  prm.qctr = a.qctr;
  prm.gt = gs.gt;
  prm.gh = gs.gh;
  prm.gw = gs.gw;
  prm.wpb = gs.wpb;
  prm.gT = (a.g.nT + gs.gt - 1) / gs.gt;
  prm.gH = (a.g.nH + gs.gh - 1) / gs.gh;
  prm.gW = (a.g.nW + gs.gw - 1) / gs.gw;
  prm.n_groups = prm.gT * prm.gH * prm.gW;
  prm.n_items = a.B * a.heads * prm.n_groups;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  prm.trace = a.trace;
  prm.plan_tag = a.plan_tag;
  prm.want_tag = plan_tag_of(a.B, a.L, a.heads, a.D, a.g);
  return prm;
}

hipError_t launch_sparse_plan(const AttnLaunch& a, int sched, const int32_t* head_xcd, hipStream_t st) {
  const bool lpt = sched != 1;  // LPT order within heads for both the stealing and the per-XCD schedules
  const AttnParams prm = sparse_params(a);
  const int BH = a.B * a.heads;
  const int n_items = prm.n_items, per_head = prm.n_groups, cpb = prm.cpb;
  hipLaunchKernelGGL(layout_kernel, dim3(a.g.N), dim3(256), 0, st, a.g, a.tok, a.blk_cnt, a.head_cost, BH);
  const unsigned slots = (unsigned)(BH * a.g.N * cpb);
  if (a.D == 128)
    hipLaunchKernelGGL(tile_kernel<128>, dim3(slots), dim3(256), 0, st, (const bf16_bits*)a.k, (const bf16_bits*)a.v,
                       a.tok, a.g, a.L, a.hd, cpb, a.tiles);
  else
    hipLaunchKernelGGL(tile_kernel<64>, dim3(slots), dim3(256), 0, st, (const bf16_bits*)a.k, (const bf16_bits*)a.v,
                       a.tok, a.g, a.L, a.hd, cpb, a.tiles);
  hipLaunchKernelGGL(cost_kernel, dim3((n_items + COST_WAVES - 1) / COST_WAVES), dim3(COST_WAVES * 64),
                     (size_t)a.g.N * sizeof(int32_t), st, prm, a.blk_cnt, a.keys, a.rank, a.qctr, a.head_cost,
                     a.plan_tag);
  hipLaunchKernelGGL(head_plan_kernel, dim3(1), dim3(256), (size_t)BH * 24, st, a.head_cost, per_head, BH, lpt,
                     sched == 2 ? head_xcd : nullptr, a.head_pos, a.qoff);
  if (lpt)
    hipLaunchKernelGGL(rank_kernel, dim3((per_head + 255) / 256, (per_head + 2047) / 2048, BH), dim3(256), 0, st,
                       a.keys, per_head, a.rank);
  hipLaunchKernelGGL(scatter_kernel, dim3((n_items + 255) / 256), dim3(256), 0, st, a.rank, a.head_pos, n_items,
                     per_head, lpt, a.order);
  return hipGetLastError();
}

hipError_t launch_sparse_exec(const AttnLaunch& a, int sched, hipStream_t st) {
  AttnParams prm = sparse_params(a);
  prm.steal = sched != 2;
  const int vol = a.g.bt * a.g.bh * a.g.bw;
  int err = 0;
  const int grid = attn_persistent_workgroups(a.D, vol, &err);
  if (err) return hipErrorInvalidValue;
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, st, a.qctr);
  void* args[] = {&prm};
  const bool grouped = group_shape(vol).wpb < WAVES;
  return hipLaunchKernel(sparse_kernel(a.D, grouped), dim3(grid), dim3(WAVES * 64), args,
                         sparse_lds_bytes(a.g.N, grouped), st);
}

// The dense reference: the whole sequence as one block of L tokens, tiled in
// natural order (chunk c = tokens 64c .. 64c+63), and query tiles of 256
// consecutive tokens as work items (one workgroup each, consecutive tiles on
// one XCD), streamed through the same chunk pipeline as the sparse path.
static Geo dense_geo(int L) { return Geo{L, 1, 1, L, 1, 1, 1, 1, 1, 1}; }

size_t dense_tile_bytes(int B, int L, int heads, int D) {
  return attn_tile_bytes(D, (int64_t)B * heads * ((L + KCH - 1) / KCH));
}

hipError_t launch_dense_attn(const void* q, const void* k, const void* v, void* o, int B, int L, int heads, int D,
                             float scale, void* tiles, hipStream_t st) {
  constexpr int QT = 1;
  AttnParams prm = {};
  prm.q = (const bf16_bits*)q;
  prm.k = (const bf16_bits*)k;
  prm.v = (const bf16_bits*)v;
  prm.o = (bf16_bits*)o;
  prm.B = B;
  prm.L = L;
  prm.heads = heads;
  prm.hd = Heads{heads, 0, heads};
  prm.g = dense_geo(L);
  prm.cpb = (L + KCH - 1) / KCH;
  prm.tiles = (const bf16_bits*)tiles;
  prm.q_tiles = (L + WAVES * QT * 32 - 1) / (WAVES * QT * 32);
  prm.n_items = B * heads * prm.q_tiles;
  prm.scale_log2 = scale * 1.4426950408889634f;
  prm.trace = nullptr;
  const unsigned slots = (unsigned)(B * heads * prm.cpb);
  if (D == 128)
    hipLaunchKernelGGL(tile_kernel<128>, dim3(slots), dim3(256), 0, st, prm.k, prm.v, nullptr, prm.g, L, prm.hd,
                       prm.cpb, (bf16_bits*)tiles);
  else
    hipLaunchKernelGGL(tile_kernel<64>, dim3(slots), dim3(256), 0, st, prm.k, prm.v, nullptr, prm.g, L, prm.hd, prm.cpb,
                       (bf16_bits*)tiles);
  const int grid = NXCD * ((prm.n_items + NXCD - 1) / NXCD);
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, WAVES, QT, true, false>), dim3(grid), dim3(WAVES * 64), 0, st, prm);
  else
    hipLaunchKernelGGL((attn_kernel<64, WAVES, QT, true, false>), dim3(grid), dim3(WAVES * 64), 0, st, prm);
  return hipGetLastError();
}

}  // namespace fva
