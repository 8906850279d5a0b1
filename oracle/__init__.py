"""ctypes binding of the fp64 CPU oracle (oracle/fvo.cpp).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg.  The product package never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fvo.cpp")
_LIB = os.path.join(_HERE, "libfvo.so")

FLAG_E1 = 1          # top-p threshold within 1e-5 of a cumulative-mass step that changes the count
FLAG_E2 = 2          # near-tie (not exact) between the last kept and first dropped block score
FLAG_NONFINITE = 4   # row had a non-finite score; repaired to all blocks


def build(force: bool = False) -> str:
    """Compile libfvo.so with g++ (C++17, plain -O2, std::thread)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_P = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        override = os.environ.get("FVO_LIB")   # another build of the same source (e.g. with sanitizers)
        if not override and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(override or _LIB)
        lib.fvo_num_blocks.restype = ctypes.c_int
        lib.fvo_num_blocks.argtypes = [_P]
        lib.fvo_block_table.restype = ctypes.c_int
        lib.fvo_block_table.argtypes = [_P, _P]
        lib.fvo_token_block.restype = ctypes.c_int
        lib.fvo_token_block.argtypes = [_P, _P]
        lib.fvo_pool.restype = ctypes.c_int
        lib.fvo_pool.argtypes = [_P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int]
        lib.fvo_scores.restype = ctypes.c_int
        lib.fvo_scores.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int]
        lib.fvo_route_scores.restype = ctypes.c_int
        lib.fvo_route_scores.argtypes = [_P, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                         ctypes.c_double, _P, _P, _P, _P, ctypes.c_int]
        lib.fvo_route.restype = ctypes.c_int
        lib.fvo_route.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P,
                                  ctypes.c_float, ctypes.c_int, ctypes.c_double, _P, _P, _P, _P, ctypes.c_int]
        lib.fvo_attn.restype = ctypes.c_int
        lib.fvo_attn.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, _P, _P,
                                 ctypes.c_double, _P, ctypes.c_int64, _P, ctypes.c_int]
        lib.fvo_real_pairs.restype = ctypes.c_int64
        lib.fvo_real_pairs.argtypes = [_P, _P, ctypes.c_int64]
        lib.fvo_hardware_threads.restype = ctypes.c_int
        lib.fvo_hardware_threads.argtypes = []
        _lib = lib
    return _lib


def host_threads() -> int:
    """Threads the oracle runs on by default: every CPU this process may run
    on (its affinity mask), capped by OMP_NUM_THREADS when the environment
    sets it (the CPU share of a shared host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("" if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def _threads(n):
    if n:
        return n
    return host_threads()


def _grid6(grid, block):
    return np.ascontiguousarray(list(grid) + list(block), dtype=np.int32)


def _c(x, dtype):
    a = np.ascontiguousarray(x, dtype=dtype)
    return a


def hardware_threads() -> int:
    return _load().fvo_hardware_threads()


def num_blocks(grid, block) -> int:
    g = _grid6(grid, block)
    return _load().fvo_num_blocks(g.ctypes.data)


def block_table(grid, block) -> np.ndarray:
    """[N, 7] int32: t0, y0, x0, et, eh, ew, real count."""
    g = _grid6(grid, block)
    n = num_blocks(grid, block)
    out = np.empty((n, 7), dtype=np.int32)
    _load().fvo_block_table(g.ctypes.data, out.ctypes.data)
    return out


def token_block(grid, block) -> np.ndarray:
    g = _grid6(grid, block)
    T, H, W = grid
    out = np.full(T * H * W, -1, dtype=np.int32)
    _load().fvo_token_block(g.ctypes.data, out.ctypes.data)
    return out


def pool(x: np.ndarray, grid, block, nthreads=None) -> np.ndarray:
    """x bf16 bits [B, L, heads, D] -> fp64 block means [B, heads, N, D]."""
    x = _c(x, np.uint16)
    B, L, heads, D = x.shape
    g = _grid6(grid, block)
    N = num_blocks(grid, block)
    out = np.empty((B, heads, N, D), dtype=np.float64)
    rc = _load().fvo_pool(x.ctypes.data, B, L, heads, D, g.ctypes.data, out.ctypes.data, _threads(nthreads))
    if rc < 0:
        raise ValueError("fvo_pool failed (%d)" % rc)
    return out


def scores(qbar: np.ndarray, kbar: np.ndarray, nthreads=None) -> np.ndarray:
    qbar = _c(qbar, np.float64)
    kbar = _c(kbar, np.float64)
    B, heads, N, D = qbar.shape
    out = np.empty((B, heads, N, N), dtype=np.float64)
    _load().fvo_scores(qbar.ctypes.data, kbar.ctypes.data, B, heads, N, D, out.ctypes.data, _threads(nthreads))
    return out


MARGIN = 1e-5   # ambiguity margin on the cumulative-mass threshold and on score gaps at the cut


def route_scores(s: np.ndarray, top_p: float, k_floor: int, nthreads=None, margin: float = MARGIN):
    """Rows of scores [..., N] -> (mask [..., ceil(N/32)] u32, cnt [...] i32, flags [...] u8, status)."""
    s = _c(s, np.float64)
    N = s.shape[-1]
    lead = s.shape[:-1]
    R = int(np.prod(lead)) if lead else 1
    words = (N + 31) // 32
    mask = np.zeros(lead + (words,), dtype=np.uint32)
    cnt = np.zeros(lead, dtype=np.int32)
    flags = np.zeros(lead, dtype=np.uint8)
    status = np.zeros(1, dtype=np.uint32)
    rc = _load().fvo_route_scores(s.ctypes.data, R, N, float(top_p), int(k_floor), float(margin), mask.ctypes.data,
                                  cnt.ctypes.data, flags.ctypes.data, status.ctypes.data, _threads(nthreads))
    if rc < 0:
        raise ValueError("fvo_route_scores rejected its arguments")
    return mask, cnt, flags, int(status[0])


def route(q: np.ndarray, k: np.ndarray, grid, block, top_p: float, k_floor: int, nthreads=None,
          margin: float = MARGIN):
    """bf16 Q, K [B, L, heads, D] -> (mask [B, heads, N, W] u32, cnt [B, heads, N], flags, status)."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    B, L, heads, D = q.shape
    g = _grid6(grid, block)
    N = num_blocks(grid, block)
    words = (N + 31) // 32
    mask = np.zeros((B, heads, N, words), dtype=np.uint32)
    cnt = np.zeros((B, heads, N), dtype=np.int32)
    flags = np.zeros((B, heads, N), dtype=np.uint8)
    status = np.zeros(1, dtype=np.uint32)
    rc = _load().fvo_route(q.ctypes.data, k.ctypes.data, B, L, heads, D, g.ctypes.data, float(top_p),
                           int(k_floor), float(margin), mask.ctypes.data, cnt.ctypes.data, flags.ctypes.data,
                           status.ctypes.data, _threads(nthreads))
    if rc < 0:
        raise ValueError("fvo_route rejected its arguments (%d)" % rc)
    return mask, cnt, flags, int(status[0])


def attn(q, k, v, grid, block, mask, scale, items=None, nthreads=None, out=None) -> np.ndarray:
    """Block-sparse attention in fp64 -> [B, L, heads, D] (NaN where not computed).

    items: optional 1-D array of item ids (b*heads + h)*N + i."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    mask = _c(mask, np.uint32)
    B, L, heads, D = q.shape
    g = _grid6(grid, block)
    if out is None:
        out = np.full((B, L, heads, D), np.nan, dtype=np.float64)
    if items is None:
        ip, n = None, 0
    else:
        items = _c(items, np.int64)
        ip, n = items.ctypes.data, items.size
    rc = _load().fvo_attn(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, L, heads, D, g.ctypes.data,
                          mask.ctypes.data, float(scale), ip, n, out.ctypes.data, _threads(nthreads))
    if rc < 0:
        raise ValueError("fvo_attn rejected its arguments (%d)" % rc)
    return out


def _block_order(grid, block):
    """(perm, start, count): the token ids of every block, blocks in index
    order and each block's tokens in ascending id (row-major over t, y, x),
    concatenated; block n's tokens are perm[start[n] : start[n] + count[n]]."""
    tb = token_block(grid, block)
    perm = np.argsort(tb, kind="stable")
    count = np.bincount(tb, minlength=num_blocks(grid, block)).astype(np.int64)
    start = np.concatenate(([0], np.cumsum(count)[:-1]))
    return perm, start, count


def attn_matmul(q, k, v, grid, block, mask, scale, items=None, nthreads=None, out=None) -> np.ndarray:
    """Block-sparse attention in fp64, the two products by a library matmul.

    The definition attn() follows (VSA guide, sections 1 and 6: a query
    block attends to the real tokens of its selected key blocks only), with
    the per-token loops replaced by matrix products over one query block:
    for item (b, h, i), Q = the real rows of block i, K and V = the real rows
    of the kept key blocks in ascending block order, all widened exactly to
    fp64; S = (Q K^T) * scale; P = exp(S - rowmax(S)); O = (P V) / rowsum(P).
    Only the order of the sums inside the two products differs from attn();
    it is the same function up to fp64 rounding, and is used where attn()'s
    plain loops would take too long.  Items run on a pool of host threads,
    each calling the matmul single-threaded.  Returns [B, L, heads, D] fp64
    (NaN where not computed; a row with no kept block gives NaN, as attn()).
    """
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    mask = _c(mask, np.uint32)
    B, L, heads, D = q.shape
    N = num_blocks(grid, block)
    if out is None:
        out = np.full((B, L, heads, D), np.nan, dtype=np.float64)
    items = np.arange(B * heads * N, dtype=np.int64) if items is None else np.asarray(items, dtype=np.int64)
    perm, start, count = _block_order(grid, block)
    keep = mask_to_bool(mask.reshape(B * heads * N, -1), N)

    def widen(x, b, h):
        return (x[b, :, h, :].astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def one(b, h, i, Qh, Kb, Vb):
        rows = perm[start[i]:start[i] + count[i]]
        sel = np.repeat(keep[(b * heads + h) * N + i], count)   # block-ordered key positions kept
        Ks, Vs = Kb[sel], Vb[sel]
        S = Qh[rows] @ Ks.T
        S *= scale
        S -= S.max(axis=1, keepdims=True) if Ks.shape[0] else 0.0
        np.exp(S, out=S)
        with np.errstate(invalid="ignore", divide="ignore"):
            out[b, rows, h, :] = (S @ Vs) / S.sum(axis=1, keepdims=True)

    by_head = {}
    for it in items.tolist():
        by_head.setdefault(it // N, []).append(it % N)
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(max_workers=_threads(nthreads)) as ex:
        for bh, blocks in sorted(by_head.items()):
            b, h = divmod(bh, heads)
            Qh = widen(q, b, h)
            Kb = widen(k, b, h)[perm]    # keys and values in block order
            Vb = widen(v, b, h)[perm]
            list(ex.map(lambda i: one(b, h, i, Qh, Kb, Vb), blocks))
    return out


def real_pairs(grid, block, mask) -> int:
    """Real (query, key) token pairs the mask asks for; attention FLOPs = 4*D*pairs."""
    mask = _c(mask, np.uint32)
    N = num_blocks(grid, block)
    rows = mask.size // (((N + 31) // 32) * N)
    g = _grid6(grid, block)
    return int(_load().fvo_real_pairs(g.ctypes.data, mask.ctypes.data, rows))


def static_mask(grid, block, local=(1, 1, 1), anchor_t=0, B=1, heads=1):
    """Static block mask: local boxes plus anchor slabs.

    Sol-Attn article (bjdmk.com.cn), section 3.2: a query-key pair is kept
    when both lie in the same local window or when either is an anchor.  The
    rule is applied to block coordinates: (t, y, x) of a block is its origin
    (from the oracle's own block table) divided by the block size; the local
    windows are boxes of local = (lt, lh, lw) blocks partitioning the block
    grid; the anchors are the blocks whose temporal coordinate is a multiple
    of anchor_t (none when anchor_t == 0).

    Returns (mask uint32 [B, heads, N, ceil(N/32)], counts int32 [B, heads, N]),
    the same pattern for every (b, h).
    """
    tab = block_table(grid, block)
    coords = tab[:, 0:3].astype(np.int64) // np.array(block, dtype=np.int64)
    box = coords // np.array(local, dtype=np.int64)
    keep = (box[:, None, :] == box[None, :, :]).all(-1)
    if anchor_t > 0:
        anchor = coords[:, 0] % anchor_t == 0
        keep = keep | anchor[:, None] | anchor[None, :]
    N = keep.shape[0]
    words = (N + 31) // 32
    padded = np.zeros((N, words * 32), dtype=np.uint64)
    padded[:, :N] = keep
    row = (padded.reshape(N, words, 32) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    mask = np.broadcast_to(row, (B, heads, N, words)).copy()
    counts = np.broadcast_to(keep.sum(1).astype(np.int32), (B, heads, N)).copy()
    return mask, counts


def sasa_row_rate(counts):
    """Steps of one 32-key half on the busiest SIMD per 64-key chunk for query
    blocks of `counts` tokens: ceil(ceil(c / 32) / 2)."""
    c = np.asarray(counts, dtype=np.int64)
    return ((c + 31) // 32 + 1) // 2


def sasa_key_chunks(counts):
    """64-key chunks of key blocks of `counts` tokens: ceil(c / 64)."""
    return (np.asarray(counts, dtype=np.int64) + 63) // 64


def sasa(scores: np.ndarray, mask: np.ndarray, grid, block, rounds: int, margin: float = MARGIN, xcd_weight=None):
    """Slack-aware sparse augmentation, one-GPU form (8 XCDs as the ranks).

    FVAttn abstract and summary, key modules 2 and 3: after load balancing the
    non-critical ranks have slack, filled with extra high-value blocks chosen
    from the attention scores without lengthening the critical path.  Steps:
      1. row cost = the attention kernel's time on the row, in steps of one
         32-key half on its busiest SIMD: r_i = ceil(ceil(c_i / 32) / 2)
         steps per 64-key chunk (row tiles of 32 on 8 wavefronts, two per
         SIMD, a ragged block's tiles splitting their key halves over two
         wavefronts) times ceil(c_j / 64) chunks summed over the row's kept
         blocks; head cost = sum over its rows;
      2. heads by cost descending (ties: lower head) each go to the XCD with
         the least load so far (ties: lower XCD); makespan M = max load;
      3. on every XCD, offers in rounds r = 0..rounds-1: for each of its heads
         (in assignment order) and each row (block order), the row's r-th
         dropped block in the router's order (score descending, lower index
         first; non-finite scores are never offered); offers are taken in
         that order until the first one whose cost r_i * ceil(c_j / 64) no
         longer fits M - load (rows without an r-th dropped block are passed
         over).
    scores: fp64 [B, heads, N, N] (oracle.scores); mask: the routed mask.
    xcd_weight: optional relative speed w_x of each XCD (integers); a head then
    goes to the XCD where it would finish first, (load_x + c) / w_x (ties:
    lower XCD), the critical XCD m has the largest load_m / w_m (ties: lower),
    and XCD x takes offers up to floor(load_m * w_x / w_m) - load_x.  None:
    all equal (the rule above).
    Returns (mask_out, counts, head_xcd [B*heads], load [8], added [8],
    flags [B, heads, N]) where a flagged row has two of its first rounds+1
    dropped candidates within margin * max(1, |s|) of each other without being
    equal (their order may differ under another fp64 rounding order).
    """
    B, heads, N, _ = scores.shape
    BH = B * heads
    c = block_table(grid, block)[:, 6].astype(np.int64)
    rate = sasa_row_rate(c)
    chunks = sasa_key_chunks(c)
    keep = mask_to_bool(mask, N).reshape(BH, N, N)
    S = scores.reshape(BH, N, N)
    row_cost = rate[None, :] * (keep * chunks[None, None, :]).sum(-1)
    head_cost = row_cost.sum(1)
    w = [1000] * 8 if xcd_weight is None else [int(v) for v in xcd_weight]
    load = [0] * 8
    heads_of = [[] for _ in range(8)]
    head_xcd = np.zeros(BH, dtype=np.int32)
    for h in sorted(range(BH), key=lambda h: (-int(head_cost[h]), h)):
        cst = int(head_cost[h])
        # the XCD where the head would finish first: compare (load + c) / w by cross-multiplying
        x = 0
        for y in range(1, 8):
            if (load[y] + cst) * w[x] < (load[x] + cst) * w[y]:
                x = y
        load[x] += cst
        heads_of[x].append(h)
        head_xcd[h] = x
    m = 0
    for y in range(1, 8):
        if load[y] * w[m] > load[m] * w[y]:
            m = y

    # each row's first rounds+1 dropped blocks in the router's order
    cand = np.full((BH, N, rounds + 1), -1, dtype=np.int64)
    flags = np.zeros((BH, N), dtype=bool)
    for h in range(BH):
        for i in range(N):
            js = np.nonzero(~keep[h, i] & np.isfinite(S[h, i]))[0]
            if js.size == 0:
                continue
            order = js[np.lexsort((js, -S[h, i, js]))][: rounds + 1]
            cand[h, i, : order.size] = order
            sv = S[h, i, order]
            gap = np.abs(np.diff(sv))
            flags[h, i] = bool(((gap > 0) & (gap < margin * np.maximum(1.0, np.abs(sv[1:])))).any())

    out = keep.copy()
    added = [0] * 8
    for x in range(8):
        slack = load[m] * w[x] // w[m] - load[x]
        acc = 0
        stop = False
        for r in range(rounds):
            for h in heads_of[x]:
                for i in range(N):
                    j = int(cand[h, i, r])
                    if j < 0:
                        continue
                    cost = int(rate[i] * chunks[j])
                    if acc + cost > slack:
                        stop = True
                        break
                    acc += cost
                    out[h, i, j] = True
                if stop:
                    break
            if stop:
                break
        added[x] = acc

    words = (N + 31) // 32
    padded = np.zeros((BH, N, words * 32), dtype=np.uint64)
    padded[..., :N] = out
    mask_out = (padded.reshape(BH, N, words, 32) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    counts = out.sum(-1).astype(np.int32)
    return (mask_out.reshape(B, heads, N, words), counts.reshape(B, heads, N), head_xcd,
            np.array(load, dtype=np.int64), np.array(added, dtype=np.int64), flags.reshape(B, heads, N))


def default_group(block) -> tuple:
    """Blocks per work item (t, y, x) of the sparse attention: an item fills 8
    wavefronts of 32 query rows, so blocks of at most 64 tokens are taken
    2 x 1 x 2 per item and blocks of 65..128 tokens 1 x 1 x 2."""
    vol = int(block[0]) * int(block[1]) * int(block[2])
    if vol <= 64:
        return (2, 1, 2)
    if vol <= 128:
        return (1, 1, 2)
    return (1, 1, 1)


def work_items(grid, block, group) -> list:
    """Member block ids of each work item of one (b, h): boxes of group =
    (gt, gh, gw) blocks tiling the block grid from its origin (cut at the
    grid's far edges), numbered t-major, then y, then x; members likewise."""
    nT, nH, nW = (-(-int(d) // int(b)) for d, b in zip(grid, block))
    gt, gh, gw = (int(x) for x in group)
    items = []
    for t0 in range(0, nT, gt):
        for y0 in range(0, nH, gh):
            for x0 in range(0, nW, gw):
                items.append([(t * nH + y) * nW + x
                              for t in range(t0, min(t0 + gt, nT))
                              for y in range(y0, min(y0 + gh, nH))
                              for x in range(x0, min(x0 + gw, nW))])
    return items


def lpt_schedule(grid, block, mask, B, heads, group=None, naive=False, head_xcd=None, queues=8):
    """Work items, their costs and the queues of the persistent attention kernel.

    FVAttn abstract (key module 1, runtime load balancing) and the workload
    model of its summary: a unit of work costs the real token pairs it
    computes.  An item = the query blocks of work_items() for one (b, h); its
    cost = (sum of its members' real rows) x (real tokens of the union of its
    members' kept blocks), the work its wavefronts stream.  List scheduling in
    LPT order over the XCD queues: heads by summed item cost descending (ties:
    lower head) each go to the queue with the least cost so far (ties: lower
    queue), or to head_xcd[h] when given; a queue holds its heads in that
    order, and each head's items by cost descending (ties: lower item id).
    naive: every head on queue 0 in head order, items in id order.
    Returns (cost int64 [B*heads*G] by item id, order int64 [B*heads*G],
    qoff int64 [queues + 1]) with item id = (b*heads + h)*G + g.
    """
    if group is None:
        group = default_group(block)
    N = num_blocks(grid, block)
    BH = B * heads
    c = block_table(grid, block)[:, 6].astype(np.int64)
    keep = mask_to_bool(np.asarray(mask, dtype=np.uint32), N).reshape(BH, N, N)
    items = work_items(grid, block, group)
    G = len(items)
    cost = np.zeros(BH * G, dtype=np.int64)
    for h in range(BH):
        for g, members in enumerate(items):
            union = keep[h, members].any(0)
            cost[h * G + g] = int(c[members].sum()) * int(c[union].sum())
    if naive:
        order = np.arange(BH * G, dtype=np.int64)
        qoff = np.array([0] + [BH * G] * queues, dtype=np.int64)
        return cost, order, qoff
    head_cost = cost.reshape(BH, G).sum(1)
    load = [0] * queues
    heads_of = [[] for _ in range(queues)]
    for h in sorted(range(BH), key=lambda h: (-int(head_cost[h]), h)):
        x = int(head_xcd[h]) if head_xcd is not None else min(range(queues), key=lambda x: (load[x], x))
        load[x] += int(head_cost[h])
        heads_of[x].append(h)
    order, qoff = [], [0]
    for x in range(queues):
        for h in heads_of[x]:
            ids = range(h * G, (h + 1) * G)
            order.extend(sorted(ids, key=lambda a: (-int(cost[a]), a)))
        qoff.append(len(order))
    return cost, np.array(order, dtype=np.int64), np.array(qoff, dtype=np.int64)


def dense_mask(B, heads, N) -> np.ndarray:
    words = (N + 31) // 32
    m = np.zeros((B, heads, N, words), dtype=np.uint32)
    for j in range(N):
        m[..., j >> 5] |= np.uint32(1 << (j & 31))
    return m


def mask_to_bool(mask: np.ndarray, N: int) -> np.ndarray:
    """u32 words [..., W] -> bool [..., N]."""
    bits = (mask[..., :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(mask.shape[:-1] + (-1,))[..., :N].astype(bool)
