"""Pins for the oracle's pooling and router (CPU only).

Pinned to: closed forms of block means, a library matmul for the pooled
scores, a subset-enumeration brute force of the Top-p/Top-k rule in exact
rational arithmetic, a stable argsort for fixed top-k, and the special cases
the pages fix (top-k == num_blocks is dense; the floor is a lower bound).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import fvgen
import oracle


def _bf16(x):
    return fvgen.f64_to_bf16(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------- pooling
def test_pool_constant_channels():
    grid, block = (5, 9, 7), (4, 8, 8)
    L, heads, D = 5 * 9 * 7, 3, 16
    vals = (np.arange(heads * D).reshape(heads, D) - 20) / 8.0     # exact in bf16
    x = np.broadcast_to(vals, (1, L, heads, D))
    m = oracle.pool(_bf16(x), grid, block)
    assert np.array_equal(m[0], np.broadcast_to(vals[:, None, :], m[0].shape))


def test_pool_t_ramp_closed_form():
    grid, block = (31, 22, 40), (4, 8, 8)
    T, H, W = grid
    t = np.repeat(np.arange(T), H * W).astype(np.float64)
    x = np.broadcast_to(t[None, :, None, None], (1, T * H * W, 1, 8))
    m = oracle.pool(_bf16(x), grid, block)
    tab = oracle.block_table(grid, block)
    expect = tab[:, 0] + (tab[:, 3] - 1) / 2.0        # mean frame index of the block's frames
    assert np.array_equal(m[0, 0, :, 0], expect)


def test_pool_random_vs_longdouble():
    grid, block = (5, 9, 7), (4, 8, 8)
    rng = np.random.default_rng(1)
    L, heads, D = 5 * 9 * 7, 2, 8
    x = _bf16(rng.normal(size=(1, L, heads, D)))
    m = oracle.pool(x, grid, block)
    T, H, W = grid
    t, y, xx = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    blk = (((t // 4) * 2 + (y // 8)) * 1 + xx // 8).reshape(-1)
    xf = fvgen.bf16_to_f64(x)[0].astype(np.longdouble)
    for n in range(4):
        ref = xf[blk == n].mean(axis=0)                # [heads, D]
        np.testing.assert_allclose(m[0, :, n, :], ref.astype(np.float64), rtol=0, atol=1e-15)


def _blockwise_constant(grid, block, B, heads, D, seed):
    """bf16 tokens equal to one vector per (b, block, h): entries are small
    multiples of 1/8, so every block mean, product and dot product is exact
    in fp64.  Returns (bf16 bits [B, L, heads, D], values [B, heads, N, D])."""
    N = oracle.num_blocks(grid, block)
    tb = oracle.token_block(grid, block)
    rng = np.random.default_rng(seed)
    vals = rng.integers(-24, 25, size=(B, heads, N, D)) / 8.0
    x = np.transpose(vals[:, :, tb, :], (0, 2, 1, 3))      # [B, L, heads, D]
    return _bf16(x), vals


@pytest.mark.parametrize("D", [64, 128])
def test_scores_closed_form_and_scale_rule(D):
    """Q constant over each query block and K over each key block: the block
    means are those constants exactly, so s[b,h,i,j] = (a_bhi . c_bhj) /
    sqrt(D) with an exact dot product: head_dim^-0.5 scaling (VSA guide,
    section 5), i indexing query blocks and j key blocks, separately per
    batch entry and head.  For D = 64 the scale is exactly 1/8."""
    grid, block, B, heads = (5, 9, 7), (4, 8, 8), 2, 3    # ragged blocks: 224, 28, 56, 7 tokens
    q, a = _blockwise_constant(grid, block, B, heads, D, seed=D)
    k, c = _blockwise_constant(grid, block, B, heads, D, seed=D + 1)
    s = oracle.scores(oracle.pool(q, grid, block), oracle.pool(k, grid, block))
    N = oracle.num_blocks(grid, block)
    for b in range(B):
        for h in range(heads):
            for i in range(N):
                for j in range(N):
                    dot = sum((Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a[b, h, i], c[b, h, j])),
                              Fraction(0))
                    assert s[b, h, i, j] == float(dot) / math.sqrt(D)
                    if D == 64:
                        assert s[b, h, i, j] == float(dot / 8)
    # not symmetric in (i, j) and not shared across heads: an index slip shows
    assert not np.array_equal(s, np.swapaxes(s, -1, -2))
    assert not np.array_equal(s[:, 0], s[:, 1])


@pytest.mark.parametrize("top_p,k_floor,expect", [(0.3, 5, 29), (0.05, 9, 9), (0.777, 3, 75)])
def test_identical_keys_keep_lowest_indices_end_to_end(top_p, k_floor, expect):
    """Every key token the same bf16 vector: all key blocks pool to it, every
    row's scores tie, P = 1/N, so the router keeps max(k_floor, ceil(p N))
    blocks, the lowest indices first.  Runs the whole oracle router (pooling,
    scores, softmax, order, cumulative mass, floor) on bf16 inputs with p N
    not an integer (N = 96: p N = 28.8, 4.8, 74.59)."""
    grid, block, heads, D = (8, 16, 24), (2, 4, 4), 2, 64
    N = oracle.num_blocks(grid, block)
    assert N == 96 and expect == max(k_floor, math.ceil(np.float32(top_p) * N))
    L = 8 * 16 * 24
    rng = np.random.default_rng(11)
    q = _bf16(rng.normal(scale=2.0, size=(1, L, heads, D)))
    k = np.broadcast_to(_bf16(rng.normal(size=D)), (1, L, heads, D))
    mask, cnt, flags, status = oracle.route(q, k, grid, block, top_p, k_floor)
    assert status == 0 and (flags == 0).all()
    assert (cnt == expect).all()
    assert all(g == set(range(expect)) for g in _mask_sets(mask, N))


def test_scores_vs_matmul():
    wl = fvgen.WORKLOADS["tiny"]
    q, k, _ = fvgen.generate_qkv(wl)
    qb = oracle.pool(q, wl.grid, wl.block)
    kb = oracle.pool(k, wl.grid, wl.block)
    s = oracle.scores(qb, kb)
    ref = np.matmul(qb, np.swapaxes(kb, -1, -2)) / math.sqrt(wl.head_dim)
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- router
def _softmax_fractions(s):
    e = np.exp(s - s.max())
    p = e / e.sum()
    return [Fraction(float(v)) for v in p]


def brute_route_row(s, top_p, k_floor):
    """Top-p by definition: the smallest number of blocks whose probability mass
    reaches p, taking among equal-size subsets the one of largest mass and then
    the lexicographically lowest indices; then the Top-k floor.  Exact sums."""
    N = len(s)
    P = _softmax_fractions(s)
    p = Fraction(float(np.float32(top_p)))

    def best(m):
        bestset, bestmass = None, None
        for sub in itertools.combinations(range(N), m):
            mass = sum((P[j] for j in sub), Fraction(0))
            if bestmass is None or mass > bestmass:
                bestset, bestmass = sub, mass
        return bestset, bestmass

    if p >= 1:
        nstar = N
    elif p <= 0:
        nstar = 0
    else:
        nstar = N
        for m in range(1, N + 1):
            if best(m)[1] >= p:
                nstar = m
                break
    keep = min(N, max(k_floor, nstar))
    return set(best(keep)[0])


def _mask_sets(mask, N):
    b = oracle.mask_to_bool(mask, N)
    return [set(np.nonzero(r)[0].tolist()) for r in b.reshape(-1, N)]


@pytest.mark.parametrize("N,top_p,k_floor", [(6, 0.9, 1), (8, 0.5, 2), (10, 0.8, 3), (12, 0.95, 1), (9, 0.3, 4)])
def test_route_vs_subset_bruteforce(N, top_p, k_floor):
    rng = np.random.default_rng(N * 100 + k_floor)
    rows = rng.normal(scale=rng.uniform(0.2, 3.0, size=(24, 1)), size=(24, N))
    rows[0] = rows[0, 0]                       # all equal: exact ties everywhere
    rows[1, 3] = rows[1, 5] = rows[1].max()    # exact tie at the top
    rows[2, :N // 2] = rows[2, N // 2: 2 * (N // 2)]  # duplicated blocks
    mask, cnt, flags, status = oracle.route_scores(rows, top_p, k_floor)
    assert status == 0
    got = _mask_sets(mask, N)
    checked = 0
    for r in range(rows.shape[0]):
        if flags[r]:
            continue
        ref = brute_route_row(rows[r], top_p, k_floor)
        assert got[r] == ref, (r, rows[r])
        assert cnt[r] == len(ref)
        checked += 1
    assert checked >= 20


def test_route_constructed_near_threshold_rows_are_flagged():
    # P = (0.5, 0.3, 0.2 - d, d): with p = 0.8 the cut sits exactly on C_2
    N = 4
    for d, expect_flag in [(0.05, True), (0.01, True)]:
        P = np.array([0.5, 0.3, 0.2 - d, d])
        s = np.log(P)
        mask, cnt, flags, _ = oracle.route_scores(s[None], 0.8, 1)
        # C_2 = 0.8 in exact arithmetic (0.8 is not exactly the fp32 p): within 1e-5 -> flagged E1
        assert bool(flags[0] & oracle.FLAG_E1) == expect_flag
    # far from any step: not flagged, and the count is the textbook nucleus size
    s = np.log(np.array([0.5, 0.3, 0.15, 0.05]))
    mask, cnt, flags, _ = oracle.route_scores(s[None], 0.7, 1)
    assert flags[0] == 0 and cnt[0] == 2 and _mask_sets(mask, N)[0] == {0, 1}
    mask, cnt, flags, _ = oracle.route_scores(s[None], 0.81, 1)
    assert flags[0] == 0 and cnt[0] == 3 and _mask_sets(mask, N)[0] == {0, 1, 2}


def test_near_tie_at_cut_flagged_exact_tie_not():
    s = np.array([3.0, 2.0, 1.0, 1.0 - 1e-9, 0.0])
    _, cnt, flags, _ = oracle.route_scores(s[None], 0.0, 3)     # fixed top-3: cut between 1.0 and 1.0-1e-9
    assert cnt[0] == 3 and flags[0] & oracle.FLAG_E2
    s = np.array([3.0, 2.0, 1.0, 1.0, 0.0])
    mask, cnt, flags, _ = oracle.route_scores(s[None], 0.0, 3)  # exact tie: lower index wins, not flagged
    assert flags[0] == 0 and _mask_sets(mask, 5)[0] == {0, 1, 2}


def test_fixed_topk_matches_stable_argsort():
    rng = np.random.default_rng(7)
    N, k = 120, 64
    s = rng.normal(size=(50, N))
    s[:, 10] = s[:, 20]                               # exact ties resolved by index
    mask, cnt, flags, _ = oracle.route_scores(s, 0.0, k)
    got = _mask_sets(mask, N)
    for r in range(s.shape[0]):
        order = np.argsort(-s[r], kind="stable")     # stable: equal scores keep index order
        if flags[r]:
            continue
        assert got[r] == set(order[:k].tolist())
        assert cnt[r] == k


def test_dense_special_cases():
    rng = np.random.default_rng(3)
    N = 120
    s = rng.normal(scale=4.0, size=(20, N))
    for top_p, k_floor in [(1.0, 1), (1.5, 8), (0.5, N), (0.0, N)]:
        mask, cnt, flags, _ = oracle.route_scores(s, top_p, k_floor)
        assert (cnt == N).all()
        assert all(g == set(range(N)) for g in _mask_sets(mask, N))


def test_uniform_scores_keep_ceil_pN_lowest():
    for N, p, kf in [(120, 0.905, 8), (360, 0.951, 16), (8, 0.93, 2), (120, 0.05, 8)]:
        s = np.zeros((3, N))
        mask, cnt, flags, _ = oracle.route_scores(s, p, kf)
        keep = max(kf, math.ceil(p * N))
        assert (cnt == keep).all() and (flags == 0).all()
        assert all(g == set(range(keep)) for g in _mask_sets(mask, N))


def test_nonfinite_row_repaired_dense():
    s = np.zeros((3, 16))
    s[0, 4] = np.nan
    s[2, 7] = np.inf
    mask, cnt, flags, status = oracle.route_scores(s, 0.9, 2)
    assert status == 1
    assert cnt[0] == 16 and cnt[2] == 16 and cnt[1] == max(2, math.ceil(0.9 * 16))
    assert flags[0] & oracle.FLAG_NONFINITE and flags[2] & oracle.FLAG_NONFINITE and not flags[1]


def test_route_rejects_bad_floor():
    with pytest.raises(ValueError):
        oracle.route_scores(np.zeros((1, 8)), 0.9, 9)
    with pytest.raises(ValueError):
        oracle.route_scores(np.zeros((1, 8)), 0.9, 0)
    with pytest.raises(ValueError):
        oracle.route_scores(np.zeros((1, 8)), float("nan"), 2)


@pytest.mark.parametrize("name", ["tiny", "wan14b"])
def test_route_invariants_on_workload(name):
    wl = fvgen.WORKLOADS[name]
    q = fvgen.generate(wl, "q")
    k = fvgen.generate(wl, "k")
    mask, cnt, flags, status = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    N = oracle.num_blocks(wl.grid, wl.block)
    qb = oracle.pool(q, wl.grid, wl.block)
    kb = oracle.pool(k, wl.grid, wl.block)
    s = oracle.scores(qb, kb).reshape(-1, N)
    kept = oracle.mask_to_bool(mask, N).reshape(-1, N)
    assert status == 0
    assert (cnt.reshape(-1) == kept.sum(1)).all()
    assert (cnt >= wl.k_floor).all() and (cnt <= N).all()
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    p = float(np.float32(wl.top_p))
    for r in range(s.shape[0]):
        ks, ds = s[r][kept[r]], s[r][~kept[r]]
        if ds.size:
            # kept set is a prefix of the descending order
            assert ks.min() >= ds.max()
        mass = P[r][kept[r]].sum()
        if cnt.reshape(-1)[r] > wl.k_floor and not flags.reshape(-1)[r]:
            assert mass >= p - 1e-12
            # minimal: dropping the weakest kept block falls below p
            assert mass - P[r][kept[r]].min() < p + 1e-12
    assert (flags != 0).mean() < 0.01


def test_top_p_monotone_in_p():
    wl = fvgen.WORKLOADS["tiny"]
    q, k, _ = fvgen.generate_qkv(wl)
    prev = None
    for p in [0.1, 0.3, 0.5, 0.7, 0.9, 0.99]:
        _, cnt, _, _ = oracle.route(q, k, wl.grid, wl.block, p, 1)
        if prev is not None:
            assert (cnt >= prev).all()
        prev = cnt
