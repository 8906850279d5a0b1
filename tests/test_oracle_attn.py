"""Pins for the oracle's block-sparse attention (CPU only).

Pinned to: a token-level brute force (explicit L x L mask and a textbook
masked softmax in numpy), torch's CPU fp64 scaled_dot_product_attention for
the dense special case (all blocks kept), and closed forms (constant V,
Q = 0, a single real key).
"""
import math

import numpy as np
import pytest
import torch

import fvgen
import oracle


def _bf16(x):
    return fvgen.f64_to_bf16(np.asarray(x, dtype=np.float64))


def _token_blocks(grid, block):
    T, H, W = grid
    bt, bh, bw = block
    nH, nW = -(-H // bh), -(-W // bw)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return (((t // bt) * nH + (y // bh)) * nW + (x // bw)).reshape(-1)


def brute_attention(q, k, v, grid, block, mask, scale):
    """Dense masked softmax over an explicit token-level mask built from the block mask."""
    Q, K, V = (fvgen.bf16_to_f64(a) for a in (q, k, v))
    B, L, heads, D = Q.shape
    N = oracle.num_blocks(grid, block)
    tb = _token_blocks(grid, block)
    kept = oracle.mask_to_bool(mask, N)                # [B, heads, N, N]
    out = np.empty_like(Q)
    for b in range(B):
        for h in range(heads):
            allow = kept[b, h][tb][:, tb]               # [L, L] token mask
            S = Q[b, :, h, :] @ K[b, :, h, :].T * scale
            S = np.where(allow, S, -np.inf)
            S -= S.max(axis=1, keepdims=True)
            Pm = np.exp(S)
            out[b, :, h, :] = (Pm @ V[b, :, h, :]) / Pm.sum(axis=1, keepdims=True)
    return out


def _random_mask(rng, B, heads, N, density):
    words = (N + 31) // 32
    m = np.zeros((B, heads, N, words), dtype=np.uint32)
    keep = rng.random((B, heads, N, N)) < density
    keep[..., np.arange(N), rng.integers(0, N, size=N)] = True   # at least one block per row
    for j in range(N):
        m[..., j >> 5] |= (keep[..., j].astype(np.uint32) << np.uint32(j & 31))
    return m


@pytest.mark.parametrize("grid,block,heads,D", [
    ((5, 9, 7), (4, 8, 8), 2, 16),       # ragged: counts 224, 28, 56, 7
    ((6, 10, 13), (4, 4, 4), 1, 32),     # 64-token tiles with ragged edges
])
def test_attn_vs_token_level_bruteforce(grid, block, heads, D):
    rng = np.random.default_rng(11)
    L = math.prod(grid)
    q, k, v = (_bf16(rng.normal(scale=s, size=(1, L, heads, D))) for s in (2.0, 1.0, 1.0))
    N = oracle.num_blocks(grid, block)
    mask = _random_mask(rng, 1, heads, N, 0.5)
    scale = 1.0 / math.sqrt(D)
    got = oracle.attn(q, k, v, grid, block, mask, scale)
    ref = brute_attention(q, k, v, grid, block, mask, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attn_tiny_workload_vs_bruteforce_on_routed_mask():
    wl = fvgen.WORKLOADS["tiny"]
    q, k, v = fvgen.generate_qkv(wl)
    mask, cnt, flags, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    scale = 1.0 / math.sqrt(wl.head_dim)
    got = oracle.attn(q, k, v, wl.grid, wl.block, mask, scale)
    ref = brute_attention(q, k, v, wl.grid, wl.block, mask, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_dense_mask_equals_torch_sdpa_fp64():
    grid, block, heads, D = (5, 9, 7), (4, 8, 8), 3, 32
    rng = np.random.default_rng(5)
    L = math.prod(grid)
    q, k, v = (_bf16(rng.normal(scale=s, size=(1, L, heads, D))) for s in (3.0, 1.0, 1.0))
    N = oracle.num_blocks(grid, block)
    got = oracle.attn(q, k, v, grid, block, oracle.dense_mask(1, heads, N), 1.0 / math.sqrt(D))
    t = [torch.from_numpy(fvgen.bf16_to_f64(a)).permute(0, 2, 1, 3) for a in (q, k, v)]   # BHLD
    ref = torch.nn.functional.scaled_dot_product_attention(*t).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_closed_forms():
    grid, block, heads, D = (5, 9, 9), (4, 8, 8), 1, 8
    L = math.prod(grid)
    N = oracle.num_blocks(grid, block)
    tab = oracle.block_table(grid, block)
    rng = np.random.default_rng(9)
    scale = 1.0 / math.sqrt(D)
    mask = _random_mask(rng, 1, heads, N, 0.6)
    q = _bf16(rng.normal(size=(1, L, heads, D)))
    k = _bf16(rng.normal(size=(1, L, heads, D)))
    # V constant -> O constant
    vc = _bf16(np.full((1, L, heads, D), 0.375))
    o = oracle.attn(q, k, vc, grid, block, mask, scale)
    assert np.abs(o - 0.375).max() < 1e-14
    # Q = 0 -> O = mean of the kept real V rows
    v = _bf16(rng.normal(size=(1, L, heads, D)))
    o = oracle.attn(_bf16(np.zeros((1, L, heads, D))), k, v, grid, block, mask, scale)
    tb = _token_blocks(grid, block)
    kept = oracle.mask_to_bool(mask, N)[0, 0]
    V = fvgen.bf16_to_f64(v)[0, :, 0, :]
    for i in range(N):
        ref = V[kept[i][tb]].mean(axis=0)
        np.testing.assert_allclose(o[0, tb == i, 0, :], np.broadcast_to(ref, (int((tb == i).sum()), D)),
                                   rtol=0, atol=1e-13)
    # one real key: the corner block (4..4, 8..8, 8..8) has a single token
    single = int(np.nonzero(tab[:, 6] == 1)[0][0])
    m1 = np.zeros_like(mask)
    m1[..., single >> 5] = np.uint32(1 << (single & 31))
    o = oracle.attn(q, k, v, grid, block, m1, scale)
    tok = int(np.nonzero(tb == single)[0][0])
    assert np.array_equal(o[0, :, 0, :], np.broadcast_to(V[tok], (L, D)))


def test_output_within_kept_value_range():
    wl = fvgen.WORKLOADS["tiny"]
    q, k, v = fvgen.generate_qkv(wl)
    mask, _, _, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    o = oracle.attn(q, k, v, wl.grid, wl.block, mask, 1.0 / math.sqrt(wl.head_dim))
    N = oracle.num_blocks(wl.grid, wl.block)
    tb = _token_blocks(wl.grid, wl.block)
    kept = oracle.mask_to_bool(mask, N)[0]
    V = fvgen.bf16_to_f64(v)[0]
    for h in range(wl.heads):
        for i in range(N):
            kv = V[kept[h, i][tb], h, :]
            oi = o[0, tb == i, h, :]
            assert (oi >= kv.min(axis=0) - 1e-12).all() and (oi <= kv.max(axis=0) + 1e-12).all()


def test_permutation_within_block():
    """Permuting tokens inside one block leaves the routing unchanged (the pooled
    mean is order-free) and permutes the block's outputs the same way."""
    wl = fvgen.WORKLOADS["tiny"]
    q, k, v = fvgen.generate_qkv(wl)
    tb = _token_blocks(wl.grid, wl.block)
    idx = np.nonzero(tb == 3)[0]
    rng = np.random.default_rng(2)
    perm = np.arange(wl.L)
    perm[idx] = rng.permutation(idx)
    qp, kp, vp = (a[:, perm] for a in (q, k, v))
    m1, c1, f1, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    m2, c2, f2, _ = oracle.route(qp, kp, wl.grid, wl.block, wl.top_p, wl.k_floor)
    ok = (f1 == 0) & (f2 == 0)
    assert np.array_equal(m1[ok], m2[ok])
    scale = 1.0 / math.sqrt(wl.head_dim)
    o1 = oracle.attn(q, k, v, wl.grid, wl.block, m1, scale)
    o2 = oracle.attn(qp, kp, vp, wl.grid, wl.block, m1, scale)
    np.testing.assert_allclose(o2, o1[:, perm], rtol=0, atol=1e-12)


def test_real_pairs_counts():
    grid, block = (31, 22, 40), (4, 8, 8)
    N = 120
    dense = oracle.dense_mask(1, 2, N)
    assert oracle.real_pairs(grid, block, dense) == 2 * 27280 * 27280


@pytest.mark.parametrize("case", ["tiny_routed", "ragged_b2_d128", "tiles64_d64", "empty_rows"])
def test_attn_matmul_equals_loops(case):
    """oracle.attn_matmul (the same definition with library matrix products,
    used for whole-workload parity) equals oracle.attn (plain loops) up to
    fp64 rounding, NaN (a row with no kept block) in the same places."""
    rng = np.random.default_rng(5)
    if case == "tiny_routed":
        wl = fvgen.WORKLOADS["tiny"]
        q, k, v = fvgen.generate_qkv(wl)
        grid, block, D = wl.grid, wl.block, wl.head_dim
        mask = oracle.route(q, k, grid, block, wl.top_p, wl.k_floor)[0]
    else:
        grid, block, B, heads, D = {"ragged_b2_d128": ((5, 9, 7), (4, 8, 8), 2, 2, 128),
                                    "tiles64_d64": ((6, 10, 13), (4, 4, 4), 1, 2, 64),
                                    "empty_rows": ((6, 10, 13), (4, 4, 4), 1, 1, 64)}[case]
        L = grid[0] * grid[1] * grid[2]
        q, k, v = (_bf16(rng.normal(scale=s, size=(B, L, heads, D))) for s in (2.0, 1.0, 1.0))
        N = oracle.num_blocks(grid, block)
        mask = _random_mask(rng, B, heads, N, 0.4)
        if case == "empty_rows":
            mask[0, 0, [0, 7, N - 1]] = 0
    scale = 1.0 / math.sqrt(D)
    a = oracle.attn(q, k, v, grid, block, mask, scale)
    b = oracle.attn_matmul(q, k, v, grid, block, mask, scale, nthreads=3)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert (case == "empty_rows") == bool(np.isnan(a).any())
    ok = ~np.isnan(a)
    assert np.abs(a[ok] - b[ok]).max() <= 1e-12


def test_attn_matmul_item_subset_and_constant_v():
    """Only the listed items are written; V constant over the kept keys gives O = that constant (up to the rounding of sum(w v) / sum(w))."""
    grid, block, heads, D = (5, 9, 7), (4, 8, 8), 2, 32
    L = 5 * 9 * 7
    rng = np.random.default_rng(9)
    q, k = (_bf16(rng.normal(size=(1, L, heads, D))) for _ in range(2))
    v = _bf16(np.broadcast_to(np.linspace(-2, 2, D), (1, L, heads, D)))
    N = oracle.num_blocks(grid, block)
    mask = _random_mask(rng, 1, heads, N, 0.5)
    items = np.array([1, N + 3])
    o = oracle.attn_matmul(q, k, v, grid, block, mask, 1.0 / math.sqrt(D), items=items)
    tb = oracle.token_block(grid, block)
    written = np.zeros((L, heads), dtype=bool)
    written[tb == 1, 0] = True
    written[tb == 3, 1] = True
    assert np.array_equal(~np.isnan(o[0, :, :, 0]), written)
    np.testing.assert_allclose(o[0][written], np.broadcast_to(fvgen.bf16_to_f64(v[0, 0, 0]), (int(written.sum()), D)),
                               rtol=0, atol=1e-13)
