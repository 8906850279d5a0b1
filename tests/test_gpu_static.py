"""Static local + anchor block masks on the GPU (MI355X): the mask kernel bit
for bit against the oracle, and block-sparse attention on those masks within
max-abs 2e-2 / mean-abs 2e-3 of the fp64 oracle."""
import math

import numpy as np
import pytest

import fvgen
import oracle

torch = pytest.importorskip("torch")
import adaptive_block_sparse_tile_amd as fva  # noqa: E402

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("grid,block,local,anchor_t", [
    ((8, 16, 16), (4, 8, 8), (1, 1, 1), 0),
    ((8, 16, 16), (4, 8, 8), (2, 2, 2), 0),
    ((9, 17, 23), (4, 8, 8), (2, 1, 2), 2),
    ((31, 22, 40), (4, 8, 8), (2, 3, 5), 4),
    ((12, 16, 24), (2, 2, 2), (2, 4, 4), 3),       # N = 576 > 512
    ((96, 64, 64), (4, 4, 4), (2, 16, 16), 6),     # N = 6144, the static workload
    ((64, 1, 1), (1, 1, 1), (8, 1, 1), 16),        # one-token blocks: the token-level rule
])
def test_static_mask_bit_exact(grid, block, local, anchor_t):
    L = grid[0] * grid[1] * grid[2]
    shape = (1, L, 2, 64)
    mask_g, cnt_g = fva.static_mask(shape, grid, block, local=local, anchor_t=anchor_t)
    torch.cuda.synchronize()
    mo, co = oracle.static_mask(grid, block, local, anchor_t, B=1, heads=2)
    assert np.array_equal(mask_g.cpu().numpy().view(np.uint32), mo)
    assert np.array_equal(cnt_g.cpu().numpy(), co)


def test_static_mask_errors():
    with pytest.raises(fva.FvaError, match="local box 0 x 1 x 1"):
        fva.static_mask((1, 2048, 2, 64), (8, 16, 16), (4, 8, 8), local=(0, 1, 1))
    with pytest.raises(fva.FvaError, match="anchor_t -1 < 0"):
        fva.static_mask((1, 2048, 2, 64), (8, 16, 16), (4, 8, 8), anchor_t=-1)


def _wl(name, heads, D, grid, block, static):
    taus = tuple([0.7, 2.5, 5.0][:heads])
    return fvgen.Workload(name, 91, heads, D, grid, block, 8, "list", taus, 0.0, 1, static=static)


@pytest.mark.parametrize("wl", [
    _wl("static_small", 2, 128, (9, 17, 23), (4, 8, 8), ((2, 1, 2), 2)),
    _wl("static_d64_ragged", 3, 64, (10, 12, 13), (4, 4, 4), ((2, 2, 1), 3)),
], ids=lambda w: w.name)
def test_static_attention_parity(wl):
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    mask_g, _ = fva.static_mask(tuple(qd.shape), wl.grid, wl.block, local=wl.static[0], anchor_t=wl.static[1])
    o = fva.sparse_attn(qd, kd, vd, wl.grid, wl.block, mask_g)
    torch.cuda.synchronize()
    mask = mask_g.cpu().numpy().view(np.uint32)
    ref = oracle.attn(q, k, v, wl.grid, wl.block, mask, 1.0 / math.sqrt(wl.head_dim))
    out = fvgen.bf16_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    e = np.abs(out - ref)
    print("\n[%s] max-abs %.3e mean-abs %.3e" % (wl.name, e.max(), e.mean()), flush=True)
    assert np.isfinite(e).all() and e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_static_workload_sampled_items():
    wl = fvgen.WORKLOADS["static"]
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    mask_g, cnt_g = fva.static_mask(tuple(qd.shape), wl.grid, wl.block, local=wl.static[0], anchor_t=wl.static[1])
    o = fva.sparse_attn(qd, kd, vd, wl.grid, wl.block, mask_g)
    torch.cuda.synchronize()
    mask = mask_g.cpu().numpy().view(np.uint32)
    N = oracle.num_blocks(wl.grid, wl.block)
    cnt = cnt_g.cpu().numpy().reshape(-1)
    rng = np.random.default_rng(3)
    # anchor rows (dense), the lightest rows, grid corners and a seeded random set
    items = {int(np.argmax(cnt)), int(np.argmin(cnt)), 0, N - 1, 4 * N + N // 2}
    while len(items) < 24:
        items.add(int(rng.integers(cnt.size)))
    items = np.array(sorted(items))
    ref = oracle.attn(q, k, v, wl.grid, wl.block, mask, 1.0 / math.sqrt(wl.head_dim), items=items)
    out = fvgen.bf16_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    tb = oracle.token_block(wl.grid, wl.block)
    errs = []
    for it in items:
        i, h = it % N, it // N
        toks = np.nonzero(tb == i)[0]
        errs.append(np.abs(out[0, toks, h] - ref[0, toks, h]).reshape(-1))
    e = np.concatenate(errs)
    print("\n[static] %d items: max-abs %.3e mean-abs %.3e" % (len(items), e.max(), e.mean()), flush=True)
    assert np.isfinite(e).all() and e.max() <= MAX_ABS and e.mean() <= MEAN_ABS
