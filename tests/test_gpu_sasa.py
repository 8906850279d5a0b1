"""Slack-aware sparse augmentation on the GPU (MI355X): the augmented mask,
counts, head placement and XCD loads equal the oracle's exactly; attention
under the per-XCD schedule equals the stealing schedule bit for bit and stays
within max-abs 2e-2 / mean-abs 2e-3 of the oracle on the augmented mask."""
import math

import numpy as np
import pytest

import fvgen
import oracle

torch = pytest.importorskip("torch")
import adaptive_block_sparse_tile_amd as fva  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _wl(name, heads, grid, block, top_p, k_floor, D=64):
    taus = tuple(np.linspace(0.4, 5.0, heads))
    return fvgen.Workload(name, 61, heads, D, grid, block, 8, "list", taus, top_p, k_floor)


CASES = [_wl("h12", 12, (9, 17, 23), (4, 8, 8), 0.8, 2), _wl("h11_small", 11, (6, 8, 8), (2, 4, 4), 0.7, 3),
         fvgen.WORKLOADS["wan14b"], fvgen.WORKLOADS["720p"]]


def _gpu_sasa(wl, qd, kd, rounds, xcd_weight=None):
    shape = tuple(qd.shape)
    ws_r = fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), qd.device)
    mask, _, _ = fva.route(qd, kd, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r)
    mo, cnt, hx, load = fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=rounds, xcd_weight=xcd_weight)
    torch.cuda.synchronize()
    return mask, mo, cnt, hx, load


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_sasa_matches_oracle(wl):
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd = _dev(q), _dev(k)
    rounds = 4
    mask_g, mo_g, cnt_g, hx_g, load_g = _gpu_sasa(wl, qd, kd, rounds)
    S = oracle.scores(oracle.pool(q, wl.grid, wl.block), oracle.pool(k, wl.grid, wl.block))
    mask_o, _, rflags, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, margin=1e-10)
    mo, co, hx, load, added, sflags = oracle.sasa(S, mask_o, wl.grid, wl.block, rounds, margin=1e-10)
    print("\n[%s] loads %s added %s, rows flagged (route, sasa) %d %d" % (
        wl.name, load.tolist(), added.tolist(), int((rflags != 0).sum()), int(sflags.sum())), flush=True)
    assert not (rflags != 0).any() and not sflags.any()
    assert np.array_equal(mask_g.cpu().numpy().view(np.uint32), mask_o)
    assert np.array_equal(mo_g.cpu().numpy().view(np.uint32), mo)
    assert np.array_equal(cnt_g.cpu().numpy(), co)
    assert np.array_equal(hx_g.cpu().numpy(), hx)
    lg = load_g.cpu().numpy()
    assert np.array_equal(lg[:8], load) and np.array_equal(lg[8:], added)


W8 = [1000, 1040, 960, 1000, 1090, 920, 1010, 980]


def test_sasa_long_video_scores_recomputed_per_slab():
    """The long video's router holds its scores in 3 slabs, so the
    augmentation recomputes them slab by slab from the pooled means (the
    other cases read the router's single slab); in place (mask_out =
    mask_in), on measured-looking XCD weights."""
    wl = fvgen.WORKLOADS["long"]
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd = _dev(q), _dev(k)
    shape = tuple(qd.shape)
    W8 = [1000, 1040, 960, 1000, 1090, 920, 1010, 980]
    ws_r = fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), qd.device)
    mask, _, _ = fva.route(qd, kd, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r)
    cnt = torch.empty(mask.shape[:-1], dtype=torch.int32, device=qd.device)
    mo_g, cnt_g, hx_g, load_g = fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=2, xcd_weight=W8,
                                         out=(mask, cnt))
    torch.cuda.synchronize()
    S = oracle.scores(oracle.pool(q, wl.grid, wl.block), oracle.pool(k, wl.grid, wl.block))
    mask_o, _, rflags, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, margin=1e-10)
    mo, co, hx, load, added, sflags = oracle.sasa(S, mask_o, wl.grid, wl.block, 2, margin=1e-10, xcd_weight=W8)
    print("\n[long] loads %s added %s, rows flagged (route, sasa) %d %d" % (
        load.tolist(), added.tolist(), int((rflags != 0).sum()), int(sflags.sum())), flush=True)
    assert not (rflags != 0).any() and not sflags.any()
    assert mo_g.data_ptr() == mask.data_ptr()
    assert np.array_equal(mo_g.cpu().numpy().view(np.uint32), mo)
    assert np.array_equal(cnt_g.cpu().numpy(), co)
    assert np.array_equal(hx_g.cpu().numpy(), hx)
    lg = load_g.cpu().numpy()
    assert np.array_equal(lg[:8], load) and np.array_equal(lg[8:], added)
    assert added.sum() > 0


@pytest.mark.parametrize("wl", [CASES[0], CASES[2], CASES[3]], ids=lambda w: w.name)
def test_sasa_weighted_matches_oracle(wl):
    """XCDs of unequal speed (xcd_weight): mask, counts, placement and loads
    bit-exact against the oracle's weighted rule."""
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd = _dev(q), _dev(k)
    mask_g, mo_g, cnt_g, hx_g, load_g = _gpu_sasa(wl, qd, kd, 4, xcd_weight=W8)
    S = oracle.scores(oracle.pool(q, wl.grid, wl.block), oracle.pool(k, wl.grid, wl.block))
    mask_o, _, rflags, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, margin=1e-10)
    mo, co, hx, load, added, sflags = oracle.sasa(S, mask_o, wl.grid, wl.block, 4, margin=1e-10, xcd_weight=W8)
    print("\n[%s weighted] loads %s added %s" % (wl.name, load.tolist(), added.tolist()), flush=True)
    assert not (rflags != 0).any() and not sflags.any()
    assert np.array_equal(mo_g.cpu().numpy().view(np.uint32), mo)
    assert np.array_equal(cnt_g.cpu().numpy(), co)
    assert np.array_equal(hx_g.cpu().numpy(), hx)
    lg = load_g.cpu().numpy()
    assert np.array_equal(lg[:8], load) and np.array_equal(lg[8:], added)
    with pytest.raises(fva.FvaError, match="xcd_weight"):
        fva.sasa(tuple(qd.shape), wl.grid, wl.block, mask_g, fva.workspace(
            fva.route_workspace_bytes(tuple(qd.shape), wl.grid, wl.block), "cuda"), rounds=1, xcd_weight=[0] * 8)


@pytest.mark.parametrize("wl", [CASES[0], CASES[2]], ids=lambda w: w.name)
def test_xcd_schedule_and_attention(wl):
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    _, mo_g, _, hx_g, _ = _gpu_sasa(wl, qd, kd, 4)
    o_lpt = fva.sparse_attn(qd, kd, vd, wl.grid, wl.block, mo_g, sched="lpt")
    ws = fva.attn_plan(kd, vd, wl.grid, wl.block, mo_g, sched="xcd", head_xcd=hx_g)
    nwg = fva.attn_workgroups(tuple(qd.shape), wl.grid, wl.block)
    tr = torch.zeros(nwg * 4, dtype=torch.int64, device="cuda")
    o_xcd = fva.attn_exec(qd, wl.grid, wl.block, mo_g, ws, sched="xcd", trace=tr)
    o_x2 = fva.sparse_attn(qd, kd, vd, wl.grid, wl.block, mo_g, sched="xcd")
    torch.cuda.synchronize()
    assert torch.equal(o_lpt.view(torch.int16), o_xcd.view(torch.int16))
    assert torch.equal(o_lpt.view(torch.int16), o_x2.view(torch.int16))
    # every item ran exactly once
    t = tr.cpu().numpy().view(np.uint64).reshape(-1, 4)
    N = oracle.num_blocks(wl.grid, wl.block)
    items = int((t[:, 3] >> np.uint64(40)).sum())
    assert items > 0
    mask = mo_g.cpu().numpy().view(np.uint32)
    rng = np.random.default_rng(5)
    sel = np.array(sorted(set(rng.integers(wl.heads * N, size=12).tolist())))
    ref = oracle.attn(q, k, v, wl.grid, wl.block, mask, 1.0 / math.sqrt(wl.head_dim), items=sel)
    out = fvgen.bf16_to_f64(o_xcd.view(torch.int16).cpu().numpy().view(np.uint16))
    tb = oracle.token_block(wl.grid, wl.block)
    e = np.concatenate([np.abs(out[0, tb == (it % N), it // N] - ref[0, tb == (it % N), it // N]).reshape(-1)
                        for it in sel])
    print("\n[%s] xcd schedule on the augmented mask: max-abs %.3e mean-abs %.3e" % (wl.name, e.max(), e.mean()))
    assert np.isfinite(e).all() and e.max() <= 2e-2 and e.mean() <= 2e-3


def test_sasa_errors():
    wl = CASES[0]
    q, k, _ = fvgen.generate_qkv(wl)
    qd, kd = _dev(q), _dev(k)
    shape = tuple(qd.shape)
    ws_r = fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), qd.device)
    mask, _, _ = fva.route(qd, kd, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r)
    with pytest.raises(fva.FvaError, match="rounds 9 outside 0..8"):
        fva.sasa(shape, wl.grid, wl.block, mask, ws_r, rounds=9)
    with pytest.raises(fva.FvaError, match="route workspace holds"):
        fva.sasa(shape, wl.grid, wl.block, mask, ws_r[:1024], rounds=2)
