"""The whole layer in one call (fva_routed_attn), on one stream and
pipelined over head groups on two streams (MI355X).

Every `groups` and stream choice must give the bits fva_route followed by
fva_sparse_attn give (mask, counts, status, O); the layer's attention is
checked against the fp64 oracle on the GPU's own mask, and its mask against
the oracle's router."""
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


def _reference(wl, qd, kd, vd):
    mask, cnt, st = fva.route(qd, kd, wl.grid, wl.block, wl.top_p, wl.k_floor)
    o = fva.sparse_attn(qd, kd, vd, wl.grid, wl.block, mask)
    torch.cuda.synchronize()
    return o.view(torch.int16).clone(), mask, cnt, st


def _same(a, b):
    return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


CASES = [
    ("tiny", None),
    ("wan14b", None),
    # B = 2, grouped 64-token blocks, D = 64, 5 heads (uneven groups of 1 and 2 heads)
    ("b2_grouped", fvgen.Workload("b2_grouped", 79, 5, 64, (8, 12, 20), (4, 4, 4), 8, "list",
                                  (0.6, 1.2, 2.5, 4.0, 6.0), 0.85, 3, batch=2)),
]


@pytest.mark.parametrize("name,custom", CASES, ids=[c[0] for c in CASES])
def test_routed_attn_bitwise_equal_to_route_then_sparse(name, custom):
    wl = custom or fvgen.WORKLOADS[name]
    q, k, v = fvgen.generate_qkv(wl)
    if name == "wan14b":
        q = q.copy()
        q[0, 100, 27, 5] = 0x7FC0     # a NaN in head 27: a side-stream group must report it
    qd, kd, vd = (_dev(a) for a in (q, k, v))
    ref = _reference(wl, qd, kd, vd)
    side = torch.cuda.Stream()
    for groups in sorted(g for g in {1, 2, 3, 5, wl.heads} if g <= wl.heads):
        for s in ((None, side) if groups > 1 else (None,)):
            for rep in range(2):
                got = fva.routed_attn(qd, kd, vd, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups,
                                      side_stream=s)
                torch.cuda.synchronize()
                assert _same(got, ref), (name, groups, s is not None, rep)
        print("\n[%s] groups %d: one stream and two streams bitwise equal to route + sparse_attn" % (name, groups),
              flush=True)
    assert int(ref[3].cpu()[0]) == (1 if name == "wan14b" else 0)


def test_routed_attn_long_video_one_head_per_group():
    wl = fvgen.WORKLOADS["long"]
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd, vd = (_dev(a) for a in (q, k, v))
    ref = _reference(wl, qd, kd, vd)
    side = torch.cuda.Stream()
    got = fva.routed_attn(qd, kd, vd, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=5, side_stream=side)
    torch.cuda.synchronize()
    assert _same(got, ref)


def test_routed_attn_against_the_oracle():
    """Pipelined over 3 groups on two streams: the mask bit-exact against the
    oracle's router on every unflagged row, and O within max-abs 2e-2 /
    mean-abs 2e-3 of the fp64 oracle on the GPU's mask, every query block."""
    wl = fvgen.Workload("routed_oracle", 80, 6, 128, (9, 17, 23), (4, 8, 8), 8, "list",
                        (0.4, 1.0, 2.0, 3.0, 4.5, 6.0), 0.9, 3)
    q, k, v = fvgen.generate_qkv(wl)
    qd, kd, vd = (_dev(a) for a in (q, k, v))
    o, mask, cnt, st = fva.routed_attn(qd, kd, vd, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=3,
                                       side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    mg = mask.cpu().numpy().view(np.uint32)
    mo, co, flags, so = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    ok = flags == 0
    assert int(st.cpu()[0]) == so == 0 and ok.mean() > 0.9
    assert not ((mg != mo).any(-1) & ok).any() and np.array_equal(cnt.cpu().numpy()[ok], co[ok])
    ref = oracle.attn_matmul(q, k, v, wl.grid, wl.block, mg, 1.0 / math.sqrt(wl.head_dim))
    og = fvgen.bf16_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    e = np.abs(og - ref)
    print("\n[routed_oracle] groups 3 on two streams: max-abs %.3e mean-abs %.3e" % (e.max(), e.mean()), flush=True)
    assert np.isfinite(e).all() and e.max() <= 2e-2 and e.mean() <= 2e-3
