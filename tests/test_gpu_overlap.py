"""Routing and planning on a second stream, overlapped with attention on the
main stream (MI355X).

The heads split into two groups held as separate contiguous tensors (the
one-GPU form of the FVAttn abstract's overlap of routing with attention):
group 0 is routed and planned on the main stream, group 1 on a side stream
while the main stream runs group 0's attention; events order each group's
attention after its plan.  Checked: three overlapped passes in a row are
bitwise equal to a pass with everything on the main stream, and each group's
output matches the fp64 oracle on that group's GPU mask."""
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


def test_route_and_plan_on_side_stream():
    wl = fvgen.Workload("overlap4", 78, 4, 128, (9, 17, 23), (4, 8, 8), 8, "list", (0.5, 1.5, 3.0, 5.0), 0.8, 2)
    q, k, v = fvgen.generate_qkv(wl)
    G, hg = 2, 2
    qs, ks, vs = ([_dev(x[:, :, g * hg:(g + 1) * hg]) for g in range(G)] for x in (q, k, v))
    shape = tuple(qs[0].shape)
    B = shape[0]
    N = fva.num_blocks(wl.grid, wl.block)
    words = (N + 31) // 32
    masks = [torch.empty((B, hg, N, words), dtype=torch.int32, device="cuda") for _ in range(G)]
    cnts = [torch.empty((B, hg, N), dtype=torch.int32, device="cuda") for _ in range(G)]
    sts = [torch.empty((1,), dtype=torch.int32, device="cuda") for _ in range(G)]
    wsr = [fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), "cuda") for _ in range(G)]
    wsa = [fva.workspace(fva.attn_workspace_bytes(shape, wl.grid, wl.block), "cuda") for _ in range(G)]
    outs = [torch.empty_like(x) for x in qs]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def prep(g, s):
        fva.route(qs[g], ks[g], wl.grid, wl.block, wl.top_p, wl.k_floor, ws=wsr[g], out=(masks[g], cnts[g], sts[g]),
                  stream=s)
        fva.attn_plan(ks[g], vs[g], wl.grid, wl.block, masks[g], ws=wsa[g], stream=s)

    for g in range(G):
        prep(g, main)
        fva.attn_exec(qs[g], wl.grid, wl.block, masks[g], wsa[g], out=outs[g], stream=main)
    torch.cuda.synchronize()
    ref = [o.view(torch.int16).clone() for o in outs]
    ref_masks = [m.clone() for m in masks]

    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        side.wait_stream(main)
        ev = []
        for g in range(G):
            s = main if g == 0 else side
            prep(g, s)
            e = torch.cuda.Event()
            e.record(s)
            ev.append(e)
        for g in range(G):
            main.wait_event(ev[g])
            fva.attn_exec(qs[g], wl.grid, wl.block, masks[g], wsa[g], out=outs[g], stream=main)
        side.wait_stream(main)
        torch.cuda.synchronize()
        print("\n[overlap4] pass %d" % rep, flush=True)
        for g in range(G):
            assert torch.equal(masks[g], ref_masks[g])
            assert torch.equal(outs[g].view(torch.int16), ref[g])

    scale = 1.0 / math.sqrt(wl.head_dim)
    for g in range(G):
        sl = slice(g * hg, (g + 1) * hg)
        mask = masks[g].cpu().numpy().view(np.uint32)
        assert int(sts[g].cpu()[0]) == 0
        o = fvgen.bf16_to_f64(outs[g].view(torch.int16).cpu().numpy().view(np.uint16))
        o_ref = oracle.attn(q[:, :, sl], k[:, :, sl], v[:, :, sl], wl.grid, wl.block, mask, scale)
        e = np.abs(o - o_ref)
        assert np.isfinite(e).all() and e.max() <= 2e-2 and e.mean() <= 2e-3
