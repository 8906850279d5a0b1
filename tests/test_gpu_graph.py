"""The layer captured once in a HIP graph and replayed (MI355X).

The library's calls enqueue kernels and event waits only (no memset or
allocation nodes, no host synchronisation), so a caller can capture a whole
layer -- router, plan, attention, or the whole-layer call with its second
stream -- and replay it.  Each replay, with eager work and synchronisations
between the replays, must give the bits the eager calls give."""
import numpy as np
import pytest

import fvgen

torch = pytest.importorskip("torch")
import adaptive_block_sparse_tile_amd as fva  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _outputs(wl, q):
    B, L, heads, D = q.shape
    N = fva.num_blocks(wl.grid, wl.block)
    return (torch.empty_like(q), torch.empty((B, heads, N, (N + 31) // 32), dtype=torch.int32, device=q.device),
            torch.empty((B, heads, N), dtype=torch.int32, device=q.device),
            torch.empty((1,), dtype=torch.int32, device=q.device))


def _replay_and_check(g, outs, ref, other):
    """Three replays; before each, the outputs are cleared and an unrelated
    eager layer runs; after each, a synchronisation and a bitwise check."""
    for _ in range(3):
        for t in outs:
            t.zero_()
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want)


@pytest.mark.parametrize("name", ["tiny", "wan14b", "long"])
def test_route_plan_exec_graph_equals_eager(name):
    wl = fvgen.WORKLOADS[name]
    q, k, v = (_dev(a) for a in fvgen.generate_qkv(wl))
    shape = tuple(q.shape)
    ws_r = fva.workspace(fva.route_workspace_bytes(shape, wl.grid, wl.block), q.device)
    ws_a = fva.workspace(fva.attn_workspace_bytes(shape, wl.grid, wl.block), q.device)
    o, mask, cnt, status = outs = _outputs(wl, q)

    def layer(s):
        fva.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor, ws=ws_r, out=(mask, cnt, status), stream=s)
        fva.attn_plan(k, v, wl.grid, wl.block, mask, ws=ws_a, stream=s)
        fva.attn_exec(q, wl.grid, wl.block, mask, ws_a, out=o, stream=s)

    main = torch.cuda.current_stream()
    layer(main)
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in outs)
    side = torch.cuda.Stream()
    side.wait_stream(main)
    layer(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layer(side)
    torch.cuda.synchronize()
    # eager work between replays: the same calls on reversed inputs, into other buffers
    q2, k2, v2 = (t.flip(1).contiguous() for t in (q, k, v))
    o2 = torch.empty_like(q)

    def other():
        m2, _, _ = fva.route(q2, k2, wl.grid, wl.block, wl.top_p, wl.k_floor)
        fva.sparse_attn(q2, k2, v2, wl.grid, wl.block, m2, out=o2)

    _replay_and_check(g, outs, ref, other)


@pytest.mark.parametrize("groups", [1, 2])
def test_routed_attn_graph_equals_eager(groups):
    """The whole-layer call, with groups = 2 forking to a second stream and
    joining back inside the capture."""
    wl = fvgen.WORKLOADS["wan5b"]
    q, k, v = (_dev(a) for a in fvgen.generate_qkv(wl))
    shape = tuple(q.shape)
    ws = fva.workspace(fva.routed_attn_workspace_bytes(shape, wl.grid, wl.block, groups), q.device)
    outs = _outputs(wl, q)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    cap = torch.cuda.Stream()
    fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups,
                    side_stream=side if groups > 1 else None, ws=ws, out=outs)
    torch.cuda.synchronize()
    ref = tuple(t.clone() for t in outs)
    cap.wait_stream(main)
    with torch.cuda.stream(cap):
        fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups,
                        side_stream=side if groups > 1 else None, ws=ws, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        fva.routed_attn(q, k, v, wl.grid, wl.block, wl.top_p, wl.k_floor, groups=groups,
                        side_stream=side if groups > 1 else None, ws=ws, out=outs)
    torch.cuda.synchronize()
    o2 = torch.empty_like(q)

    def other():
        m2, _, _ = fva.route(k, q, wl.grid, wl.block, wl.top_p, wl.k_floor)
        fva.sparse_attn(k, q, v, wl.grid, wl.block, m2, out=o2)

    _replay_and_check(g, outs, ref, other)
