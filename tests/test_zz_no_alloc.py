"""The allocation-free router entry point (fva_route_noalloc, static
scratch) against fva_route with a caller workspace, through the raw C ABI:
two calls in a row on one GPU, the second on a smaller input, each bitwise
equal to fva_route's mask, counts and status."""
import ctypes

import numpy as np
import pytest

import fvgen

torch = pytest.importorskip("torch")
import adaptive_block_sparse_tile_amd as fva  # noqa: E402

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _outputs(B, heads, N):
    return (torch.full((B, heads, N, (N + 31) // 32), -1, dtype=torch.int32, device="cuda"),
            torch.full((B, heads, N), -1, dtype=torch.int32, device="cuda"),
            torch.full((1,), -1, dtype=torch.int32, device="cuda"))


def _call(fn_name, q, k, wl, out, ws=None):
    lib = fva.load()
    desc = fva.make_desc(*q.shape)
    grid = fva.make_grid(wl.grid, wl.block)
    cfg = fva.RouteCfg(float(wl.top_p), int(wl.k_floor))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [t.data_ptr() for t in out]
    if fn_name == "fva_route":
        rc = lib.fva_route(q.data_ptr(), k.data_ptr(), ctypes.byref(desc), ctypes.byref(grid), ctypes.byref(cfg),
                           *ptrs, ws.data_ptr(), ws.numel(), stream)
    else:
        rc = lib.fva_route_noalloc(q.data_ptr(), k.data_ptr(), ctypes.byref(desc), ctypes.byref(grid),
                                   ctypes.byref(cfg), *ptrs, stream)
    assert rc == 0, (fn_name, rc, lib.fva_last_error().decode())


def test_route_noalloc_matches_route_twice_second_smaller():
    # the long video first (pooled means 60 MiB: the score slab fills the
    # rest of the scratch, several slabs), then the 27280-token Wan layer on
    # the same scratch; a router row with a NaN query in the second input
    # checks that the status word starts from zero on every call
    cases = [fvgen.WORKLOADS["long"], fvgen.WORKLOADS["wan14b"]]
    for n, wl in enumerate(cases):
        q, k, _ = fvgen.generate_qkv(wl)
        if n == 1:
            q = q.copy()
            q[0, 5, 3, 7] = 0x7FC0
        qd, kd = _dev(q), _dev(k)
        B, L, heads, D = qd.shape
        N = fva.num_blocks(wl.grid, wl.block)
        ws = fva.workspace(fva.route_workspace_bytes(tuple(qd.shape), wl.grid, wl.block), "cuda")
        ref = _outputs(B, heads, N)
        _call("fva_route", qd, kd, wl, ref, ws)
        got = _outputs(B, heads, N)
        print("\n[noalloc %s] call %d: B=%d heads=%d N=%d" % (wl.name, n + 1, B, heads, N), flush=True)
        _call("fva_route_noalloc", qd, kd, wl, got)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        assert int(got[2].cpu()[0]) == (1 if n == 1 else 0)
        del ws


def test_route_noalloc_rejects_oversize_shape():
    wl = fvgen.WORKLOADS["tiny"]
    lib = fva.load()
    q = torch.zeros(16, dtype=torch.bfloat16, device="cuda")      # never read: rejected on the host
    out = _outputs(1, 1, 1)
    desc = fva.make_desc(1, 393216, 40, 128)
    grid = fva.make_grid((96, 64, 64), (4, 4, 4))
    cfg = fva.RouteCfg(0.85, 32)
    rc = lib.fva_route_noalloc(q.data_ptr(), q.data_ptr(), ctypes.byref(desc), ctypes.byref(grid), ctypes.byref(cfg),
                               out[0].data_ptr(), None, None, None)
    assert rc == 6 and "static scratch" in lib.fva_last_error().decode()
    assert wl.name == "tiny"
