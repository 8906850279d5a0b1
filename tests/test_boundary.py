"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before touching
the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import adaptive_block_sparse_tile_amd as fva

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fva.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fva.LIB_PATH), reason="libfva.so not built")

FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fva_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(fva.EXPORTS)


def test_exports_every_declared_symbol():
    lib = fva.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_num_blocks():
    assert fva.num_blocks((31, 22, 40), (4, 8, 8)) == 120
    assert fva.num_blocks((21, 45, 80), (4, 8, 8)) == 360
    assert fva.num_blocks((96, 64, 64), (4, 4, 4)) == 6144
    assert fva.num_blocks((8, 16, 16), (4, 8, 8)) == 8
    assert fva.num_blocks((0, 16, 16), (4, 8, 8)) == -1


def test_workspace_sizes():
    shape = (1, 27280, 40, 128)
    r = fva.route_workspace_bytes(shape, (31, 22, 40), (4, 8, 8))
    rows = 40 * 120
    assert r >= 2 * rows * 128 * 8 + rows * 120 * 8
    # long video: pooled means plus one score slab of 512 MiB (170 tiles of 64 x 6144 fp64), not 30720 x 6144
    rl = fva.route_workspace_bytes((1, 393216, 5, 128), (96, 64, 64), (4, 4, 4))
    assert rl == 2 * 5 * 6144 * 128 * 8 + 170 * 64 * 6144 * 8
    a = fva.attn_workspace_bytes(shape, (31, 22, 40), (4, 8, 8))
    assert a >= 27280 * 4 + rows * (8 + 4 + 4)
    assert fva.route_workspace_bytes((1, 27281, 40, 128), (31, 22, 40), (4, 8, 8)) == 0   # T*H*W != L


def _route(desc, grid, cfg, ws_bytes=1 << 30, ws=FAKE, mask=FAKE):
    lib = fva.load()
    return lib.fva_route(FAKE, FAKE, ctypes.byref(desc), ctypes.byref(grid), ctypes.byref(cfg), mask, None, None,
                         ws, ws_bytes, None)


def _err():
    return fva.load().fva_last_error().decode()


def test_route_validation_errors():
    desc = fva.make_desc(1, 27280, 40, 128)
    grid = fva.make_grid((31, 22, 40), (4, 8, 8))
    assert _route(desc, grid, fva.RouteCfg(0.9, 130)) == 3
    assert _err() == "k_floor 130 > num_blocks 120"
    assert _route(desc, grid, fva.RouteCfg(0.9, 0)) == 3
    assert _route(desc, grid, fva.RouteCfg(float("nan"), 8)) == 1
    assert _route(fva.make_desc(1, 27281, 40, 128), grid, fva.RouteCfg(0.9, 8)) == 2
    assert _route(fva.make_desc(1, 27280, 40, 96), grid, fva.RouteCfg(0.9, 8)) == 6
    assert _route(desc, fva.make_grid((31, 22, 40), (4, 8, 16)), fva.RouteCfg(0.9, 8)) == 6
    assert _route(desc, grid, fva.RouteCfg(0.9, 8), ws_bytes=16) == 5
    assert _route(desc, grid, fva.RouteCfg(0.9, 8), ws=ctypes.c_void_p(0x10010)) == 5   # misaligned
    assert _route(desc, grid, fva.RouteCfg(0.9, 8), ws=None) == 5
    assert _route(desc, grid, fva.RouteCfg(0.9, 8), mask=None) == 1
    # long video with 2x2x2 blocks: 48*32*32 = 49152 blocks > 8192
    assert _route(fva.make_desc(1, 393216, 5, 128), fva.make_grid((96, 64, 64), (2, 2, 2)),
                  fva.RouteCfg(0.9, 8)) == 6


def test_attn_validation_errors():
    lib = fva.load()
    desc = fva.make_desc(1, 27280, 40, 128)
    grid = fva.make_grid((31, 22, 40), (4, 8, 8))

    def call(scale=128 ** -0.5, sched=0, ws_bytes=1 << 30, desc=desc):
        return lib.fva_sparse_attn(FAKE, FAKE, FAKE, FAKE, ctypes.byref(desc), ctypes.byref(grid), FAKE, scale,
                                   sched, None, FAKE, ws_bytes, None)

    assert call(scale=0.088) == 4
    assert "head_dim^-0.5" in _err()
    assert call(sched=7) == 1
    assert call(ws_bytes=100) == 5
    assert call(desc=fva.make_desc(1, 100, 40, 128)) == 2
    # more than 8192 blocks: (132, 64, 64) in (4, 4, 4) tiles is 33 * 16 * 16 = 8448
    big_desc, big_grid = fva.make_desc(1, 132 * 64 * 64, 1, 64), fva.make_grid((132, 64, 64), (4, 4, 4))
    assert lib.fva_sparse_attn(FAKE, FAKE, FAKE, FAKE, ctypes.byref(big_desc), ctypes.byref(big_grid), FAKE,
                               64 ** -0.5, 0, None, FAKE, 1 << 40, None) == 6
    assert "num_blocks 8448 > 8192" in _err()
    assert lib.fva_attn_plan(FAKE, FAKE, ctypes.byref(big_desc), ctypes.byref(big_grid), FAKE, 0, None, FAKE,
                             1 << 40, None) == 6
    need = lib.fva_dense_workspace_bytes(ctypes.byref(desc))
    # 40 heads x ceil(27280 / 64) = 427 chunk images of 32,768 bytes (64 keys x 128 x bf16, K and V)
    assert need == 40 * 427 * 32768
    good = 128 ** -0.5

    def dense(o=FAKE, scale=good, ws=FAKE, ws_bytes=need):
        return lib.fva_dense_attn_ref(FAKE, FAKE, FAKE, o, ctypes.byref(desc), ctypes.c_float(scale), ws, ws_bytes,
                                      None)
    assert dense(scale=0.1) == 4
    assert dense(o=None) == 1
    assert dense(ws=None) == 5
    assert dense(ws_bytes=need - 1) == 5
    assert "workspace" in _err()


def test_status_names():
    lib = fva.load()
    for i, n in enumerate(fva.STATUS_NAMES):
        assert lib.fva_status_name(i).decode() == n


def test_trace_imbalance_host_helper():
    import numpy as np
    # 4 workgroups on 2 CUs (cu_id 0 and 1): busy 10+10 and 20+0 -> max/mean = 20/20 = 1
    def rec(t0, t1, busy, cu, items=1):
        return [t0, t1, busy, (items << 40) | (cu << 8)]
    t = np.array([rec(0, 10, 10, 0), rec(0, 10, 10, 0), rec(0, 20, 20, 1), rec(0, 0, 0, 1, items=0)],
                 dtype=np.uint64)
    b, f, n = fva.trace_imbalance(t)
    assert n == 2 and abs(b - 1.0) < 1e-12 and abs(f - 20 / 15) < 1e-12


def test_attn_items_and_schedule_validation():
    lib = fva.load()
    # one item per block for 256-token blocks; 2x1x2 groups of 64-token blocks; 1x1x2 of 128-token blocks
    assert fva.attn_items((1, 27280, 40, 128), (31, 22, 40), (4, 8, 8)) == 40 * 120
    assert fva.attn_items((1, 393216, 5, 128), (96, 64, 64), (4, 4, 4)) == 5 * 12 * 16 * 8
    assert fva.attn_items((2, 3840, 3, 64), (6, 16, 40), (2, 8, 8)) == 2 * 3 * 3 * 2 * 3
    assert fva.attn_items((1, 7 * 6 * 5, 2, 64), (7, 6, 5), (2, 2, 2)) == 2 * 2 * 3 * 2
    bad = fva.make_desc(1, 27281, 40, 128)
    assert lib.fva_attn_items(ctypes.byref(bad), ctypes.byref(fva.make_grid((31, 22, 40), (4, 8, 8)))) == -1
    desc, grid = fva.make_desc(1, 27280, 40, 128), fva.make_grid((31, 22, 40), (4, 8, 8))
    need = lib.fva_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(grid))

    def call(ws=FAKE, ws_bytes=need, order=FAKE, qoff=FAKE, desc=desc):
        return lib.fva_attn_schedule(ctypes.byref(desc), ctypes.byref(grid), ws, ws_bytes, order, qoff, None, None)

    assert call(order=None) == 1 and "must not be null" in _err()
    assert call(qoff=None) == 1
    assert call(ws_bytes=need - 1) == 5 and "needed" in _err()
    assert call(ws=None) == 5
    assert call(desc=bad) == 2


def test_launch_size_limits():
    """Shapes inside the accepted ranges whose kernel grids would pass 2^32
    threads, or whose B*heads passes 4096, are rejected on the host."""
    lib = fva.load()
    grid8k = fva.make_grid((128, 64, 64), (4, 4, 4))      # 8192 blocks of 64 tokens
    L8k = 128 * 64 * 64
    # B*heads > 4096, for every entry point that takes a shape
    many = fva.make_desc(1, L8k, 4097, 64)
    assert _route(many, grid8k, fva.RouteCfg(0.9, 8), ws_bytes=1 << 62) == 6 and "B*heads = 4097" in _err()
    assert lib.fva_static_mask(ctypes.byref(many), ctypes.byref(grid8k), ctypes.byref(fva.StaticCfg(1, 1, 1, 0)),
                               FAKE, None, None) == 6
    assert lib.fva_dense_attn_ref(FAKE, FAKE, FAKE, FAKE, ctypes.byref(many), ctypes.c_float(0.125), FAKE,
                                  1 << 62, None) == 6
    # 2048 heads of 8192 blocks: 16.7M chunk images of 256 threads; the router
    # routes one slab of rows per launch, so it only runs out of workspace
    wide = fva.make_desc(1, L8k, 2048, 64)
    assert lib.fva_sparse_attn(FAKE, FAKE, FAKE, FAKE, ctypes.byref(wide), ctypes.byref(grid8k), FAKE, 0.125, 0,
                               None, FAKE, 1 << 62, None) == 6 and "chunk tiling" in _err()
    assert _route(wide, grid8k, fva.RouteCfg(0.9, 8), ws_bytes=16) == 5
    # one fewer head fits the tiling launch (it then fails only on the workspace size)
    ok = fva.make_desc(1, L8k, 2047, 64)
    assert lib.fva_sparse_attn(FAKE, FAKE, FAKE, FAKE, ctypes.byref(ok), ctypes.byref(grid8k), FAKE, 0.125, 0,
                               None, FAKE, 16, None) == 5
    # dense reference: 4096 heads of 2^24 - 1 tokens is 1.07e9 chunk images
    long_desc = fva.make_desc(1, (1 << 24) - 1, 4096, 64)
    assert lib.fva_dense_attn_ref(FAKE, FAKE, FAKE, FAKE, ctypes.byref(long_desc), ctypes.c_float(0.125), FAKE,
                                  1 << 62, None) == 6


def test_binding_allocates_on_the_call_stream(monkeypatch):
    """The binding runs each call with its `stream` as torch's current stream
    (so outputs and the temporary workspace belong to the stream the kernels
    use); without a stream it leaves the current stream alone."""
    import contextlib
    import types

    entered = []

    @contextlib.contextmanager
    def fake_stream(s):
        entered.append(s)
        yield

    fake = types.SimpleNamespace(cuda=types.SimpleNamespace(stream=fake_stream))
    monkeypatch.setattr(fva, "_torch", lambda: fake)

    @fva._on_stream
    def call(a, b=None, stream=None):
        return (a, b, list(entered))

    assert call(1) == (1, None, [])
    assert call(1, 2, "side") == (1, 2, ["side"])
    assert call(1, stream="other") == (1, None, ["side", "other"])
    for name in ("route", "sparse_attn", "static_mask", "attn_plan", "attn_exec", "attn_schedule", "sasa",
                 "dense_attn_ref"):
        assert getattr(fva, name).__wrapped__ is not None, name


def test_route_noalloc_host_validation():
    """The allocation-free router rejects on the host, before any device call,
    what fva_route rejects, and shapes whose pooled means leave no room for
    one tile of scores in its static scratch."""
    lib = fva.load()

    def call(desc, grid, cfg, mask=FAKE):
        return lib.fva_route_noalloc(FAKE, FAKE, ctypes.byref(desc), ctypes.byref(grid), ctypes.byref(cfg), mask,
                                     None, None, None)
    desc = fva.make_desc(1, 27280, 40, 128)
    grid = fva.make_grid((31, 22, 40), (4, 8, 8))
    assert call(desc, grid, fva.RouteCfg(0.9, 130)) == 3 and _err() == "k_floor 130 > num_blocks 120"
    assert call(desc, grid, fva.RouteCfg(0.9, 8), mask=None) == 1
    assert call(fva.make_desc(1, 27281, 40, 128), grid, fva.RouteCfg(0.9, 8)) == 2
    # 40 heads of 6144 blocks: 2 * 40 * 6144 * 128 * 8 bytes of pooled means > 128 MiB
    big = fva.make_desc(1, 393216, 40, 128)
    assert call(big, fva.make_grid((96, 64, 64), (4, 4, 4)), fva.RouteCfg(0.85, 32)) == 6
    assert "static scratch" in _err()
    assert fva.ROUTE_SCRATCH_BYTES == 128 << 20


def test_routed_attn_host_validation_and_workspace():
    lib = fva.load()
    desc = fva.make_desc(1, 27280, 40, 128)
    grid = fva.make_grid((31, 22, 40), (4, 8, 8))
    one = lib.fva_routed_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(grid), 1)
    assert one == fva.route_workspace_bytes((1, 27280, 40, 128), (31, 22, 40), (4, 8, 8)) + \
        fva.attn_workspace_bytes((1, 27280, 40, 128), (31, 22, 40), (4, 8, 8))
    # two streams' sets, each for the largest group (14 of 40 heads in 3 groups)
    three = lib.fva_routed_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(grid), 3)
    assert three == 2 * (fva.route_workspace_bytes((1, 27280, 14, 128), (31, 22, 40), (4, 8, 8)) +
                         fva.attn_workspace_bytes((1, 27280, 14, 128), (31, 22, 40), (4, 8, 8)))
    assert lib.fva_routed_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(grid), 41) == 0

    def call(groups=2, cfg=fva.RouteCfg(0.9, 8), scale=128 ** -0.5, ws_bytes=1 << 40, side=FAKE, o=FAKE):
        return lib.fva_routed_attn(FAKE, FAKE, FAKE, o, ctypes.byref(desc), ctypes.byref(grid), ctypes.byref(cfg),
                                   scale, groups, FAKE, None, None, FAKE, ws_bytes, None, side)
    assert call(groups=0) == 1 and "groups 0" in _err()
    assert call(groups=41) == 1
    assert call(cfg=fva.RouteCfg(0.9, 121)) == 3
    assert call(scale=0.1) == 4
    assert call(o=None) == 1
    assert call(ws_bytes=three - 1, groups=3) == 5 and "needed" in _err()
    # one stream: one set suffices, so a two-set workspace minus a byte still covers it
    assert call(ws_bytes=three // 2 - 1, groups=3, side=None) == 5


def test_trace_xcd_speed_host_helper():
    import numpy as np
    # 16 workgroups, 2 per XCD; XCD x does load 1000*(x+1) in busy time 10*(x+1)*(1 + x/100) ticks
    recs = []
    for x in range(8):
        busy = 10.0 * (x + 1) * (1 + x / 100.0) * 1000
        for _ in range(2):
            recs.append([0, 1, int(busy / 2), (1 << 40) | (x << 32)])
    t = np.array(recs, dtype=np.uint64)
    load = np.array([1000 * (x + 1) for x in range(8)], dtype=np.int64)
    w = fva.xcd_speed(t, load)
    speed = np.array([1.0 / (1 + x / 100.0) for x in range(8)])
    assert w.tolist() == np.round(1000 * speed / speed.mean()).astype(int).tolist()
    load[3] = 0
    with pytest.raises(fva.FvaError, match="XCD 3 has no measured work"):
        fva.xcd_speed(t, load)
