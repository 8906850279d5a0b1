"""Routed block-sparse attention for video DiTs on MI355X -- Python binding.

Thin ctypes marshalling over libfva.so (include/fva.h).  Every step of the
path runs in the library's HIP kernels; torch provides device memory and the
current stream only.  There is no CPU or eager fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import inspect
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# FVA_LIB: another build of the same sources (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("FVA_LIB") or os.path.join(_HERE, "libfva.so")

FVA_OK = 0
STATUS_NAMES = ["FVA_OK", "FVA_ERR_INVALID_ARG", "FVA_ERR_SHAPE", "FVA_ERR_TOPK", "FVA_ERR_SCALE",
                "FVA_ERR_WORKSPACE", "FVA_ERR_UNSUPPORTED", "FVA_ERR_DEVICE"]
ROUTE_SCRATCH_BYTES = 128 << 20   # FVA_ROUTE_SCRATCH_BYTES: the static scratch of fva_route_noalloc per GPU
SCHED_LPT = 0
SCHED_NAIVE = 1
SCHED_XCD = 2
SCHEDS = {"lpt": SCHED_LPT, "naive": SCHED_NAIVE, "xcd": SCHED_XCD}

# every symbol include/fva.h declares
EXPORTS = ["fva_num_blocks", "fva_route_workspace_bytes", "fva_attn_workspace_bytes", "fva_attn_workgroups",
           "fva_route", "fva_route_noalloc", "fva_static_mask", "fva_sparse_attn", "fva_attn_plan", "fva_attn_exec", "fva_routed_attn_workspace_bytes", "fva_routed_attn", "fva_attn_items",
           "fva_attn_schedule", "fva_sasa_workspace_bytes", "fva_sasa",
           "fva_dense_workspace_bytes", "fva_dense_attn_ref",
           "fva_trace_imbalance", "fva_trace_xcd_speed", "fva_last_error", "fva_status_name"]


class FvaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s: %s" % (self.name, detail))


class Grid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("bt", ctypes.c_int32), ("bh", ctypes.c_int32), ("bw", ctypes.c_int32)]


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("L", ctypes.c_int32), ("heads", ctypes.c_int32), ("D", ctypes.c_int32)]


class RouteCfg(ctypes.Structure):
    _fields_ = [("top_p", ctypes.c_float), ("k_floor", ctypes.c_int32)]


class StaticCfg(ctypes.Structure):
    _fields_ = [("lt", ctypes.c_int32), ("lh", ctypes.c_int32), ("lw", ctypes.c_int32), ("anchor_t", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def load():
    """Load libfva.so (built in-tree by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfva.so is not built: run `python adaptive_block_sparse_tile_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    G, D, C = ctypes.POINTER(Grid), ctypes.POINTER(Desc), ctypes.POINTER(RouteCfg)
    lib.fva_num_blocks.restype = ctypes.c_int32
    lib.fva_num_blocks.argtypes = [G]
    lib.fva_route_workspace_bytes.restype = ctypes.c_size_t
    lib.fva_route_workspace_bytes.argtypes = [D, G]
    lib.fva_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.fva_attn_workspace_bytes.argtypes = [D, G]
    lib.fva_attn_workgroups.restype = ctypes.c_int32
    lib.fva_attn_workgroups.argtypes = [D, G]
    lib.fva_route.restype = ctypes.c_int
    lib.fva_route.argtypes = [_P, _P, D, G, C, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.fva_route_noalloc.restype = ctypes.c_int
    lib.fva_route_noalloc.argtypes = [_P, _P, D, G, C, _P, _P, _P, _P]
    lib.fva_static_mask.restype = ctypes.c_int
    lib.fva_static_mask.argtypes = [D, G, ctypes.POINTER(StaticCfg), _P, _P, _P]
    lib.fva_sparse_attn.restype = ctypes.c_int
    lib.fva_sparse_attn.argtypes = [_P, _P, _P, _P, D, G, _P, ctypes.c_float, ctypes.c_int32, _P, _P,
                                    ctypes.c_size_t, _P]
    lib.fva_attn_plan.restype = ctypes.c_int
    lib.fva_attn_plan.argtypes = [_P, _P, D, G, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]
    lib.fva_attn_exec.restype = ctypes.c_int
    lib.fva_attn_exec.argtypes = [_P, _P, D, G, _P, ctypes.c_float, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]
    lib.fva_routed_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.fva_routed_attn_workspace_bytes.argtypes = [D, G, ctypes.c_int32]
    lib.fva_routed_attn.restype = ctypes.c_int
    lib.fva_routed_attn.argtypes = [_P, _P, _P, _P, D, G, C, ctypes.c_float, ctypes.c_int32, _P, _P, _P, _P,
                                    ctypes.c_size_t, _P, _P]
    lib.fva_attn_items.restype = ctypes.c_int32
    lib.fva_attn_items.argtypes = [D, G]
    lib.fva_attn_schedule.restype = ctypes.c_int
    lib.fva_attn_schedule.argtypes = [D, G, _P, ctypes.c_size_t, _P, _P, _P, _P]
    lib.fva_sasa_workspace_bytes.restype = ctypes.c_size_t
    lib.fva_sasa_workspace_bytes.argtypes = [D, G, ctypes.c_int32]
    lib.fva_sasa.restype = ctypes.c_int
    lib.fva_sasa.argtypes = [D, G, _P, _P, ctypes.c_size_t, ctypes.c_int32, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                             _P]
    lib.fva_trace_xcd_speed.restype = ctypes.c_int
    lib.fva_trace_xcd_speed.argtypes = [_P, ctypes.c_int32, _P, _P]
    lib.fva_dense_workspace_bytes.restype = ctypes.c_size_t
    lib.fva_dense_workspace_bytes.argtypes = [D]
    lib.fva_dense_attn_ref.restype = ctypes.c_int
    lib.fva_dense_attn_ref.argtypes = [_P, _P, _P, _P, D, ctypes.c_float, _P, ctypes.c_size_t, _P]
    lib.fva_trace_imbalance.restype = ctypes.c_int
    lib.fva_trace_imbalance.argtypes = [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    lib.fva_last_error.restype = ctypes.c_char_p
    lib.fva_last_error.argtypes = []
    lib.fva_status_name.restype = ctypes.c_char_p
    lib.fva_status_name.argtypes = [ctypes.c_int32]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != FVA_OK:
        raise FvaError(rc, load().fva_last_error().decode())


def make_grid(grid, block) -> Grid:
    return Grid(*[int(x) for x in tuple(grid) + tuple(block)])


def make_desc(B, L, heads, D) -> Desc:
    return Desc(int(B), int(L), int(heads), int(D))


def num_blocks(grid, block) -> int:
    return load().fva_num_blocks(ctypes.byref(make_grid(grid, block)))


def route_workspace_bytes(shape, grid, block) -> int:
    return load().fva_route_workspace_bytes(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)))


def attn_workspace_bytes(shape, grid, block) -> int:
    return load().fva_attn_workspace_bytes(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)))


def attn_workgroups(shape, grid, block) -> int:
    n = load().fva_attn_workgroups(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)))
    if n < 0:
        raise FvaError(1, "fva_attn_workgroups failed")
    return n


# ----------------------------------------------------------------------- torch-facing calls
def _torch():
    import torch
    return torch


def _on_stream(fn):
    """Run fn with its `stream` argument (when given) as torch's current
    stream, so that every tensor fn allocates -- outputs and the temporary
    workspace freed on return -- belongs to the stream the kernels are
    enqueued on: the caching allocator then hands a freed block only to work
    ordered after those kernels."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        ctx = _torch().cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, **kwargs)
    return wrapped


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_qkv(*ts):
    torch = _torch()
    shape = ts[0].shape
    for t in ts:
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 4 or t.shape != shape:
            raise ValueError("q, k, v must be contiguous bf16 device tensors of one shape [B, L, heads, D]")
    return tuple(int(x) for x in shape)


def workspace(nbytes: int, device):
    """Caller-owned device workspace (256-byte aligned by the torch allocator)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@_on_stream
def route(q, k, grid, block, top_p: float, k_floor: int, ws=None, out=None, stream=None):
    """Block router on the GPU -> (mask u32 [B, heads, N, W] as int32 bits, kv_cnt int32 [B, heads, N],
    status int32 [1])."""
    torch = _torch()
    shape = _check_qkv(q, k)
    B, L, heads, D = shape
    N = num_blocks(grid, block)
    words = (N + 31) // 32
    if out is None:
        mask = torch.empty((B, heads, N, words), dtype=torch.int32, device=q.device)
        cnt = torch.empty((B, heads, N), dtype=torch.int32, device=q.device)
        status = torch.empty((1,), dtype=torch.int32, device=q.device)
    else:
        mask, cnt, status = out
    need = route_workspace_bytes(shape, grid, block)
    if ws is None:
        ws = workspace(need, q.device)
    _check(load().fva_route(q.data_ptr(), k.data_ptr(), ctypes.byref(make_desc(*shape)),
                            ctypes.byref(make_grid(grid, block)), ctypes.byref(RouteCfg(float(top_p), int(k_floor))),
                            mask.data_ptr(), cnt.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(),
                            _stream_ptr(stream)))
    return mask, cnt, status


@_on_stream
def route_noalloc(q, k, grid, block, top_p: float, k_floor: int, out=None, stream=None):
    """The router on the library's static scratch (fva_route_noalloc: no
    workspace, no device allocation inside the call; outputs are allocated
    here unless `out` gives them) -> (mask, kv_cnt, status) as route()."""
    torch = _torch()
    shape = _check_qkv(q, k)
    B, L, heads, D = shape
    N = num_blocks(grid, block)
    if out is None:
        out = (torch.empty((B, heads, N, (N + 31) // 32), dtype=torch.int32, device=q.device),
               torch.empty((B, heads, N), dtype=torch.int32, device=q.device),
               torch.empty((1,), dtype=torch.int32, device=q.device))
    mask, cnt, status = out
    _check(load().fva_route_noalloc(q.data_ptr(), k.data_ptr(), ctypes.byref(make_desc(*shape)),
                                    ctypes.byref(make_grid(grid, block)),
                                    ctypes.byref(RouteCfg(float(top_p), int(k_floor))), mask.data_ptr(),
                                    cnt.data_ptr(), status.data_ptr(), _stream_ptr(stream)))
    return mask, cnt, status


@_on_stream
def sparse_attn(q, k, v, grid, block, mask, scale=None, sched: str = "lpt", trace=None, ws=None, out=None,
                stream=None):
    """Block-sparse attention on the GPU -> O bf16 [B, L, heads, D].

    trace: optional uint64-sized device tensor (int64) of attn_workgroups()*4 entries."""
    torch = _torch()
    shape = _check_qkv(q, k, v)
    B, L, heads, D = shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    need = attn_workspace_bytes(shape, grid, block)
    if ws is None:
        ws = workspace(need, q.device)
    sch = SCHEDS[sched]
    tp = trace.data_ptr() if trace is not None else None
    _check(load().fva_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)),
                                  mask.data_ptr(), float(scale), sch, tp, ws.data_ptr(), ws.numel(),
                                  _stream_ptr(stream)))
    return o


@_on_stream
def static_mask(shape, grid, block, local=(1, 1, 1), anchor_t=0, out=None, device="cuda", stream=None):
    """Static local-box + anchor-slab block mask of every (b, h) on the GPU -> (mask, kv_cnt)."""
    torch = _torch()
    B, L, heads, D = (int(x) for x in shape)
    N = num_blocks(grid, block)
    words = (N + 31) // 32
    if out is None:
        mask = torch.empty((B, heads, N, words), dtype=torch.int32, device=device)
        cnt = torch.empty((B, heads, N), dtype=torch.int32, device=device)
    else:
        mask, cnt = out
    cfg = StaticCfg(*[int(x) for x in local], int(anchor_t))
    _check(load().fva_static_mask(ctypes.byref(make_desc(B, L, heads, D)), ctypes.byref(make_grid(grid, block)),
                                  ctypes.byref(cfg), mask.data_ptr(), cnt.data_ptr(), _stream_ptr(stream)))
    return mask, cnt


@_on_stream
def attn_plan(k, v, grid, block, mask, sched: str = "lpt", head_xcd=None, ws=None, stream=None):
    """First half of sparse_attn: chunk images, item costs and the schedule,
    written into ws (allocated if None and returned).  head_xcd: optional
    device int32 [B*heads] (from sasa) for sched="xcd"."""
    shape = _check_qkv(k, k, v)
    need = attn_workspace_bytes(shape, grid, block)
    if ws is None:
        ws = workspace(need, k.device)
    hx = head_xcd.data_ptr() if head_xcd is not None else None
    _check(load().fva_attn_plan(k.data_ptr(), v.data_ptr(), ctypes.byref(make_desc(*shape)),
                                ctypes.byref(make_grid(grid, block)), mask.data_ptr(), SCHEDS[sched], hx,
                                ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    return ws


@_on_stream
def attn_exec(q, grid, block, mask, ws, scale=None, sched: str = "lpt", trace=None, out=None, stream=None):
    """Second half of sparse_attn: the attention kernel over the plan in ws
    (sched as given to attn_plan)."""
    torch = _torch()
    shape = _check_qkv(q, q, q)
    D = shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    tp = trace.data_ptr() if trace is not None else None
    _check(load().fva_attn_exec(q.data_ptr(), o.data_ptr(), ctypes.byref(make_desc(*shape)),
                                ctypes.byref(make_grid(grid, block)), mask.data_ptr(), float(scale), SCHEDS[sched],
                                tp, ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    return o


def routed_attn_workspace_bytes(shape, grid, block, groups=1) -> int:
    return int(load().fva_routed_attn_workspace_bytes(ctypes.byref(make_desc(*shape)),
                                                      ctypes.byref(make_grid(grid, block)), int(groups)))


@_on_stream
def routed_attn(q, k, v, grid, block, top_p: float, k_floor: int, groups: int = 1, side_stream=None, scale=None,
                ws=None, out=None, stream=None):
    """The whole layer (fva_routed_attn): routing, then sparse attention on
    its mask, pipelined over `groups` head groups alternating between the
    current stream and `side_stream` -> (o, mask, kv_cnt, status)."""
    torch = _torch()
    shape = _check_qkv(q, k, v)
    B, L, heads, D = shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    N = num_blocks(grid, block)
    if out is None:
        out = (torch.empty_like(q), torch.empty((B, heads, N, (N + 31) // 32), dtype=torch.int32, device=q.device),
               torch.empty((B, heads, N), dtype=torch.int32, device=q.device),
               torch.empty((1,), dtype=torch.int32, device=q.device))
    o, mask, cnt, status = out
    if ws is None:
        ws = workspace(routed_attn_workspace_bytes(shape, grid, block, groups), q.device)
    side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else None
    if side_stream is not None:
        ws.record_stream(side_stream)     # the side stream's kernels use the workspace too
    _check(load().fva_routed_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)),
                                  ctypes.byref(RouteCfg(float(top_p), int(k_floor))), float(scale), int(groups),
                                  mask.data_ptr(), cnt.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream_ptr(stream), side))
    return o, mask, cnt, status


def attn_items(shape, grid, block) -> int:
    """Number of work items of the sparse attention for q/k/v of shape [B, L, heads, D]."""
    n = int(load().fva_attn_items(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block))))
    if n < 0:
        raise FvaError(1, load().fva_last_error().decode() or "invalid shape or grid")
    return n


@_on_stream
def attn_schedule(shape, grid, block, ws, stream=None):
    """The schedule a plan wrote into ws -> (order int32 [items], qoff int32 [9],
    cost int32 [items] holding the uint32 item costs), device tensors."""
    torch = _torch()
    n = attn_items(shape, grid, block)
    order = torch.empty(n, dtype=torch.int32, device=ws.device)
    qoff = torch.empty(9, dtype=torch.int32, device=ws.device)
    cost = torch.empty(n, dtype=torch.int32, device=ws.device)
    _check(load().fva_attn_schedule(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)),
                                    ws.data_ptr(), ws.numel(), order.data_ptr(), qoff.data_ptr(), cost.data_ptr(),
                                    _stream_ptr(stream)))
    return order, qoff, cost


def sasa_workspace_bytes(shape, grid, block, rounds) -> int:
    return load().fva_sasa_workspace_bytes(ctypes.byref(make_desc(*shape)), ctypes.byref(make_grid(grid, block)),
                                           int(rounds))


@_on_stream
def sasa(shape, grid, block, mask, route_ws, rounds=4, xcd_weight=None, out=None, ws=None, stream=None):
    """Slack-aware augmentation of a routed mask on the GPU (8 XCDs as ranks).

    route_ws: the workspace of the fva_route call that produced mask.
    xcd_weight: optional 8 relative XCD speeds (per mille), e.g. from xcd_speed().
    Returns (mask_out, kv_cnt, head_xcd int32 [B*heads], xcd_load int64 [16])."""
    torch = _torch()
    B, L, heads, D = (int(x) for x in shape)
    desc, g = make_desc(B, L, heads, D), make_grid(grid, block)
    if out is None:
        mask_out = torch.empty_like(mask)
        cnt = torch.empty(mask.shape[:-1], dtype=torch.int32, device=mask.device)
    else:
        mask_out, cnt = out
    head_xcd = torch.empty(B * heads, dtype=torch.int32, device=mask.device)
    xcd_load = torch.empty(16, dtype=torch.int64, device=mask.device)
    if ws is None:
        ws = workspace(sasa_workspace_bytes(shape, grid, block, rounds), mask.device)
    wts = None
    if xcd_weight is not None:
        wts = np.ascontiguousarray(xcd_weight, dtype=np.int32)
        assert wts.shape == (8,)
    _check(load().fva_sasa(ctypes.byref(desc), ctypes.byref(g), mask.data_ptr(), route_ws.data_ptr(),
                           route_ws.numel(), int(rounds), wts.ctypes.data if wts is not None else None,
                           mask_out.data_ptr(), cnt.data_ptr(), head_xcd.data_ptr(),
                           xcd_load.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream)))
    return mask_out, cnt, head_xcd, xcd_load


def dense_workspace_bytes(shape):
    """Workspace bytes of dense_attn_ref for q/k/v of shape [B, L, heads, D]."""
    return int(load().fva_dense_workspace_bytes(ctypes.byref(make_desc(*shape))))


@_on_stream
def dense_attn_ref(q, k, v, scale=None, out=None, ws=None, stream=None):
    """Dense attention over all tokens on the GPU (same kernel and numerics)."""
    torch = _torch()
    shape = _check_qkv(q, k, v)
    D = shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    if ws is None:
        ws = workspace(dense_workspace_bytes(shape), q.device)
    _check(load().fva_dense_attn_ref(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     ctypes.byref(make_desc(*shape)), float(scale), ws.data_ptr(), ws.numel(),
                                     _stream_ptr(stream)))
    return o


def xcd_speed(trace_host: np.ndarray, xcd_load) -> np.ndarray:
    """Relative XCD speeds (per mille) from a host copy of a per-XCD-schedule
    trace and the cost sasa() placed on each XCD (fva_trace_xcd_speed).  The
    traces of several launches may be stacked (any leading shape): their item
    times add up per XCD."""
    t = np.ascontiguousarray(trace_host).view(np.uint64).reshape(-1)
    ld = np.ascontiguousarray(np.asarray(xcd_load)[:8], dtype=np.int64)
    out = np.zeros(8, dtype=np.int32)
    _check(load().fva_trace_xcd_speed(t.ctypes.data, t.size // 4, ld.ctypes.data, out.ctypes.data))
    return out


def trace_imbalance(trace_host: np.ndarray):
    """(busy max/mean, finish max/mean, CUs used) from a host copy of the trace."""
    t = np.ascontiguousarray(trace_host).view(np.uint64).reshape(-1)
    n_wg = t.size // 4
    b, f, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
    _check(load().fva_trace_imbalance(t.ctypes.data, n_wg, ctypes.byref(b), ctypes.byref(f), ctypes.byref(n)))
    return b.value, f.value, n.value
