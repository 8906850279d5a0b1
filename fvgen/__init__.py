"""Seeded synthetic inputs for the routed block-sparse attention path.

Harness only: this module draws Q/K/V and holds none of the method's
arithmetic.  The GPU library and the CPU oracle both consume its bytes.

The workloads mirror the latent shapes the pages work with: the Wan2.2
post-patch grid (31, 22, 40) = 27280 tokens with (4, 8, 8) blocks from the
vLLM-Omni FastVideo VSA guide (section 3, its routing log line), a 720p-like
grid, and the 96*64*64 = 393,216-token long video of the Sol-Attn article
(section on memory), tiled with the (4, 4, 4) 64-token blocks that the VSA
guide names for its H3 route (section 1).  Q, K and V of a head share one
smooth random field plus independent noise; a per-head temperature scales Q
and so sets how peaked the head's block scores are.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fvgen.c")
_LIB = os.path.join(_HERE, "libfvgen.so")

STREAM_TAU = 4


def build(force: bool = False) -> str:
    """Compile libfvgen.so with gcc (plain C, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        override = os.environ.get("FVGEN_LIB")   # another build of the same source (e.g. with sanitizers)
        if not override and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(override or _LIB)
        lib.fvgen_qkv.restype = ctypes.c_int
        lib.fvgen_qkv.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.fvgen_uniform.restype = ctypes.c_double
        lib.fvgen_uniform.argtypes = [ctypes.c_uint64] * 5
        lib.fvgen_normal_at.restype = ctypes.c_double
        lib.fvgen_normal_at.argtypes = [ctypes.c_uint64] * 4
        _lib = lib
    return _lib


def uniform(seed: int, tag: int, stream: int, a: int, b: int) -> float:
    return _load().fvgen_uniform(seed, tag, stream, a, b)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass(frozen=True)
class Workload:
    """One attention layer: shape, block geometry, temperatures and routing knobs."""
    name: str
    tag: int
    heads: int
    head_dim: int
    grid: tuple            # (T, H, W)
    block: tuple           # (bt, bh, bw)
    modes: int
    tau_kind: str          # "list" | "loguniform"
    tau_args: tuple
    top_p: float           # <= 0: fixed top-k (= k_floor); >= 1: dense rows
    k_floor: int
    batch: int = 1
    global_heads: tuple = field(default_factory=tuple)   # (first_head, tau) overrides
    static: tuple = field(default_factory=tuple)         # ((lt, lh, lw), anchor_t): static block mask, no router

    @property
    def L(self) -> int:
        T, H, W = self.grid
        return T * H * W

    def taus(self, seed: int = 0) -> np.ndarray:
        if self.tau_kind == "list":
            t = np.array(self.tau_args, dtype=np.float64)
            assert t.size == self.heads
        else:
            lo, hi = self.tau_args
            u = np.array([uniform(seed, self.tag, STREAM_TAU, h, 0) for h in range(self.heads)])
            t = np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
        if self.global_heads:
            first, tau = self.global_heads
            t[first:] = tau
        return t


WORKLOADS = {
    "tiny": Workload("tiny", 0, 2, 64, (8, 16, 16), (4, 8, 8), 8, "list", (1.0, 3.0), 0.9, 2),
    "wan5b": Workload("wan5b", 1, 24, 128, (31, 22, 40), (4, 8, 8), 8, "loguniform", (0.5, 4.0), 0.0, 64),
    "wan14b": Workload("wan14b", 2, 40, 128, (31, 22, 40), (4, 8, 8), 8, "loguniform", (0.3, 6.0), 0.9, 8),
    "720p": Workload("720p", 3, 40, 128, (21, 45, 80), (4, 8, 8), 8, "loguniform", (0.3, 6.0), 0.95, 16,
                     global_heads=(36, 0.2)),
    "long": Workload("long", 4, 5, 128, (96, 64, 64), (4, 4, 4), 16, "list", (0.5, 1.0, 2.0, 4.0, 8.0), 0.85, 32),
    # the long-video grid under a static local + anchor block mask: local boxes of 2 x 16 x 16 blocks (8 latent
    # frames, whole frames), anchor slabs every 6 temporal blocks (24 latent frames)
    "static": Workload("static", 5, 5, 128, (96, 64, 64), (4, 4, 4), 16, "list", (0.5, 1.0, 2.0, 4.0, 8.0), 0.0, 1,
                       static=((2, 16, 16), 6)),
}


def generate(wl: Workload, which: str, seed: int = 0, nthreads: int | None = None, taus=None) -> np.ndarray:
    """Return bf16 bits (uint16) of shape [B, L, heads, D] for which in {'q','k','v'}.

    Batch entries b > 0 use tag wl.tag + 1000*b so that they differ."""
    lib = _load()
    T, H, W = wl.grid
    idx = {"q": 0, "k": 1, "v": 2}[which]
    tau = wl.taus(seed) if taus is None else np.asarray(taus, dtype=np.float64)
    tau = np.ascontiguousarray(tau, dtype=np.float64)
    out = np.empty((wl.batch, wl.L, wl.heads, wl.head_dim), dtype=np.uint16)
    nt = nthreads or default_threads()
    for b in range(wl.batch):
        view = out[b]
        rc = lib.fvgen_qkv(seed, wl.tag + 1000 * b, T, H, W, wl.heads, wl.head_dim, wl.modes,
                           tau.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), idx,
                           view.ctypes.data, nt)
        if rc != 0:
            raise RuntimeError("fvgen_qkv failed")
    return out


def generate_qkv(wl: Workload, seed: int = 0, nthreads: int | None = None):
    return tuple(generate(wl, w, seed, nthreads) for w in ("q", "k", "v"))


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    """Widen bf16 bits exactly to float64."""
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 -> fp32 -> bf16 bits (RNE), as the generator does."""
    f = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = ((f & 0x7F800000) == 0x7F800000) & ((f & 0x007FFFFF) != 0)
    r = ((f + np.uint32(0x7FFF) + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((f[nan] >> 16) | 0x40).astype(np.uint16)
    return r
