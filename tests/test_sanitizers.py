"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

The fp64 oracle (oracle/fvo.cpp), the input generator (fvgen/fvgen.c) and
the library's host side (adaptive_block_sparse_tile_amd/csrc/fva_api.cpp:
argument validation, workspace layout, launch-size checks; its device code
is built as usual and not instrumented) are rebuilt with clang's ASan and
UBSan into a temporary directory, and the oracle, generator and boundary
CPU tests run against those builds in a child process with the sanitizer
runtime preloaded.  Any sanitizer report aborts the child (no recovery).
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANGXX) and os.path.exists(HIPCC)), reason="needs ROCm clang")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-6000:])
    return res


def _build_sanitized(tmp):
    fvo = os.path.join(tmp, "libfvo_san.so")
    fvgen = os.path.join(tmp, "libfvgen_san.so")
    fva = os.path.join(tmp, "libfva_san.so")
    _run([CLANGXX, "-std=c++17", "-fPIC", "-shared", "-pthread"] + SAN +
         [os.path.join(ROOT, "oracle", "fvo.cpp"), "-o", fvo])
    _run([CLANG, "-std=c11", "-fPIC", "-shared", "-pthread"] + SAN +
         [os.path.join(ROOT, "fvgen", "fvgen.c"), "-o", fvgen, "-lm"])
    sys.path.insert(0, ROOT)
    from adaptive_block_sparse_tile_amd import build as libbuild
    csrc = os.path.join(ROOT, "adaptive_block_sparse_tile_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    for src in libbuild.SOURCES:
        obj = os.path.join(tmp, src + ".o")
        extra = libbuild.SOURCE_FLAGS.get(src, [])
        if src.endswith(".cpp"):   # host code only: sanitize the host compilation, never the device one
            extra = extra + ["-g", "-fno-omit-frame-pointer"] + [x for f in (
                "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all") for x in ("-Xarch_host", f)]
        _run([HIPCC] + libbuild.HIPCC_FLAGS + extra + inc + ["-c", os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", fva])
    return fvo, fvgen, fva


@pytest.mark.slow
def test_cpu_code_under_asan_and_ubsan():
    runtime = _run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    assert os.path.exists(runtime), runtime
    with tempfile.TemporaryDirectory() as tmp:
        fvo, fvgen, fva = _build_sanitized(tmp)
        env = dict(os.environ, FVO_LIB=fvo, FVGEN_LIB=fvgen, FVA_LIB=fva, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
        # the child maps the sanitized builds, and ASan reports a write past the end of an output buffer (a
        # block table one row too short handed to the oracle)
        probe = ("import sys; sys.path.insert(0, %r)\n"
                 "import numpy as np, ctypes, oracle, fvgen, adaptive_block_sparse_tile_amd as fva\n"
                 "oracle._load(); fvgen._load(); fva.load()\n"
                 "maps = open('/proc/self/maps').read()\n"
                 "assert all(n in maps for n in ('libfvo_san.so', 'libfvgen_san.so', 'libfva_san.so')), 'not loaded'\n"
                 "print('sanitized builds loaded', flush=True)\n"
                 "g = np.array([31, 22, 40, 4, 8, 8], dtype=np.int32)\n"
                 "out = np.empty((119, 7), dtype=np.int32)\n"
                 "oracle._load().fvo_block_table(g.ctypes.data, out.ctypes.data)\n" % ROOT)
        res = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300)
        assert "sanitized builds loaded" in res.stdout, res.stdout + res.stderr[-3000:]
        assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr, res.stderr[-3000:]
        tests = ["tests/test_oracle_geometry.py", "tests/test_oracle_route.py", "tests/test_oracle_attn.py",
                 "tests/test_oracle_schedule.py", "tests/test_oracle_static.py", "tests/test_oracle_sasa.py",
                 "tests/test_fvgen.py", "tests/test_boundary.py"]
        res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow",
                              "-p", "no:cacheprovider", "-k", "not sdpa"] + tests,
                             cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        out = res.stdout + res.stderr
        print(out[-1500:])
        assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
        assert res.returncode == 0, out[-6000:]
        assert " passed" in res.stdout
