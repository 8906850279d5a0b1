"""The seeded input generator: reproducible, thread-count independent, and
shaped as the workloads state (CPU only)."""
import numpy as np
import pytest

import fvgen
import oracle


def test_thread_count_independent():
    wl = fvgen.WORKLOADS["tiny"]
    a = fvgen.generate(wl, "k", nthreads=1)
    b = fvgen.generate(wl, "k", nthreads=7)
    assert np.array_equal(a, b)


def test_seed_changes_bytes():
    wl = fvgen.WORKLOADS["tiny"]
    assert not np.array_equal(fvgen.generate(wl, "q", seed=0), fvgen.generate(wl, "q", seed=1))


def test_moments_and_shared_field():
    wl = fvgen.WORKLOADS["tiny"]
    q, k, v = (fvgen.bf16_to_f64(a) for a in fvgen.generate_qkv(wl))
    # K and V: 0.7 * (unit-variance field) + 0.3 * N(0,1) -> variance 0.58
    for x in (k, v):
        assert abs(x.mean()) < 0.02
        assert abs(x.var() - 0.58) < 0.03
    # Q is the same recipe scaled by the head temperature (1.0 and 3.0)
    assert abs(q[..., 0, :].var() - 0.58) < 0.03
    assert abs(q[..., 1, :].var() - 9 * 0.58) < 0.3
    # shared field: corr(K, V) = 0.49 / 0.58 per channel
    kk, vv = k[0, :, 0, :], v[0, :, 0, :]
    c = ((kk - kk.mean(0)) * (vv - vv.mean(0))).mean(0) / (kk.std(0) * vv.std(0))
    assert abs(c.mean() - 0.49 / 0.58) < 0.03


def test_bf16_roundtrip_helpers():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0, -0.0])
    b = fvgen.f64_to_bf16(x)
    y = fvgen.bf16_to_f64(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    assert fvgen.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80       # tie -> even
    assert fvgen.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_temperatures():
    t = fvgen.WORKLOADS["wan14b"].taus()
    assert t.shape == (40,) and (t >= 0.3).all() and (t <= 6.0).all()
    t = fvgen.WORKLOADS["720p"].taus()
    assert (t[36:] == 0.2).all() and (t[:36] >= 0.3).all()
    assert list(fvgen.WORKLOADS["long"].taus()) == [0.5, 1.0, 2.0, 4.0, 8.0]


@pytest.mark.slow
def test_wan14b_kept_fraction_spread():
    """The 14B-like layer is meant to give per-head kept fractions from about 5%
    to 80% of the 120 blocks (top_p 0.9, floor 8)."""
    wl = fvgen.WORKLOADS["wan14b"]
    q = fvgen.generate(wl, "q")
    k = fvgen.generate(wl, "k")
    _, cnt, flags, _ = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    frac = cnt[0].mean(axis=1) / 120.0
    assert frac.min() < 0.10 and frac.max() > 0.75
    assert (flags != 0).mean() < 0.01
