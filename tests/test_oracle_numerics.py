"""Pins of the oracle's scalar numerics against IEEE 754 and library routines.

fp16 conversions are pinned to numpy's IEEE binary16 conversion (round half to even, with
subnormals); the pair norm is pinned to correct rounding by an exact float64 bracket test.
"""
import numpy as np
import pytest


def test_h2f_all_fp16(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.h2f(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _boundary_fp32():
    """Every binary16 value, every midpoint between neighbours, and their fp32 neighbours:
    all the places where a round-to-nearest-even decision can change."""
    h = np.arange(0, 0x7C01, dtype=np.uint32).astype(np.uint16)  # +0 .. +inf
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0  # exact in fp32 (binary16 midpoints need 12 bits)
    pts = np.concatenate([v[:-1], mids, [65520.0, 65504.0, 2.0 ** -25, 2.0 ** -24]])
    f = pts.astype(np.float32)
    u = f.view(np.uint32)
    allv = np.concatenate([u, u + 1, u - 1, u + 2, u - 2]).astype(np.uint32)
    allv = allv[(allv & 0x7F800000) != 0x7F800000]
    f = allv.view(np.float32)
    return np.concatenate([f, -f])


def test_f2h_round_half_even_boundaries(orc):
    f = _boundary_fp32()
    got = orc.f2h(f)
    ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f2h_random_bits(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    got = orc.f2h(f)
    ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


@pytest.mark.slow
def test_f2h_exhaustive(orc):
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        f = bits.view(np.float32)
        nan = np.isnan(f)
        assert np.array_equal(orc.f2h(f)[~nan], f.astype(np.float16).view(np.uint16)[~nan])


def _check_correctly_rounded_sqrt(a32: np.ndarray, r32: np.ndarray):
    """r = fl32(sqrt(a)) iff (r - ulp/2)^2 <= a <= (r + ulp/2)^2 with ties broken to even.
    r +- ulp/2 has 25 significant bits, so its square is exact in float64 (50 bits)."""
    a = a32.astype(np.float64)
    r = r32.astype(np.float64)
    nz = a > 0
    a, r = a[nz], r[nz]
    up = np.nextafter(r32[nz], np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r32[nz], np.float32(0)).astype(np.float64)
    hi = (r + up) / 2.0
    lo = (r + dn) / 2.0
    assert np.all(lo * lo <= a)
    assert np.all(a <= hi * hi)
    tie_hi = a == hi * hi
    tie_lo = a == lo * lo
    odd = (r32[nz].view(np.uint32) & 1) == 1
    assert not np.any((tie_hi | tie_lo) & odd)


def test_pair_norm_correctly_rounded(orc):
    rng = np.random.default_rng(11)
    x = rng.integers(0, 1 << 16, size=1 << 21, dtype=np.uint32).astype(np.uint16)
    y = rng.integers(0, 1 << 16, size=1 << 21, dtype=np.uint32).astype(np.uint16)
    fin = ((x & 0x7C00) != 0x7C00) & ((y & 0x7C00) != 0x7C00)
    x, y = x[fin], y[fin]
    n = orc.pair_norm(x, y)
    fx = x.view(np.float16).astype(np.float32)
    fy = y.view(np.float16).astype(np.float32)
    a = fx * fx + fy * fy  # numpy float32: one IEEE product each, one IEEE sum (no FMA)
    ok = np.isfinite(a)
    _check_correctly_rounded_sqrt(a[ok], n[ok])
    # the sum of squares itself: two roundings, never contracted
    a64 = fx.astype(np.float64) ** 2 + fy.astype(np.float64) ** 2
    assert np.all(np.abs(a[ok] - a64[ok]) <= 2.0 ** -23 * a64[ok] + 1e-45)


def test_pair_norm_special_values(orc):
    f16 = lambda v: np.array([v], np.float16).view(np.uint16)
    assert orc.pair_norm(f16(3.0), f16(4.0))[0] == 5.0
    assert orc.pair_norm(f16(-3.0), f16(4.0))[0] == 5.0
    assert orc.pair_norm(f16(0.0), f16(-0.0))[0] == 0.0
    assert orc.pair_norm(f16(0.0), f16(-2.0))[0] == 2.0
    # largest finite binary16: 65504^2 * 2 fits in fp32
    assert orc.pair_norm(f16(65504.0), f16(65504.0))[0] == np.float32(np.sqrt(np.float32(65504.0 ** 2) * 2))
    # smallest subnormal: (2^-24)^2 is 2^-48, a normal fp32
    assert orc.pair_norm(f16(2.0 ** -24), f16(0.0))[0] == np.float32(2.0 ** -24)
