"""Pins of the oracle's 16-bit decode / RNE encode against definitions outside the oracle.

- decode: exhaustive over all 65536 patterns, against numpy's IEEE binary16 and against
  the bit reinterpretation of bfloat16 as the top half of an IEEE binary32;
- encode: round-trip of every finite pattern; every midpoint between adjacent finite
  values goes to the even neighbour and its two double neighbours go to the nearer value
  (the definition of round-to-nearest-even); random doubles against numpy's
  double->binary16 conversion; overflow and underflow boundaries computed by hand.
"""
import math

import numpy as np
import pytest

import oracle

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _bf16_ref(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f16_ref(bits):
    return bits.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("dt,ref", [(oracle.F16, _f16_ref), (oracle.BF16, _bf16_ref)])
def test_decode_exhaustive(dt, ref):
    got = oracle.decode(dt, ALL)
    exp = ref(ALL)
    nan = np.isnan(exp)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], exp[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(exp[~nan]))


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_encode_roundtrip_every_pattern(dt):
    vals = oracle.decode(dt, ALL)
    back = oracle.encode_rne(dt, vals)
    nan = np.isnan(vals)
    assert np.array_equal(back[~nan], ALL[~nan])
    canon = 0x7E00 if dt == oracle.F16 else 0x7FC0
    assert np.all(back[nan] == canon)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_encode_midpoints_ties_to_even(dt):
    # all positive finite patterns in increasing order of value
    emax_bits = 0x7C00 if dt == oracle.F16 else 0x7F80
    pos = np.arange(0, emax_bits, dtype=np.uint32).astype(np.uint16)
    v = oracle.decode(dt, pos)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2.0                       # exact in double
    assert np.all((mid > lo) & (mid < hi))
    got = oracle.encode_rne(dt, mid)
    even_lo = (pos[:-1] & 1) == 0
    expect = np.where(even_lo, pos[:-1], pos[1:])
    assert np.array_equal(got, expect)
    # just off the midpoint: the nearer value
    assert np.array_equal(oracle.encode_rne(dt, np.nextafter(mid, -np.inf)), pos[:-1])
    assert np.array_equal(oracle.encode_rne(dt, np.nextafter(mid, np.inf)), pos[1:])
    # negative side mirrors the positive side
    assert np.array_equal(oracle.encode_rne(dt, -mid), expect | 0x8000)


def test_encode_f16_matches_numpy_random_doubles():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(50000) * 1e-5,        # subnormal range
        rng.standard_normal(50000) * 3e4,         # near overflow
        rng.uniform(-1, 1, 50000) * 2.0 ** -24,   # around the smallest subnormal
    ])
    got = oracle.encode_rne(oracle.F16, x)
    exp = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp)


def test_encode_boundaries_by_hand():
    F16, BF16 = oracle.F16, oracle.BF16
    enc = lambda dt, x: int(oracle.encode_rne(dt, np.array([x]))[0])
    # binary16 largest finite 65504 = 0x7BFF; halfway to 65536 ties to even -> inf
    assert enc(F16, 65504.0) == 0x7BFF
    assert enc(F16, 65519.999) == 0x7BFF
    assert enc(F16, 65520.0) == 0x7C00
    assert enc(F16, -1e30) == 0xFC00
    # smallest subnormal 2^-24; half of it ties to even (zero), a bit more rounds up
    assert enc(F16, 2.0 ** -24) == 0x0001
    assert enc(F16, 2.0 ** -25) == 0x0000
    assert enc(F16, -2.0 ** -25) == 0x8000
    assert enc(F16, 3 * 2.0 ** -26) == 0x0001
    # largest subnormal rounding into the smallest normal 2^-14 = 0x0400
    assert enc(F16, 2.0 ** -14 - 2.0 ** -26) == 0x0400
    # bfloat16: 1 + 2^-8 is the tie between 1.0 and 1 + 2^-7 -> even (1.0 = 0x3F80)
    assert enc(BF16, 1.0 + 2.0 ** -8) == 0x3F80
    assert enc(BF16, 1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert enc(BF16, 1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    # bfloat16 largest finite (2 - 2^-7) * 2^127 = 0x7F7F; its upper midpoint ties to inf
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    assert enc(BF16, mx) == 0x7F7F
    assert enc(BF16, mx + 2.0 ** 119) == 0x7F80
    assert math.isnan(oracle.decode(BF16, np.array([enc(BF16, float("nan"))], dtype=np.uint16))[0])
