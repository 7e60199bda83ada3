"""Pins of the oracle's gather + contraction against what the pages and mathematics fix.

- exact rational brute force (fractions.Fraction) on tiny shapes, within the fp64
  summation bound K * 2^-53 * sum|a*b|, and RNE of the exact value via an independent
  pure-Python rounding on rationals;
- a library fp64 matmul of the gathered A (a special case that reduces to a library
  routine);
- identity, permutation and zero B (closed forms), exact-integer inputs;
- invariance to the shard count D (the same A cut into 1, 2, 4 or 8 shards);
- the hand-written shard-order fixture in tests/golden (the Helion thread's local-tile
  index formula: shard r holds global rows [r*M_per_rank, (r+1)*M_per_rank));
- the sampled entry point agrees with the full one bit for bit;
- planted mistakes (a transposed operand, a swapped shard order, a dropped K term, a
  flipped sign) each fail at least one of these pins.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import Workload, bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_bits(dt, shape, rng, scale=1.0):
    x = torch.from_numpy(rng.uniform(-1, 1, size=shape) * scale).to(torch.float32)
    t = x.to(torch.float16 if dt == oracle.F16 else torch.bfloat16)
    return bits(t)


def _split(A_bits, D):
    M = A_bits.shape[0]
    ms = M // D
    return [A_bits[d * ms:(d + 1) * ms].copy() for d in range(D)]


def _frac_rne(dt, q: Fraction) -> int:
    """Independent RNE of an exact rational into the 16-bit format (pure Python)."""
    p, emin, emax, bias = (11, -14, 15, 15) if dt == oracle.F16 else (8, -126, 127, 127)
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    n = a / Fraction(2) ** (e - (p - 1))
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl >= 2 ** p:
        fl //= 2
        e += 1
    if e > emax:
        return sign | (((1 << (16 - p)) - 1) << (p - 1)) if dt == oracle.F16 else sign | 0x7F80
    if fl < 2 ** (p - 1):
        return sign | fl
    return sign | ((e + bias) << (p - 1)) | (fl - 2 ** (p - 1))


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
@pytest.mark.parametrize("D,Ms,N,K", [(1, 3, 5, 7), (2, 2, 3, 16), (4, 1, 4, 9), (2, 4, 1, 1)])
def test_brute_force_rational(dt, D, Ms, N, K):
    rng = np.random.default_rng(D * 1000 + Ms * 100 + N * 10 + K)
    M = D * Ms
    A = _rand_bits(dt, (M, K), rng)
    B = _rand_bits(dt, (K, N), rng)
    bias = _rand_bits(dt, (N,), rng)
    Ad, Bd, bd = oracle.decode(dt, A), oracle.decode(dt, B), oracle.decode(dt, bias)
    for use_bias in (False, True):
        C, out16, _ = oracle.agmm(dt, _split(A, D), B, bias if use_bias else None)
        for i in range(M):
            for j in range(N):
                exact = sum(Fraction(float(Ad[i, k])) * Fraction(float(Bd[k, j])) for k in range(K))
                absum = sum(abs(float(Ad[i, k]) * float(Bd[k, j])) for k in range(K))
                if use_bias:
                    exact += Fraction(float(bd[j]))
                    absum += abs(float(bd[j]))
                err = abs(Fraction(C[i, j]) - exact)
                assert err <= Fraction((K + 1) * absum) * Fraction(1, 2 ** 53)
                if Fraction(C[i, j]) == exact:
                    assert int(out16[i, j]) == _frac_rne(dt, exact)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_against_library_fp64_matmul(dt):
    rng = np.random.default_rng(7)
    D, Ms, N, K = 4, 24, 40, 56
    A = _rand_bits(dt, (D * Ms, K), rng)
    B = _rand_bits(dt, (K, N), rng)
    bias = _rand_bits(dt, (N,), rng)
    C, _, _ = oracle.agmm(dt, _split(A, D), B, bias)
    ref = torch.from_numpy(oracle.decode(dt, A)) @ torch.from_numpy(oracle.decode(dt, B))
    ref = ref.numpy() + oracle.decode(dt, bias)[None, :]
    np.testing.assert_allclose(C, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_identity_and_permutation_B(dt):
    rng = np.random.default_rng(11)
    D, Ms, K = 2, 8, 32
    A = _rand_bits(dt, (D * Ms, K), rng)
    one = 0x3C00 if dt == oracle.F16 else 0x3F80
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = one
    C, out16, _ = oracle.agmm(dt, _split(A, D), eye)
    np.testing.assert_array_equal(C, oracle.decode(dt, A))
    nz = oracle.decode(dt, A) != 0          # -0 * 1 + 0 * x gives +0
    np.testing.assert_array_equal(out16[nz], A[nz])
    perm = rng.permutation(K)
    P = np.zeros((K, K), dtype=np.uint16)
    P[perm, np.arange(K)] = one             # column j picks row perm[j]
    C, out16, _ = oracle.agmm(dt, _split(A, D), P)
    np.testing.assert_array_equal(C, oracle.decode(dt, A)[:, perm])


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_zero_B_with_bias(dt):
    rng = np.random.default_rng(12)
    A = _rand_bits(dt, (6, 10), rng)
    B = np.zeros((10, 9), dtype=np.uint16)
    bias = _rand_bits(dt, (9,), rng)
    C, out16, _ = oracle.agmm(dt, _split(A, 3), B, bias)
    for i in range(6):
        np.testing.assert_array_equal(C[i], oracle.decode(dt, bias))
        nz = oracle.decode(dt, bias) != 0
        np.testing.assert_array_equal(out16[i][nz], bias[nz])


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_shard_count_invariance(dt):
    rng = np.random.default_rng(13)
    M, N, K = 32, 12, 20
    A = _rand_bits(dt, (M, K), rng)
    B = _rand_bits(dt, (K, N), rng)
    ref = oracle.agmm(dt, [A], B)[0]
    for D in (2, 4, 8):
        np.testing.assert_array_equal(oracle.agmm(dt, _split(A, D), B)[0], ref)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_exact_integer_inputs(dt):
    w = Workload("int", 4, 64, 48, 96, dt, "int", True, "k_contiguous", True, 21)
    inp = make_inputs(w)
    sh = [bits(s) for s in inp.shards]
    C, out16, _ = oracle.agmm(dt, sh, bits(inp.B), bits(inp.bias))
    A = np.concatenate([s.float().numpy() for s in inp.shards]).astype(np.int64)
    ref = A @ inp.B.float().numpy().astype(np.int64) + inp.bias.float().numpy().astype(np.int64)
    np.testing.assert_array_equal(C, ref.astype(np.float64))
    # |C| <= 4K + 2 < 2^11: exact in binary16; bfloat16 rounds, checked against the
    # independent rational RNE
    if dt == "f16":
        np.testing.assert_array_equal(oracle.decode(dt, out16), ref.astype(np.float64))
    else:
        exp = np.array([_frac_rne(oracle.BF16, Fraction(int(v))) for v in ref.reshape(-1)])
        np.testing.assert_array_equal(out16.reshape(-1), exp.astype(np.uint16))


def _read_fixture(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rhs = line.split("=", 1)
            rows = [r.strip() for r in rhs.split(";")]
            vals[key.strip()] = np.array([[float(x) for x in r.split()] for r in rows])
    return vals


def _f16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


@pytest.mark.parametrize("name", ["shard_order_d2.txt", "shard_order_d4_bias.txt"])
def test_golden_shard_order(name):
    v = _read_fixture(name)
    shards = [_f16_bits(v[k]) for k in sorted(v) if k.startswith("shard")]
    bias = _f16_bits(v["bias"][0]) if "bias" in v else None
    C, out16, _ = oracle.agmm(oracle.F16, shards, _f16_bits(v["B"]), bias)
    np.testing.assert_array_equal(C, v["out"])
    np.testing.assert_array_equal(out16, _f16_bits(v["out"]))


def test_sampled_matches_full():
    rng = np.random.default_rng(14)
    dt = oracle.BF16
    A = _rand_bits(dt, (48, 64), rng)
    B = _rand_bits(dt, (64, 40), rng)
    bias = _rand_bits(dt, (40,), rng)
    sh = _split(A, 4)
    C, _, _ = oracle.agmm(dt, sh, B, bias)
    rows = rng.integers(0, 48, 300)
    cols = rng.integers(0, 40, 300)
    np.testing.assert_array_equal(oracle.agmm_at(dt, sh, B, bias, rows, cols), C[rows, cols])
    C2, _, _ = oracle.agmm(dt, sh, B, bias, row_begin=13, row_end=29)
    np.testing.assert_array_equal(C2, C[13:29])


def test_check_reports_first_mismatch():
    C = np.linspace(-1, 1, 64).reshape(8, 8)
    good = oracle.encode_rne(oracle.F16, C)
    r = oracle.check(oracle.F16, good, C)
    assert r["bad"] == 0 and r["first_bad"] == -1
    bad = good.copy()
    bad[3, 5] = oracle.encode_rne(oracle.F16, np.array([C[3, 5] + 0.01]))[0]
    r = oracle.check(oracle.F16, bad, C)
    assert r["bad"] == 1 and r["first_bad_index"] == (3, 5)
    nan = good.copy()
    nan[0, 0] = 0x7E00
    assert oracle.check(oracle.F16, nan, C)["bad"] == 1


def test_planted_mistakes_are_caught():
    """Each plausible oracle mistake, simulated on the CPU, fails a pin above."""
    rng = np.random.default_rng(15)
    dt = oracle.F16
    K = 16
    A = _rand_bits(dt, (K, K), rng)
    B = _rand_bits(dt, (K, K), rng)
    lib = (torch.from_numpy(oracle.decode(dt, A)) @ torch.from_numpy(oracle.decode(dt, B))).numpy()
    good = oracle.agmm(dt, _split(A, 2), B)[0]
    assert np.allclose(good, lib, rtol=1e-12, atol=1e-14)
    # transposed operand
    assert not np.allclose(oracle.agmm(dt, _split(A, 2), B.T.copy())[0], lib, rtol=1e-6)
    # swapped shard order
    sh = _split(A, 2)
    assert not np.allclose(oracle.agmm(dt, sh[::-1], B)[0], lib, rtol=1e-6)
    # a dropped K term (last column of A zeroed)
    A2 = A.copy()
    A2[:, -1] = 0
    assert not np.allclose(oracle.agmm(dt, _split(A2, 2), B)[0], lib, rtol=1e-6)
    # a flipped sign on B
    assert not np.allclose(oracle.agmm(dt, _split(A, 2), B ^ 0x8000)[0], lib, rtol=1e-6)


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_check_tolerance_edge(dt):
    """The pass/fail edge of the output check sits exactly at |got - C| = rtol*|C| + atol, with
    C the unrounded reference: an error of 0.99 of the tolerance passes and 1.01 fails, on
    both sides of C, where the relative term dominates (|C| large) and where the absolute
    term does (|C| small). A check built with a wrong rtol or atol moves the edge and fails
    one of these."""
    rtol, atol = oracle.TOL[dt]
    # representable 16-bit values: large ones (rtol*|g| >> atol) and small ones (<< atol)
    g = np.array([3.0, -5.5, 96.0, 0.0, 1.0 / 1024, -1.0 / 512])
    gb = oracle.encode_rne(dt, g)
    g = oracle.decode(dt, gb)  # exact values of the encoded patterns
    for f, want_bad in ((0.99, 0), (1.01, len(g))):
        for side in (1.0, -1.0):
            # C = g + side * d with d = f * (rtol * |C| + atol); |C| = |g| + side * sign(g) * d
            # for g != 0 (and |C| = d when g == 0), solved for d
            s = np.where(g == 0, 1.0, side * np.sign(g))
            d = f * (rtol * np.abs(g) + atol) / (1.0 - s * f * rtol)
            C = g + side * d
            # keep the cases where C stays on g's side of zero (the solved |C| holds there)
            keep = (g == 0) | (np.sign(C) == np.sign(g))
            assert keep.sum() >= 4
            r = oracle.check(dt, gb[keep], C[keep])
            assert r["bad"] == (want_bad and int(keep.sum())), (f, side, r)
            assert abs(r["max_ratio"] - f) < 1e-9, (f, side, r)
