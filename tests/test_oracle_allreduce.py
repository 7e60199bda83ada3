"""Pins of the oracle's all-reduced GEMM (ROCm/iris PR "Let's make Iris' All-reduce the best!",
atomics example: every rank ends with C = sum_r A_r @ B_r, rank r holding A's columns K_r and
B's rows K_r).

- closed form: A = the identity cut into column slices, so C must be B exactly (and B + bias);
- every part counts: the K slices of a random product, summed, give what one unsplit
  product gives to fp64 rounding;
- planted mistakes (a rank's A slice paired with another rank's B slice, a rank left out)
  each break the closed form.
"""
import numpy as np
import pytest
import torch

import oracle


def _f16_bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def _identity_parts(K, cuts):
    eye = _f16_bits(np.eye(K))
    return [eye[:, a:b] for a, b in zip(cuts[:-1], cuts[1:])]


@pytest.mark.parametrize("K,cuts", [(48, [0, 16, 32, 48]), (40, [0, 8, 32, 40]), (24, [0, 24])])
def test_identity_closed_form(K, cuts):
    rng = np.random.default_rng(K)
    B = _f16_bits(rng.uniform(-2, 2, size=(K, 24)))
    A_parts = _identity_parts(K, cuts)
    B_parts = [B[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    C, out16, _ = oracle.gemm_allreduce(oracle.F16, A_parts, B_parts)
    np.testing.assert_array_equal(C, oracle.decode(oracle.F16, B))
    np.testing.assert_array_equal(out16, B)
    bias = _f16_bits(rng.uniform(-1, 1, size=24))
    Cb, _, _ = oracle.gemm_allreduce(oracle.F16, A_parts, B_parts, bias)
    np.testing.assert_array_equal(Cb, oracle.decode(oracle.F16, B) + oracle.decode(oracle.F16, bias))


def test_parts_sum_to_the_whole_product():
    rng = np.random.default_rng(5)
    dt = oracle.BF16
    A = torch.from_numpy(rng.standard_normal((20, 64))).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    B = torch.from_numpy(rng.standard_normal((64, 12))).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    whole = (oracle.decode(dt, A) @ oracle.decode(dt, B))
    C, _, _ = oracle.gemm_allreduce(dt, [A[:, :16], A[:, 16:40], A[:, 40:]], [B[:16], B[16:40], B[40:]])
    np.testing.assert_allclose(C, whole, rtol=1e-13, atol=1e-13)


def test_planted_mistakes_are_caught():
    K, cuts = 48, [0, 16, 32, 48]
    rng = np.random.default_rng(9)
    B = _f16_bits(rng.uniform(-2, 2, size=(K, 24)))
    A_parts = _identity_parts(K, cuts)
    B_parts = [B[a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    want = oracle.decode(oracle.F16, B)
    swapped = [B_parts[1], B_parts[0], B_parts[2]]
    assert not np.array_equal(oracle.gemm_allreduce(oracle.F16, A_parts, swapped)[0], want)
    dropped_A = [A_parts[0], np.zeros_like(A_parts[1]), A_parts[2]]
    assert not np.array_equal(oracle.gemm_allreduce(oracle.F16, dropped_A, B_parts)[0], want)
