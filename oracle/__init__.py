"""Oracle for the fused all-gather + GEMM (TEST INFRASTRUCTURE ONLY).

Only the tests, the package smoke check and the bench's CPU-baseline leg may import this
package. The GPU library never calls it, and it shares no code with the GPU library.

The arithmetic lives in ``agmm_oracle.c`` (plain C, fp64, OpenMP over output rows), loaded
here with ctypes; this file only marshals numpy arrays. See that file's header for what is
computed and which passage of the pages each step follows. The bookkeeping model (fetch
units, flags, tile order) is in ``schedule_model.py``.

Parity pins (each checked by ``tests/test_oracle_*.py`` against something other than the
oracle itself): 16-bit decode exhaustively against numpy / bit reinterpretation; RNE encode
against round-trips, all midpoints and numpy's double->half rounding; the contraction
against exact rational brute force, a library fp64 matmul, identity / permutation / zero B,
shard-count invariance, exact-integer inputs and the hand-written shard-order fixture; the
gathered A against its closed form (each shard filled with its own index and row number);
the all-reduced GEMM against an identity closed form and planted slice mistakes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

F16 = 0
BF16 = 1
_DT = {"f16": F16, "bf16": BF16, F16: F16, BF16: BF16}

# Tolerances for the output checks: max|C_gpu - C_ref| <= rtol*|C_ref| + atol, with C_ref
# the unrounded fp64 result.
TOL = {F16: (2.0 ** -10, 1e-3), BF16: (2.0 ** -7, 1e-2)}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_uint16]
    lib.oracle_decode.restype = ctypes.c_double
    lib.oracle_encode_rne.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_encode_rne.restype = ctypes.c_uint16
    lib.oracle_decode_array.argtypes = [ctypes.c_int, ctypes.c_int64, u16p, f64p]
    lib.oracle_encode_array.argtypes = [ctypes.c_int, ctypes.c_int64, f64p, u16p]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_agmm_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.POINTER(u16p), u16p, u16p,
                                     ctypes.c_int64, ctypes.c_int64, f64p, u16p]
    lib.oracle_agmm_rows.restype = ctypes.c_int
    lib.oracle_agmm_at.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.POINTER(u16p), u16p, u16p,
                                   ctypes.c_int64, i64p, i64p, f64p]
    lib.oracle_check.argtypes = [ctypes.c_int, ctypes.c_int64, u16p, f64p, ctypes.c_double,
                                 ctypes.c_double, f64p, f64p, i64p]
    lib.oracle_check.restype = ctypes.c_int64
    lib.oracle_all_gather.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.POINTER(u16p), u16p]
    _lib = lib
    return lib


def _u16(a: np.ndarray):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _f64(a: np.ndarray):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def decode(dtype, bits: np.ndarray) -> np.ndarray:
    """16-bit patterns -> exact float64 values."""
    lib = _load()
    b, bp = _u16(bits)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_decode_array(_DT[dtype], b.size, bp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def encode_rne(dtype, values: np.ndarray) -> np.ndarray:
    """float64 values -> 16-bit patterns, round-to-nearest-even, rounded once."""
    lib = _load()
    v, vp = _f64(values)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_encode_array(_DT[dtype], v.size, vp, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())


class _Args:
    """Keeps the contiguous uint16 copies alive while C holds their pointers."""

    def __init__(self, shards: Sequence[np.ndarray], B: np.ndarray, bias: Optional[np.ndarray]):
        self.shards = [_u16(s)[0] for s in shards]
        u16p = ctypes.POINTER(ctypes.c_uint16)
        self.ptrs = (u16p * len(self.shards))(*[s.ctypes.data_as(u16p) for s in self.shards])
        self.B, self.Bp = _u16(B)
        if bias is None:
            self.bias, self.biasp = None, None
        else:
            self.bias, self.biasp = _u16(bias)


def agmm(dtype, shards: Sequence[np.ndarray], B: np.ndarray, bias: Optional[np.ndarray] = None,
         row_begin: int = 0, row_end: Optional[int] = None):
    """out = concat(shards) @ B (+ bias), in fp64.

    shards: D uint16 arrays [M_s, K]; B: uint16 [K, N]; bias: uint16 [N] or None.
    Returns (C, out16, threads): C float64 [rows, N] unrounded, out16 uint16 [rows, N]
    rounded once with RNE, for global rows [row_begin, row_end).
    """
    lib = _load()
    D = len(shards)
    M_s, K = shards[0].shape
    for s in shards:
        if s.shape != (M_s, K):
            raise ValueError("all shards must have the same shape")
    K2, N = B.shape
    if K2 != K:
        raise ValueError("B must be [K, N]")
    M = D * M_s
    if row_end is None:
        row_end = M
    args = _Args(shards, B, bias)
    rows = row_end - row_begin
    C = np.empty((rows, N), dtype=np.float64)
    out16 = np.empty((rows, N), dtype=np.uint16)
    used = lib.oracle_agmm_rows(_DT[dtype], D, M, N, K, args.ptrs, args.Bp, args.biasp,
                                row_begin, row_end,
                                C.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                out16.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return C, out16, int(used)


def all_gather(shards: Sequence[np.ndarray]) -> np.ndarray:
    """The gathered A, [D * M_s, K] uint16: shard d's rows at rows d*M_s .. (d+1)*M_s - 1."""
    lib = _load()
    D = len(shards)
    M_s, K = shards[0].shape
    for s in shards:
        if s.shape != (M_s, K):
            raise ValueError("all shards must have the same shape")
    args = _Args(shards, np.zeros((0, 0), dtype=np.uint16), None)
    A = np.empty((D * M_s, K), dtype=np.uint16)
    lib.oracle_all_gather(D, M_s, K, args.ptrs, A.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    return A


def gemm_allreduce(dtype, A_parts: Sequence[np.ndarray], B_parts: Sequence[np.ndarray],
                   bias: Optional[np.ndarray] = None):
    """The all-reduced result of the GEMM + all-reduce op (ROCm/iris PR "Let's make Iris'
    All-reduce the best!", the atomics example): rank r holds A_r [M, K_r] and B_r [K_r, N],
    and every rank ends with C = sum_r A_r @ B_r (+ bias), which is the product of the
    column-concatenated A and the row-concatenated B. Returns (C, out16, threads) as agmm."""
    A = np.concatenate([_u16(a)[0] for a in A_parts], axis=1)
    B = np.concatenate([_u16(b)[0] for b in B_parts], axis=0)
    return agmm(dtype, [A], B, bias)


def agmm_at(dtype, shards: Sequence[np.ndarray], B: np.ndarray, bias: Optional[np.ndarray],
            rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Unrounded C[rows[s], cols[s]] for each sample s, each summed on its own."""
    lib = _load()
    D = len(shards)
    M_s, K = shards[0].shape
    N = B.shape[1]
    args = _Args(shards, B, bias)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    c = np.ascontiguousarray(cols, dtype=np.int64)
    if r.shape != c.shape:
        raise ValueError("rows and cols must have the same shape")
    if r.size and (r.min() < 0 or r.max() >= D * M_s or c.min() < 0 or c.max() >= N):
        raise ValueError("sample index out of range")
    out = np.empty(r.shape, dtype=np.float64)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_agmm_at(_DT[dtype], D, D * M_s, N, K, args.ptrs, args.Bp, args.biasp, r.size,
                       r.ctypes.data_as(i64p), c.ctypes.data_as(i64p),
                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def check(dtype, got_bits: np.ndarray, C_ref: np.ndarray, rtol: Optional[float] = None,
          atol: Optional[float] = None) -> dict:
    """Element-wise tolerance check of 16-bit results against the unrounded reference."""
    lib = _load()
    dt = _DT[dtype]
    if rtol is None or atol is None:
        rtol, atol = TOL[dt]
    g, gp = _u16(got_bits)
    c, cp = _f64(C_ref)
    if g.size != c.size:
        raise ValueError("size mismatch")
    mae = ctypes.c_double()
    mr = ctypes.c_double()
    first = ctypes.c_int64()
    bad = lib.oracle_check(dt, g.size, gp, cp, rtol, atol, ctypes.byref(mae), ctypes.byref(mr),
                           ctypes.byref(first))
    res = {"bad": int(bad), "max_abs_err": mae.value, "max_ratio": mr.value,
           "first_bad": int(first.value), "rtol": rtol, "atol": atol, "count": int(g.size)}
    if bad and g.ndim >= 1:
        idx = np.unravel_index(first.value, g.shape) if g.ndim > 1 else (first.value,)
        res["first_bad_index"] = tuple(int(i) for i in idx)
        res["first_bad_got"] = float(decode(dt, g.reshape(-1)[first.value:first.value + 1])[0])
        res["first_bad_expected"] = float(c.reshape(-1)[first.value])
    return res
