"""Fused all-gather + GEMM for AMD MI355X (gfx950): Python binding of libagmm.so.

out[M, N] = concat(shard_0, ..., shard_{D-1}) @ B (+ bias), computed by hand-written gfx950
HIP kernels behind the C ABI in include/agmm.h. This module only marshals arguments: it
builds the descriptor struct, passes device pointers and the current HIP stream, and turns
error codes into exceptions. Every step of the computation runs in the library's kernels;
there is no fallback path. If libagmm.so is missing, importing this module raises.

The functions mirror the C names: ag_matmul_desc_init, ag_matmul_create, ag_matmul_run,
ag_matmul_run_gather, ag_matmul_destroy, ag_matmul_workspace_bytes, ag_matmul_strerror,
ag_matmul_get_config, ag_matmul_debug_query, ag_matmul_debug_fill_staging. `AgMatmul` wraps a handle for torch
tensors (data pointers and torch's current stream only).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libagmm.so")

AGMM_MAX_SHARDS = 64
AGMM_OK = 0
ERRORS = {-1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "HIP", -4: "OOM", -5: "TIMEOUT",
          -6: "WRONG_DEVICE", -7: "POISONED", -8: "TOO_LARGE"}
F16, BF16 = 0, 1
K_CONTIGUOUS, M_CONTIGUOUS = 0, 1
ALGO_FUSED, ALGO_BASELINE, ALGO_PIPELINED = 0, 1, 2
(Q_FLAGS, Q_STAGING, Q_TRACE, Q_TRACE_COUNT, Q_STATUS, Q_UNITS, Q_MTILES, Q_QUEUES, Q_PARTIALS,
 Q_CHUNK_SIZES, Q_CHUNK_UNITS, Q_CHUNK_MTILES) = range(1, 13)
EV_FETCH, EV_GEMM, EV_GEMM_WAIT = 1, 2, 3

EXPORTED = [
    "ag_matmul_desc_init", "ag_matmul_create", "ag_matmul_run", "ag_matmul_destroy",
    "ag_matmul_workspace_bytes", "ag_matmul_strerror", "ag_matmul_last_hip_error",
    "ag_matmul_get_config", "ag_matmul_debug_query", "ag_matmul_debug_fill_staging",
    "ag_matmul_run_gather", "ag_matmul_plan_query", "ag_gemm_ar_create", "ag_gemm_ar_run",
    "ag_gemm_ar_finalize", "ag_gemm_ar_flags_create", "ag_gemm_ar_flags_run",
    "ag_gemm_ar_flags_plan", "ag_matmul_sync_status", "ag_matmul_run_static",
    "ag_matmul_debug_run_part", "ag_matmul_debug_mfma_loop", "ag_matmul_debug_set_runs",
]
PART_COPY, PART_GEMM = 1, 2


class agmm_desc(ctypes.Structure):
    _fields_ = [
        ("D", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32), ("algo", ctypes.c_int32),
        ("direct_local", ctypes.c_int32), ("has_bias", ctypes.c_int32), ("debug", ctypes.c_int32),
        ("block_m", ctypes.c_int32), ("k_per_flag", ctypes.c_int32),
        ("num_fetch_wgs", ctypes.c_int32), ("num_wgs", ctypes.c_int32),
        ("trace_cap", ctypes.c_int32), ("spin_limit", ctypes.c_uint32),
        ("debug_skip_unit", ctypes.c_int32), ("tail_split", ctypes.c_int32),
        ("gather_a", ctypes.c_int32), ("pipeline_chunks", ctypes.c_int32),
        ("debug_fetch_delay", ctypes.c_int32), ("debug_fetch_seed", ctypes.c_uint32),
        ("debug_fetch_reverse", ctypes.c_int32), ("fetch_kernel", ctypes.c_int32),
    ]


class agmm_config(ctypes.Structure):
    _fields_ = [
        ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("k_per_flag", ctypes.c_int32), ("T_m", ctypes.c_int32), ("T_n", ctypes.c_int32),
        ("G", ctypes.c_int32), ("num_units", ctypes.c_int32), ("num_tiles", ctypes.c_int32),
        ("num_fetch_wgs", ctypes.c_int32), ("num_wgs", ctypes.c_int32),
        ("num_copy_wgs", ctypes.c_int32), ("trace_cap", ctypes.c_int32),
        ("epoch", ctypes.c_uint32), ("staging_elems", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64), ("device", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("split_tiles", ctypes.c_int32),
        ("split_pieces", ctypes.c_int32), ("num_items", ctypes.c_int32),
        ("row_wait", ctypes.c_int32), ("pipeline_chunks", ctypes.c_int32),
        ("pipeline_streams", ctypes.c_int32), ("fetch_kernel", ctypes.c_int32),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


class agmm_trace_rec(ctypes.Structure):
    _fields_ = [("event", ctypes.c_uint32), ("id", ctypes.c_uint32), ("a", ctypes.c_uint32),
                ("b", ctypes.c_uint32), ("t0", ctypes.c_uint64), ("t1", ctypes.c_uint64)]


TRACE_DTYPE = np.dtype([("event", "<u4"), ("id", "<u4"), ("a", "<u4"), ("b", "<u4"),
                        ("t0", "<u8"), ("t1", "<u8")])


class AgmmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({strerror(code)})"
                         + (f", hipError {last_hip_error()}" if code == -3 else ""))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run all_gather_gemm_amd/build.py "
                          "(or __graft_entry__.build()) first")
    # torch first: it brings its own copy of the HIP runtime, and the library must bind to
    # that same copy (its runtime symbols resolve to whatever libamdhip64 is loaded first).
    # Loaded the other way round, the process holds two runtimes, and the library's calls
    # then fail with "no device" while torch's work.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.ag_matmul_desc_init.argtypes = [ctypes.POINTER(agmm_desc)]
    lib.ag_matmul_desc_init.restype = None
    lib.ag_matmul_create.argtypes = [ctypes.POINTER(agmm_desc), vp, ctypes.c_size_t,
                                     ctypes.POINTER(vp)]
    lib.ag_matmul_sync_status.argtypes = [vp]
    lib.ag_matmul_debug_run_part.argtypes = [vp, ctypes.c_int, ctypes.POINTER(vp), vp, vp, vp, vp]
    lib.ag_matmul_debug_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, vp, vp]
    lib.ag_matmul_run_static.argtypes = [ctypes.POINTER(agmm_desc), ctypes.POINTER(vp), vp, vp,
                                         vp, vp]
    lib.ag_matmul_run.argtypes = [vp, ctypes.POINTER(vp), vp, vp, vp, vp]
    lib.ag_matmul_run_gather.argtypes = [vp, ctypes.POINTER(vp), vp, vp, vp, vp, vp]
    lib.ag_matmul_plan_query.argtypes = [ctypes.POINTER(agmm_desc), ctypes.c_int, ctypes.c_int,
                                         vp, ctypes.c_size_t]
    lib.ag_gemm_ar_create.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp)]
    lib.ag_gemm_ar_run.argtypes = [vp, vp, vp, ctypes.POINTER(vp), vp]
    lib.ag_gemm_ar_finalize.argtypes = [vp, vp, vp, vp, vp]
    lib.ag_gemm_ar_flags_create.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(vp)]
    lib.ag_gemm_ar_flags_run.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp]
    lib.ag_gemm_ar_flags_plan.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.POINTER(agmm_config),
                                          ctypes.POINTER(ctypes.c_uint32),
                                          ctypes.POINTER(ctypes.c_int64)]
    lib.ag_matmul_destroy.argtypes = [vp]
    lib.ag_matmul_workspace_bytes.argtypes = [ctypes.POINTER(agmm_desc)]
    lib.ag_matmul_workspace_bytes.restype = ctypes.c_int64
    lib.ag_matmul_strerror.argtypes = [ctypes.c_int]
    lib.ag_matmul_strerror.restype = ctypes.c_char_p
    lib.ag_matmul_last_hip_error.restype = ctypes.c_int
    lib.ag_matmul_get_config.argtypes = [vp, ctypes.POINTER(agmm_config)]
    lib.ag_matmul_debug_query.argtypes = [vp, ctypes.c_int, vp, ctypes.c_size_t]
    lib.ag_matmul_debug_fill_staging.argtypes = [vp, ctypes.c_uint16, vp]
    lib.ag_matmul_debug_set_runs.argtypes = [vp, ctypes.c_uint32, vp]
    return lib


lib = _load()


# ---- C-named functions (argument marshalling only) ----

def ag_matmul_desc_init(**fields) -> agmm_desc:
    d = agmm_desc()
    lib.ag_matmul_desc_init(ctypes.byref(d))
    for k, v in fields.items():
        if not hasattr(d, k):
            raise AttributeError(f"agmm_desc has no field {k!r}")
        setattr(d, k, int(v))
    return d


def ag_matmul_create(desc: agmm_desc, workspace: Optional[int] = None,
                     workspace_bytes: int = 0) -> int:
    h = ctypes.c_void_p()
    rc = lib.ag_matmul_create(ctypes.byref(desc), ctypes.c_void_p(workspace) if workspace else None,
                              workspace_bytes, ctypes.byref(h))
    if rc != AGMM_OK:
        raise AgmmError(rc, "ag_matmul_create")
    return h.value


def ag_matmul_run(handle: int, shard_ptrs: Sequence[int], B_ptr: int, bias_ptr: Optional[int],
                  out_ptr: int, stream: int = 0) -> int:
    arr = (ctypes.c_void_p * max(1, len(shard_ptrs)))(*[ctypes.c_void_p(p) for p in shard_ptrs])
    return lib.ag_matmul_run(ctypes.c_void_p(handle), arr, ctypes.c_void_p(B_ptr),
                             ctypes.c_void_p(bias_ptr) if bias_ptr else None,
                             ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream))


def ag_matmul_run_gather(handle: int, shard_ptrs: Sequence[int], B_ptr: int,
                         bias_ptr: Optional[int], out_ptr: int, a_ptr: int, stream: int = 0) -> int:
    arr = (ctypes.c_void_p * max(1, len(shard_ptrs)))(*[ctypes.c_void_p(p) for p in shard_ptrs])
    return lib.ag_matmul_run_gather(ctypes.c_void_p(handle), arr, ctypes.c_void_p(B_ptr),
                                    ctypes.c_void_p(bias_ptr) if bias_ptr else None,
                                    ctypes.c_void_p(out_ptr), ctypes.c_void_p(a_ptr),
                                    ctypes.c_void_p(stream))


def ag_matmul_plan_query(desc: agmm_desc, num_cus: int = 256) -> dict:
    """The planner's decisions for `desc` on a device with `num_cus` CUs (host only): the
    config and every schedule table, as ag_matmul_debug_query lays them out."""
    def q(what, nbytes, buf=None):
        buf = buf if buf is not None else (ctypes.c_uint8 * max(1, nbytes))()
        rc = lib.ag_matmul_plan_query(ctypes.byref(desc), num_cus, what, ctypes.byref(buf), nbytes)
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_matmul_plan_query")
        return buf
    cfg = q(0, ctypes.sizeof(agmm_config), agmm_config())
    u32 = lambda what, n: np.frombuffer(bytes(q(what, n * 4))[:n * 4], dtype="<u4")
    out = {"config": cfg,
           "units": u32(Q_UNITS, 2 * cfg.num_units).reshape(-1, 2),
           "mtiles": u32(Q_MTILES, cfg.T_m)}
    raw = u32(Q_QUEUES, 2 * 9 + cfg.num_items)
    out["queues"] = [list(map(int, raw[18 + raw[x]:18 + raw[x] + raw[9 + x]])) for x in range(9)]
    if cfg.pipeline_chunks:
        sizes = u32(Q_CHUNK_SIZES, 2 * cfg.pipeline_chunks).reshape(-1, 2)
        cu = u32(Q_CHUNK_UNITS, 2 * int(sizes[:, 0].sum())).reshape(-1, 2)
        cm = u32(Q_CHUNK_MTILES, int(sizes[:, 1].sum()))
        chunks, u0, m0 = [], 0, 0
        for a, b in sizes:
            chunks.append(([tuple(map(int, r)) for r in cu[u0:u0 + a]], list(map(int, cm[m0:m0 + b]))))
            u0 += int(a)
            m0 += int(b)
        out["chunks"] = chunks
    return out


def ag_matmul_run_static(desc: agmm_desc, shard_ptrs: Sequence[int], B_ptr: int,
                         bias_ptr: Optional[int], out_ptr: int, stream: int = 0) -> int:
    arr = (ctypes.c_void_p * max(1, len(shard_ptrs)))(*[ctypes.c_void_p(p) for p in shard_ptrs])
    return lib.ag_matmul_run_static(ctypes.byref(desc), arr, ctypes.c_void_p(B_ptr),
                                    ctypes.c_void_p(bias_ptr) if bias_ptr else None,
                                    ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream))


def ag_matmul_debug_run_part(handle: int, part: int, shard_ptrs: Sequence[int], B_ptr: int,
                             bias_ptr: Optional[int], out_ptr: int, stream: int = 0) -> int:
    arr = (ctypes.c_void_p * max(1, len(shard_ptrs)))(*[ctypes.c_void_p(p) for p in shard_ptrs])
    return lib.ag_matmul_debug_run_part(ctypes.c_void_p(handle), part, arr, ctypes.c_void_p(B_ptr),
                                        ctypes.c_void_p(bias_ptr) if bias_ptr else None,
                                        ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream))


def ag_matmul_debug_mfma_loop(dtype: int, vary: bool, grid: int, iters: int, sink_ptr: int,
                              stream: int = 0) -> int:
    return lib.ag_matmul_debug_mfma_loop(dtype, int(vary), grid, iters, ctypes.c_void_p(sink_ptr),
                                         ctypes.c_void_p(stream))


def ag_matmul_sync_status(handle: int) -> int:
    return lib.ag_matmul_sync_status(ctypes.c_void_p(handle))


def ag_matmul_destroy(handle: Optional[int]) -> int:
    return lib.ag_matmul_destroy(ctypes.c_void_p(handle) if handle else None)


def ag_matmul_workspace_bytes(desc: agmm_desc) -> int:
    return int(lib.ag_matmul_workspace_bytes(ctypes.byref(desc)))


def strerror(code: int) -> str:
    return lib.ag_matmul_strerror(code).decode()


ag_matmul_strerror = strerror


def last_hip_error() -> int:
    return int(lib.ag_matmul_last_hip_error())


def ag_matmul_get_config(handle: int) -> agmm_config:
    c = agmm_config()
    rc = lib.ag_matmul_get_config(ctypes.c_void_p(handle), ctypes.byref(c))
    if rc != AGMM_OK:
        raise AgmmError(rc, "ag_matmul_get_config")
    return c


def ag_matmul_debug_query(handle: int, what: int, nbytes: int) -> bytes:
    buf = (ctypes.c_uint8 * max(1, nbytes))()
    rc = lib.ag_matmul_debug_query(ctypes.c_void_p(handle), what, buf, nbytes)
    if rc != AGMM_OK:
        raise AgmmError(rc, "ag_matmul_debug_query")
    return bytes(buf)[:nbytes]


def ag_matmul_debug_set_runs(handle: int, runs: int, stream: int = 0) -> int:
    return lib.ag_matmul_debug_set_runs(ctypes.c_void_p(handle), runs & 0xFFFFFFFF,
                                        ctypes.c_void_p(stream))


def ag_matmul_debug_fill_staging(handle: int, pattern: int, stream: int = 0) -> int:
    return lib.ag_matmul_debug_fill_staging(ctypes.c_void_p(handle), pattern & 0xFFFF,
                                            ctypes.c_void_p(stream))


# ---- torch convenience wrapper (pointers and the current stream only) ----

class AgMatmul:
    """One handle for one problem shape. run() takes D shard tensors [M/D, K], B [K, N],
    an optional bias [N] and an output [M, N], all contiguous on the handle's device.
    With gather_a=True, run() also takes (or allocates) a_out [M, K], which receives the
    gathered A, and returns (a_out, out)."""

    def __init__(self, D: int, M: int, N: int, K: int, dtype="f16", layout="k_contiguous",
                 algo="fused", rank: int = 0, direct_local: bool = True, has_bias: bool = False,
                 debug: bool = False, gather_a: bool = False, **tunables):
        self.desc = ag_matmul_desc_init(
            D=D, M=M, N=N, K=K, rank=rank,
            dtype={"f16": F16, "bf16": BF16}[dtype],
            layout={"k_contiguous": K_CONTIGUOUS, "m_contiguous": M_CONTIGUOUS}[layout],
            algo={"fused": ALGO_FUSED, "baseline": ALGO_BASELINE, "pipelined": ALGO_PIPELINED}[algo],
            direct_local=int(direct_local), has_bias=int(has_bias), debug=int(debug),
            gather_a=int(gather_a), **tunables)
        self.dtype = dtype
        self.handle = ag_matmul_create(self.desc)
        self.config = ag_matmul_get_config(self.handle)

    def close(self):
        if self.handle:
            ag_matmul_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def run(self, shards, B, bias=None, out=None, stream=None, check: bool = True, a_out=None):
        import torch
        d = self.desc
        if a_out is not None and not d.gather_a:
            raise ValueError("a_out needs a handle created with gather_a=True")
        if len(shards) != d.D:
            raise ValueError(f"expected {d.D} shards, got {len(shards)}")
        tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        for t in list(shards) + [B] + ([bias] if bias is not None else []):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("inputs must be contiguous device tensors of the handle's dtype")
        if out is None:
            out = torch.empty((d.M, d.N), dtype=tdt, device=B.device)
        s = stream if stream is not None else torch.cuda.current_stream(B.device)
        if d.gather_a:
            if a_out is None:
                a_out = torch.empty((d.M, d.K), dtype=tdt, device=B.device)
            if a_out.dtype != tdt or not a_out.is_cuda or not a_out.is_contiguous() or \
                    tuple(a_out.shape) != (d.M, d.K):
                raise ValueError("a_out must be a contiguous [M, K] device tensor of the handle's dtype")
            rc = ag_matmul_run_gather(self.handle, [t.data_ptr() for t in shards], B.data_ptr(),
                                      bias.data_ptr() if bias is not None else None,
                                      out.data_ptr(), a_out.data_ptr(), s.cuda_stream)
            if check and rc != AGMM_OK:
                raise AgmmError(rc, "ag_matmul_run_gather")
            return a_out, out
        rc = ag_matmul_run(self.handle, [t.data_ptr() for t in shards], B.data_ptr(),
                           bias.data_ptr() if bias is not None else None, out.data_ptr(),
                           s.cuda_stream)
        if check and rc != AGMM_OK:
            raise AgmmError(rc, "ag_matmul_run")
        return out

    # ---- bookkeeping access ----
    def flags(self) -> np.ndarray:
        c = self.config
        n = c.T_m * c.G
        return np.frombuffer(ag_matmul_debug_query(self.handle, Q_FLAGS, n * 4), dtype="<u4")

    def staging(self) -> np.ndarray:
        n = self.config.staging_elems
        return np.frombuffer(ag_matmul_debug_query(self.handle, Q_STAGING, n * 2), dtype="<u2")

    def units(self) -> np.ndarray:
        n = self.config.num_units
        return np.frombuffer(ag_matmul_debug_query(self.handle, Q_UNITS, n * 8),
                             dtype="<u4").reshape(-1, 2)

    def chunks(self):
        """AGMM_ALGO_PIPELINED: per chunk, (units [(m-tile, k-group)], m-tiles in GEMM order
        with bit 31 = read in place)."""
        S = self.config.pipeline_chunks
        sizes = np.frombuffer(ag_matmul_debug_query(self.handle, Q_CHUNK_SIZES, S * 8),
                              dtype="<u4").reshape(-1, 2)
        nu, nm = int(sizes[:, 0].sum()), int(sizes[:, 1].sum())
        units = np.frombuffer(ag_matmul_debug_query(self.handle, Q_CHUNK_UNITS, nu * 8),
                              dtype="<u4").reshape(-1, 2)
        mt = np.frombuffer(ag_matmul_debug_query(self.handle, Q_CHUNK_MTILES, nm * 4), dtype="<u4")
        out, u0, m0 = [], 0, 0
        for a, b in sizes:
            out.append(([tuple(int(x) for x in r) for r in units[u0:u0 + a]],
                        [int(x) for x in mt[m0:m0 + b]]))
            u0 += int(a)
            m0 += int(b)
        return out

    def mtiles(self) -> np.ndarray:
        n = self.config.T_m
        return np.frombuffer(ag_matmul_debug_query(self.handle, Q_MTILES, n * 4), dtype="<u4")

    def queues(self):
        """The 9 queues (8 per-XCD, then the tail queue of split-tile pieces) as lists of
        entries: tile id | piece << 24 | (pieces - 1) << 28."""
        n = self.config.num_items
        raw = np.frombuffer(ag_matmul_debug_query(self.handle, Q_QUEUES, (18 + n) * 4), dtype="<u4")
        off, ln, ents = raw[:9], raw[9:18], raw[18:]
        return [list(map(int, ents[o:o + l])) for o, l in zip(off, ln)]

    def partials(self) -> np.ndarray:
        """fp32 partial sums of the split tiles, [split tile][piece][block_m * block_n] in the
        slot layout of AGMM_Q_PARTIALS."""
        c = self.config
        n = c.split_tiles * c.split_pieces * c.block_m * c.block_n
        raw = np.frombuffer(ag_matmul_debug_query(self.handle, Q_PARTIALS, n * 4), dtype="<f4")
        return raw.reshape(c.split_tiles, max(1, c.split_pieces), c.block_m * c.block_n)

    def status(self) -> np.ndarray:
        return np.frombuffer(ag_matmul_debug_query(self.handle, Q_STATUS, 16), dtype="<u4")

    def run_part(self, part: int, shards, B, bias=None, out=None, check: bool = True):
        """A baseline handle's copy (PART_COPY) or GEMM (PART_GEMM) phase alone."""
        import torch
        d = self.desc
        tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        if out is None:
            out = torch.empty((d.M, d.N), dtype=tdt, device=B.device)
        rc = ag_matmul_debug_run_part(self.handle, part, [t.data_ptr() for t in shards],
                                      B.data_ptr(), bias.data_ptr() if bias is not None else None,
                                      out.data_ptr(), torch.cuda.current_stream(B.device).cuda_stream)
        if check and rc != AGMM_OK:
            raise AgmmError(rc, "ag_matmul_debug_run_part")
        return out

    def sync_status(self) -> int:
        """Waits for the device; AGMM_OK, or the TIMEOUT / POISONED code of a recorded
        flag-wait timeout."""
        return ag_matmul_sync_status(self.handle)

    def trace(self):
        """Per-workgroup trace counts and records: the persistent grid's workgroups, then (with
        a fetch kernel) the fetch kernel's."""
        c = self.config
        W = c.num_wgs + (c.num_fetch_wgs if c.fetch_kernel else 0)
        counts = np.frombuffer(ag_matmul_debug_query(self.handle, Q_TRACE_COUNT, W * 4), dtype="<u4")
        recs = np.frombuffer(ag_matmul_debug_query(self.handle, Q_TRACE,
                                                   W * c.trace_cap * TRACE_DTYPE.itemsize),
                             dtype=TRACE_DTYPE).reshape(W, c.trace_cap)
        return counts, recs

    def set_runs(self, runs: int, stream=None):
        """Test knob: put the flags, split counters and device run counter where `runs` runs
        would have left them (ag_matmul_debug_set_runs)."""
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = ag_matmul_debug_set_runs(self.handle, runs, s.cuda_stream)
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_matmul_debug_set_runs")

    def fill_staging(self, pattern: int, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = ag_matmul_debug_fill_staging(self.handle, pattern, s.cuda_stream)
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_matmul_debug_fill_staging")


class GemmAllReduce:
    """One rank's share of GEMM + all-reduce (atomics): run() adds A_local @ B_local (fp32)
    into each of the D result buffers; finalize() rounds one buffer (+ bias) to 16 bits."""

    def __init__(self, D: int, rank: int, M: int, N: int, K_local: int, dtype="f16",
                 block_m: int = 0):
        h = ctypes.c_void_p()
        rc = lib.ag_gemm_ar_create(D, rank, M, N, K_local, {"f16": F16, "bf16": BF16}[dtype],
                                   block_m, ctypes.byref(h))
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_gemm_ar_create")
        self.handle, self.D, self.M, self.N, self.K, self.dtype = h.value, D, M, N, K_local, dtype
        self.config = ag_matmul_get_config(self.handle)

    def close(self):
        if self.handle:
            ag_matmul_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, A_local, B_local, C, stream=None, check: bool = True) -> int:
        import torch
        if len(C) != self.D:
            raise ValueError(f"expected {self.D} result buffers")
        for t in C:
            if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise ValueError("result buffers must be contiguous fp32 device tensors")
        s = stream if stream is not None else torch.cuda.current_stream(A_local.device)
        arr = (ctypes.c_void_p * self.D)(*[ctypes.c_void_p(t.data_ptr()) for t in C])
        rc = lib.ag_gemm_ar_run(ctypes.c_void_p(self.handle), ctypes.c_void_p(A_local.data_ptr()),
                                ctypes.c_void_p(B_local.data_ptr()), arr,
                                ctypes.c_void_p(s.cuda_stream))
        if check and rc != AGMM_OK:
            raise AgmmError(rc, "ag_gemm_ar_run")
        return rc

    def finalize(self, C, bias=None, out=None, stream=None):
        import torch
        tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        if out is None:
            out = torch.empty((self.M, self.N), dtype=tdt, device=C.device)
        s = stream if stream is not None else torch.cuda.current_stream(C.device)
        rc = lib.ag_gemm_ar_finalize(ctypes.c_void_p(self.handle), ctypes.c_void_p(C.data_ptr()),
                                     ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_gemm_ar_finalize")
        return out


class GemmAllReduceFlags:
    """GEMM + all-reduce with a ready flag per tile, every rank's share in one launch:
    run(A_parts, B_parts, bias) returns RNE(sum_r A_parts[r] @ B_parts[r] + bias)."""

    def __init__(self, D: int, M: int, N: int, K_local: int, dtype="f16", block_m: int = 0):
        h = ctypes.c_void_p()
        rc = lib.ag_gemm_ar_flags_create(D, M, N, K_local, {"f16": F16, "bf16": BF16}[dtype],
                                         block_m, ctypes.byref(h))
        if rc != AGMM_OK:
            raise AgmmError(rc, "ag_gemm_ar_flags_create")
        self.handle, self.D, self.M, self.N, self.K, self.dtype = h.value, D, M, N, K_local, dtype
        self.config = ag_matmul_get_config(self.handle)

    def close(self):
        if self.handle:
            ag_matmul_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, A_parts, B_parts, bias=None, out=None, stream=None, check: bool = True):
        import torch
        if len(A_parts) != self.D or len(B_parts) != self.D:
            raise ValueError(f"expected {self.D} A and B parts")
        tdt = torch.float16 if self.dtype == "f16" else torch.bfloat16
        for t in list(A_parts) + list(B_parts) + ([bias] if bias is not None else []):
            if t.dtype != tdt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("inputs must be contiguous device tensors of the handle's type")
        if out is None:
            out = torch.empty((self.M, self.N), dtype=tdt, device=A_parts[0].device)
        s = stream if stream is not None else torch.cuda.current_stream(out.device)
        ap = (ctypes.c_void_p * self.D)(*[ctypes.c_void_p(t.data_ptr()) for t in A_parts])
        bp = (ctypes.c_void_p * self.D)(*[ctypes.c_void_p(t.data_ptr()) for t in B_parts])
        rc = lib.ag_gemm_ar_flags_run(ctypes.c_void_p(self.handle), ap, bp,
                                      ctypes.c_void_p(bias.data_ptr()) if bias is not None else None,
                                      ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
        if check and rc != AGMM_OK:
            raise AgmmError(rc, "ag_gemm_ar_flags_run")
        return out


def ag_gemm_ar_flags_plan(D: int, M: int, N: int, K_local: int, dtype="f16", block_m: int = 0,
                          num_cus: int = 256):
    """Host only: (config dict, item list) that a per-tile flag handle would use."""
    import numpy as np
    cfg = agmm_config()
    n = ctypes.c_int64(0)
    dt = {"f16": F16, "bf16": BF16}[dtype]
    rc = lib.ag_gemm_ar_flags_plan(D, M, N, K_local, dt, block_m, num_cus, ctypes.byref(cfg),
                                   None, ctypes.byref(n))
    if rc != AGMM_OK:
        raise AgmmError(rc, "ag_gemm_ar_flags_plan")
    items = np.zeros(n.value, dtype=np.uint32)
    rc = lib.ag_gemm_ar_flags_plan(D, M, N, K_local, dt, block_m, num_cus, None,
                                   items.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                   ctypes.byref(n))
    if rc != AGMM_OK:
        raise AgmmError(rc, "ag_gemm_ar_flags_plan")
    return cfg.as_dict(), items
