"""Oracle for the data-parallel sync path: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the GPU
library (gradient_sync_amd) and never imports it.

The arithmetic lives in dp_oracle.c (built by oracle/build.py into
liboracle.so); this module only marshals numpy arrays. bf16 tensors are
carried as numpy uint16 bit patterns. ring_sim.py is a second, literal
message-passing model of the ring used to pin the closed-form fold order.

Pins that tie this code to the pages and to mathematics (not to itself) are in
tests/test_oracle_pins.py; every function here has at least one. Some
choices are readings rather than facts the pages fix (which rank owns which
chunk, and with it the fp32 fold order; the pad value; bf16 rounding; no
fused multiply-add in the weighted fold; documents per rank in the
token-count recipe). The pins check that the oracle computes each reading
correctly (the literal ring adds in the closed-form order once rank c owns
chunk c; bf16 rounding equals torch's conversion), but no pin can show that
the pages meant that reading rather than another.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

SUM, AVG = 0, 1
ORDERS = {"ring": 0, "rank": 1}
_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.int32): 2}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_shard_len.restype = _i64
        L.orc_shard_len.argtypes = [_i64, _int]
        L.orc_shard_valid.restype = _i64
        L.orc_shard_valid.argtypes = [_i64, _i64, _int]
        L.orc_fold_rank.restype = _int
        L.orc_fold_rank.argtypes = [_int, _int, _int, _int]
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_from_f32.argtypes = [ctypes.c_float]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        for name in ("orc_rs_f32", "orc_rs_bf16"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_vp, _vp, _i64, _i64, _int, _int, _int, _int, _int]
        L.orc_rs_i32.restype = None
        L.orc_rs_i32.argtypes = [_vp, _vp, _i64, _i64, _int, _int, _int, _int]
        for name in ("orc_rs_weighted_f32", "orc_rs_weighted_bf16"):
            getattr(L, name).restype = _int
            getattr(L, name).argtypes = [_vp, _vp, _vp, _i64, _i64, _int, _int, _int, _int]
        for name in ("orc_rs_f32_at", "orc_rs_bf16_at"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_vp, _vp, _i64, _i64, _int, _int, _int, _vp]
        for name in ("orc_fold_f32_at", "orc_fold_bf16_at"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [_vp, _vp, _i64, _int, _int, _int, _vp]
        L.orc_scatter_accumulate.restype = None
        L.orc_scatter_accumulate.argtypes = [_int, _vp, _vp, _i64, _i64, _int]
        L.orc_settle.restype = None
        L.orc_settle.argtypes = [_int, _vp, _vp, _i64, _i64, _int, ctypes.c_float]
        L.orc_ag.restype = None
        L.orc_ag.argtypes = [_int, _vp, _vp, _i64, _i64, _int, _int]
        L.orc_ar.restype = _int
        L.orc_ar.argtypes = [_int, _vp, _vp, _i64, _int, _int, _int, _int]
        L.orc_ar_weighted.restype = _int
        L.orc_ar_weighted.argtypes = [_int, _vp, _vp, _vp, _i64, _int, _int, _int]
        L.orc_gemm_f64.restype = None
        L.orc_gemm_f64.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int]
        L.orc_gemm_bf16_at.restype = None
        L.orc_gemm_bf16_at.argtypes = [_vp, _vp, _i64, _i64, _int, _vp, _vp, _i64, _vp, _vp, _int]
        L.orc_fsdp_layer.restype = None
        L.orc_fsdp_layer.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _int]
        _lib = L
    return _lib


def _ptrs(arrays):
    for a in arrays:
        assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return (_vp * max(1, len(arrays)))(*[a.ctypes.data for a in arrays])


def _dtype_code(arrays):
    dts = {a.dtype for a in arrays}
    assert len(dts) == 1, "all ranks must share one dtype"
    return _DT[dts.pop()]


def shard_len(n: int, k: int) -> int:
    return int(lib().orc_shard_len(n, k))


def shard_valid(n: int, L: int, c: int) -> int:
    return int(lib().orc_shard_valid(n, L, c))


def fold_rank(c: int, m: int, k: int, order: str = "ring") -> int:
    return int(lib().orc_fold_rank(c, m, k, ORDERS[order]))


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Element-wise RNE fp32 -> bf16 bits through the oracle's scalar routine."""
    f = lib().orc_bf16_from_f32
    flat = np.asarray(x, dtype=np.float32).ravel()
    return np.array([f(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def reduce_scatter(xs, op: str = "sum", order: str = "ring", L: int | None = None,
                   write_pads: bool = True, nthreads: int = 1):
    """K shards of length L (default ceil(n/K)); shard c = fold over rho_c."""
    k = len(xs)
    n = int(xs[0].size)
    L = shard_len(n, k) if L is None else L
    dt = _dtype_code(xs)
    outs = [np.zeros(L, dtype=xs[0].dtype) for _ in range(k)]
    if L == 0:
        return outs
    xp, op_ = _ptrs(xs), {"sum": SUM, "avg": AVG}[op]
    if dt == 0:
        lib().orc_rs_f32(xp, _ptrs(outs), n, L, k, op_, ORDERS[order], int(write_pads), nthreads)
    elif dt == 1:
        lib().orc_rs_bf16(xp, _ptrs(outs), n, L, k, op_, ORDERS[order], int(write_pads), nthreads)
    else:
        if op != "sum":
            raise ValueError("int32 supports only sum")
        lib().orc_rs_i32(xp, _ptrs(outs), n, L, k, ORDERS[order], int(write_pads), nthreads)
    return outs


def weighted_reduce_scatter(gs, tokens, order: str = "ring", L: int | None = None,
                            write_pads: bool = True, nthreads: int = 1):
    k = len(gs)
    n = int(gs[0].size)
    L = shard_len(n, k) if L is None else L
    dt = _dtype_code(gs)
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    outs = [np.zeros(L, dtype=gs[0].dtype) for _ in range(k)]
    fn = {0: lib().orc_rs_weighted_f32, 1: lib().orc_rs_weighted_bf16}[dt]
    if L == 0:
        return outs
    rc = fn(_ptrs(gs), _ptrs(outs), t.ctypes.data, n, L, k, ORDERS[order], int(write_pads),
            nthreads)
    if rc != 0:
        raise ValueError("token counts must be >= 0 with a positive total")
    return outs


def rs_at(xs, idx, op: str = "sum", order: str = "ring", L: int | None = None):
    """Reduced values at global indices idx (sampled check of large inputs)."""
    k = len(xs)
    n = int(xs[0].size)
    L = shard_len(n, k) if L is None else L
    dt = _dtype_code(xs)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.zeros(idx.size, dtype=xs[0].dtype)
    fn = {0: lib().orc_rs_f32_at, 1: lib().orc_rs_bf16_at}[dt]
    fn(_ptrs(xs), idx.ctypes.data, idx.size, L, k, {"sum": SUM, "avg": AVG}[op],
       ORDERS[order], out.ctypes.data)
    return out


def fold_at(xs_compact, shard_ids, op: str = "sum", order: str = "ring"):
    """Reduced values of compact samples: xs_compact[r][s] is rank r's value of
    sample s, which belongs to shard shard_ids[s]."""
    k = len(xs_compact)
    dt = _dtype_code(xs_compact)
    sid = np.ascontiguousarray(shard_ids, dtype=np.int32)
    out = np.zeros(sid.size, dtype=xs_compact[0].dtype)
    fn = {0: lib().orc_fold_f32_at, 1: lib().orc_fold_bf16_at}[dt]
    fn(_ptrs(xs_compact), sid.ctypes.data, sid.size, k, {"sum": SUM, "avg": AVG}[op],
       ORDERS[order], out.ctypes.data)
    return out


def scatter_accumulate(g, acc, k: int, L: int | None = None):
    """Push gradient g (n elements) into the K owners' fp32 accumulators acc
    (list of K float32 arrays of length L, updated in place)."""
    n = int(g.size)
    L = shard_len(n, k) if L is None else L
    dt = _dtype_code([g])
    assert dt in (0, 1) and all(a.dtype == np.float32 and a.size >= L for a in acc)
    if n:
        lib().orc_scatter_accumulate(dt, g.ctypes.data, _ptrs(acc), n, L, k)
    return acc


def settle(acc, n: int, k: int, dtype=np.float32, divisor: float = 1.0, L: int | None = None):
    """Final shards from the accumulators: cast(acc / divisor), pads zero."""
    L = shard_len(n, k) if L is None else L
    outs = [np.zeros(L, dtype=dtype) for _ in range(k)]
    if L:
        lib().orc_settle(_DT[np.dtype(dtype)], _ptrs(acc), _ptrs(outs), n, L, k, divisor)
    return outs


def all_gather(shards, n: int, L: int | None = None, nthreads: int = 1):
    k = len(shards)
    L = shard_len(n, k) if L is None else L
    outs = [np.zeros(n, dtype=shards[0].dtype) for _ in range(k)]
    if n:
        lib().orc_ag(shards[0].dtype.itemsize, _ptrs(shards), _ptrs(outs), n, L, k, nthreads)
    return outs


def all_reduce(xs, op: str = "sum", order: str = "ring", nthreads: int = 1):
    k, n = len(xs), int(xs[0].size)
    outs = [np.zeros(n, dtype=xs[0].dtype) for _ in range(k)]
    if n:
        rc = lib().orc_ar(_dtype_code(xs), _ptrs(xs), _ptrs(outs), n, k,
                          {"sum": SUM, "avg": AVG}[op], ORDERS[order], nthreads)
        assert rc == 0
    return outs


def weighted_all_reduce(gs, tokens, order: str = "ring", nthreads: int = 1):
    k, n = len(gs), int(gs[0].size)
    t = np.ascontiguousarray(tokens, dtype=np.int64)
    outs = [np.zeros(n, dtype=gs[0].dtype) for _ in range(k)]
    if n:
        rc = lib().orc_ar_weighted(_dtype_code(gs), _ptrs(gs), _ptrs(outs), t.ctypes.data, n,
                                   k, ORDERS[order], nthreads)
        if rc != 0:
            raise ValueError("token counts must be >= 0 with a positive total")
    return outs


def gemm_f64(a: np.ndarray, b: np.ndarray, trans_a: bool = False, nthreads: int = 1):
    """(C, sum|A||B|) in fp64 for C = op(A) B; a, b fp32 row-major."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    m = a.shape[1] if trans_a else a.shape[0]
    kk = a.shape[0] if trans_a else a.shape[1]
    assert b.shape[0] == kk
    n = b.shape[1]
    c = np.zeros((m, n), dtype=np.float64)
    ab = np.zeros((m, n), dtype=np.float64)
    lib().orc_gemm_f64(a.ctypes.data, b.ctypes.data, c.ctypes.data, ab.ctypes.data, m, n, kk,
                       int(trans_a), nthreads)
    return c, ab


def gemm_bf16_at(a_bits: np.ndarray, b_bits: np.ndarray, rows, cols, nthreads: int = 1,
                 b_layout: str = "kn"):
    """fp64 (value, sum|a||b|) of C[rows[s], cols[s]] for bf16 A [m,kk] (uint16
    bits) and B stored [kk,n] (b_layout "kn": C = A B) or [n,kk] ("nk": C = A B^T)."""
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    if b_layout == "kn":
        kk, n = b.shape
    elif b_layout == "nk":
        n, kk = b.shape
    else:
        raise ValueError("b_layout must be 'kn' or 'nk'")
    assert a.shape[1] == kk
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    vals = np.zeros(rows.size, dtype=np.float64)
    absv = np.zeros(rows.size, dtype=np.float64)
    lib().orc_gemm_bf16_at(a.ctypes.data, b.ctypes.data, n, kk, int(b_layout == "nk"),
                           rows.ctypes.data, cols.ctypes.data, rows.size, vals.ctypes.data,
                           absv.ctypes.data, nthreads)
    return vals, absv


def fsdp_layer(x_local, w_shard, dy_local=None, d: int | None = None, nthreads: int = 1):
    """FSDP layer step on K ranks; returns w_full (fp32), y (fp64) and, with dy,
    dw_full (fp64) and dw_shard (fp64)."""
    k = len(x_local)
    m_local, dd = x_local[0].shape
    d = dd if d is None else d
    f = w_shard[0].shape[1]
    w_full = [np.zeros((d, f), dtype=np.float32) for _ in range(k)]
    y = [np.zeros((m_local, f), dtype=np.float64) for _ in range(k)]
    R = shard_len(d, k)
    dw_full = [np.zeros((d, f), dtype=np.float64) for _ in range(k)]
    dw_shard = [np.zeros((R, f), dtype=np.float64) for _ in range(k)]
    lib().orc_fsdp_layer(k, m_local, d, f, _ptrs(x_local), _ptrs(w_shard),
                         _ptrs(dy_local) if dy_local is not None else None, _ptrs(w_full),
                         _ptrs(y), _ptrs(dw_full), _ptrs(dw_shard), nthreads)
    out = {"w_full": w_full, "y": y}
    if dy_local is not None:
        out["dw_full"] = dw_full
        out["dw_shard"] = dw_shard
    return out
