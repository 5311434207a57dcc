"""gradient_sync_amd: data-parallel gradient and parameter synchronisation on
one MI355X, with K data-parallel ranks emulated as K buffers in HBM.

This module is a thin ctypes binding over libdpsync.so (include/dpsync.h).
It only marshals arguments: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and a non-zero status becomes a
DpsyncError. Every step of the computation runs in the library's HIP kernels;
there is no fallback path. If libdpsync.so has not been built this import
fails loudly.

Calls (same names and meaning as the C ABI):
  dp_reduce_scatter(send, recv, op="sum", s_chunks=1, stream=None)
  dp_all_gather(send, recv, n=None, s_chunks=1, stream=None)
  dp_all_reduce(send, recv, op="sum", s_chunks=1, stream=None)
  dp_weighted_reduce(send, recv, tokens, s_chunks=1, stream=None)
  dp_fsdp_layer(x_local, w_shard, dy_local, w_full, y_local, dw_full, dw_shard, stream=None,
                dx_local=None)                # dx_local: dp_fsdp_layer_ex
  dp_gemm_bf16(a, b, c, stream=None)          # c = a @ b (b_layout="nk": a @ b.T)
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to

__all__ = [
    "DpsyncError", "lib", "dp_shard_len", "dp_status_string", "dp_last_hip_error", "dp_version",
    "dp_reduce_scatter", "dp_all_gather", "dp_all_reduce", "dp_weighted_reduce",
    "dp_fsdp_layer", "dp_gemm_bf16", "DP_MAX_K", "EXPORTS", "LaunchOpts",
    "dp_reduce_scatter_ex", "dp_all_gather_ex", "dp_all_reduce_ex", "dp_gemm_bf16_ex",
    "dp_weighted_reduce_ex", "dp_scatter_accumulate", "dp_settle", "GradPiece", "HipEvents",
    "dp_backward_allreduce_overlap", "dp_reduce_scatter_all_gather", "dp_fsdp_layer_static",
    "DP_STATIC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpsync.so")

DP_OK, DP_ERR_INVALID_ARG, DP_ERR_UNSUPPORTED, DP_ERR_ALIAS, DP_ERR_HIP, DP_ERR_SCRATCH = range(6)
DP_STATIC_SCRATCH_BYTES = 32 << 20      # include/dpsync.h
DP_F32, DP_BF16, DP_I32 = 0, 1, 2
DP_SUM, DP_AVG = 0, 1
DP_MAX_K = 64

# every symbol include/dpsync.h declares
EXPORTS = ("dp_shard_len", "dp_status_string", "dp_last_hip_error", "dp_version",
           "dp_reduce_scatter", "dp_all_gather", "dp_all_reduce", "dp_weighted_reduce",
           "dp_fsdp_layer", "dp_gemm_bf16", "dp_reduce_scatter_ex", "dp_all_gather_ex",
           "dp_all_reduce_ex", "dp_gemm_bf16_ex", "dp_weighted_reduce_ex",
           "dp_scatter_accumulate", "dp_settle", "dp_backward_allreduce_overlap",
           "dp_reduce_scatter_all_gather", "dp_fsdp_layer_ex", "dp_fsdp_layer_static")

_DTYPES = {torch.float32: DP_F32, torch.bfloat16: DP_BF16, torch.int32: DP_I32}
_OPS = {"sum": DP_SUM, "avg": DP_AVG}
DP_LAUNCH_SHARE_CU = 1
DP_LAUNCH_TWO_PHASE = 2
DP_LAUNCH_LEAN = 4
DP_LAUNCH_B_NK = 8

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t
_lib = None


class LaunchOpts(ctypes.Structure):
    """dp_launch_opts_t: max_workgroups (0 = one workgroup per tile), flags."""
    _fields_ = [("max_workgroups", ctypes.c_int), ("flags", ctypes.c_int),
                ("reserved", ctypes.c_int * 2)]

    @classmethod
    def make(cls, max_workgroups: int = 0, share_cu: bool = False, two_phase: bool = False,
             lean: bool = False):
        flags = ((DP_LAUNCH_SHARE_CU if share_cu else 0) | (DP_LAUNCH_TWO_PHASE if two_phase else 0)
                 | (DP_LAUNCH_LEAN if lean else 0))
        return cls(max_workgroups, flags, (ctypes.c_int * 2)(0, 0))


class GradPiece(ctypes.Structure):
    """dp_grad_piece_t: an [m, n] weight gradient at element `offset` of the
    flat per-rank gradient vector."""
    _fields_ = [("offset", ctypes.c_int64), ("m", ctypes.c_int64), ("n", ctypes.c_int64)]


class HipEvents:
    """n hipEvent_t handles (timing disabled) from the HIP runtime the process
    already uses, for the calls that order two streams with caller-owned
    events. Destroyed with the object."""

    _hip = None

    def __init__(self, n: int):
        if HipEvents._hip is None:
            h = ctypes.CDLL("libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_vp), ctypes.c_uint]
            h.hipEventCreateWithFlags.restype = _int
            h.hipEventDestroy.argtypes = [_vp]
            h.hipEventDestroy.restype = _int
            HipEvents._hip = h
        self.handles = []
        for _ in range(n):
            ev = _vp()
            rc = HipEvents._hip.hipEventCreateWithFlags(ctypes.byref(ev), 0x2)   # hipEventDisableTiming
            if rc != 0:
                self.close()
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
            self.handles.append(ev.value)
        self.array = (_vp * max(1, n))(*self.handles)

    def close(self):
        for h in self.handles:
            HipEvents._hip.hipEventDestroy(_vp(h))
        self.handles = []

    def __len__(self):
        return len(self.handles)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DpsyncError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = dp_status_string(code)
        if code == DP_ERR_HIP:
            msg += f" (hipError {dp_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def lib():
    """The loaded libdpsync (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.dp_shard_len.restype = _sz
        L.dp_shard_len.argtypes = [_sz, _int]
        L.dp_status_string.restype = ctypes.c_char_p
        L.dp_status_string.argtypes = [_int]
        L.dp_last_hip_error.restype = _int
        L.dp_last_hip_error.argtypes = []
        L.dp_version.restype = _int
        L.dp_version.argtypes = []
        L.dp_reduce_scatter.restype = _int
        L.dp_reduce_scatter.argtypes = [_vp, _vp, _sz, _int, _int, _int, _int, _vp]
        L.dp_all_gather.restype = _int
        L.dp_all_gather.argtypes = [_vp, _vp, _sz, _int, _int, _int, _vp]
        L.dp_all_reduce.restype = _int
        L.dp_all_reduce.argtypes = [_vp, _vp, _sz, _int, _int, _int, _int, _vp]
        L.dp_weighted_reduce.restype = _int
        L.dp_weighted_reduce.argtypes = [_vp, _vp, _vp, _sz, _int, _int, _int, _vp]
        L.dp_fsdp_layer.restype = _int
        L.dp_fsdp_layer.argtypes = [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.dp_fsdp_layer_ex.restype = _int
        L.dp_fsdp_layer_ex.argtypes = [_int, _i64, _i64, _i64] + [_vp] * 9
        L.dp_fsdp_layer_static.restype = _int
        L.dp_fsdp_layer_static.argtypes = [_int, _i64, _i64, _i64] + [_vp] * 7
        L.dp_gemm_bf16.restype = _int
        L.dp_gemm_bf16.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp]
        P = ctypes.POINTER(LaunchOpts)
        L.dp_reduce_scatter_ex.restype = _int
        L.dp_reduce_scatter_ex.argtypes = [_vp, _vp, _sz, _int, _int, _int, _int, P, _vp]
        L.dp_all_gather_ex.restype = _int
        L.dp_all_gather_ex.argtypes = [_vp, _vp, _sz, _int, _int, _int, P, _vp]
        L.dp_all_reduce_ex.restype = _int
        L.dp_all_reduce_ex.argtypes = [_vp, _vp, _sz, _int, _int, _int, _int, P, _vp]
        L.dp_gemm_bf16_ex.restype = _int
        L.dp_gemm_bf16_ex.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, P, _vp]
        L.dp_weighted_reduce_ex.restype = _int
        L.dp_weighted_reduce_ex.argtypes = [_vp, _vp, _vp, _sz, _int, _int, _int, P, _vp]
        L.dp_scatter_accumulate.restype = _int
        L.dp_scatter_accumulate.argtypes = [_vp, _int, _int, _vp, _sz, _int, _vp]
        L.dp_settle.restype = _int
        L.dp_reduce_scatter_all_gather.restype = _int
        L.dp_reduce_scatter_all_gather.argtypes = [_vp, _vp, _sz, _vp, _vp, _sz, _int, _int, _int,
                                                   _int, _vp]
        L.dp_backward_allreduce_overlap.restype = _int
        L.dp_backward_allreduce_overlap.argtypes = [
            _int, _int, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _int, P, _vp, _vp, _vp, _int]
        L.dp_settle.argtypes = [_vp, _vp, _sz, _int, _int, ctypes.c_float, _int, _vp]
        _lib = L
    return _lib


def dp_shard_len(n: int, k: int) -> int:
    return int(lib().dp_shard_len(n, k))


def dp_status_string(code: int) -> str:
    return lib().dp_status_string(code).decode()


def dp_last_hip_error() -> int:
    return int(lib().dp_last_hip_error())


def dp_version() -> int:
    return int(lib().dp_version())


# ----------------------------------------------------------------- marshalling

def ptr_array(ptrs):
    """Host array of device pointers (ints), as the ABI's `const void* const*`."""
    arr = (_vp * max(1, len(ptrs)))(*[int(p) for p in ptrs])
    return arr


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(int(stream))


def _check(code: int, where: str):
    if code != DP_OK:
        raise DpsyncError(code, where)


def _tensors(ts, what, dtype=None):
    ts = list(ts)
    if not ts:
        raise ValueError(f"{what}: need at least one rank")
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{what}: expected torch tensors")
        if t.device.type != "cuda":
            raise ValueError(f"{what}: tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{what}: tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if len({t.dtype for t in ts}) != 1:
        raise TypeError(f"{what}: all ranks must share one dtype")
    return ts


def _dt(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _numel_check(ts, n, what):
    for t in ts:
        if t.numel() < n:
            raise ValueError(f"{what}: buffer of {t.numel()} elements, need {n}")


# ----------------------------------------------------------------- the calls

def _rs(send, recv, op, s_chunks, stream, n, opts):
    send = _tensors(send, "send")
    recv = _tensors(recv, "recv", send[0].dtype)
    k = len(send)
    n = send[0].numel() if n is None else n
    _numel_check(send, n, "send")
    _numel_check(recv, dp_shard_len(n, k), "recv")
    if len(recv) != k:
        raise ValueError("send and recv need one buffer per rank")
    args = (ptr_array([t.data_ptr() for t in send]), ptr_array([t.data_ptr() for t in recv]), n, k,
            _dt(send[0]), _OPS[op], s_chunks)
    if opts is None:
        _check(lib().dp_reduce_scatter(*args, _stream(stream)), "dp_reduce_scatter")
    else:
        _check(lib().dp_reduce_scatter_ex(*args, opts, _stream(stream)), "dp_reduce_scatter_ex")


def dp_reduce_scatter(send, recv, op: str = "sum", s_chunks: int = 1, stream=None, n=None):
    """recv[c] (ceil(n/K) elements) <- shard c of the ring-order sum of send[r]."""
    _rs(send, recv, op, s_chunks, stream, n, None)


def dp_reduce_scatter_ex(send, recv, op: str = "sum", s_chunks: int = 1, max_workgroups: int = 0,
                         stream=None, n=None, lean: bool = False):
    """dp_reduce_scatter with a cap on resident workgroups (0 = default grid)
    and the lean (64-VGPR) kernel variant."""
    _rs(send, recv, op, s_chunks, stream, n,
        ctypes.byref(LaunchOpts.make(max_workgroups, lean=lean)))


def _ag(send, recv, n, s_chunks, stream, opts):
    send = _tensors(send, "send")
    recv = _tensors(recv, "recv", send[0].dtype)
    k = len(send)
    n = recv[0].numel() if n is None else n
    _numel_check(recv, n, "recv")
    L = dp_shard_len(n, k)
    for c, t in enumerate(send):
        _numel_check([t], max(0, min(L, n - c * L)), f"send[{c}]")
    if len(recv) != k:
        raise ValueError("send and recv need one buffer per rank")
    args = (ptr_array([t.data_ptr() for t in send]), ptr_array([t.data_ptr() for t in recv]), n, k,
            _dt(send[0]), s_chunks)
    if opts is None:
        _check(lib().dp_all_gather(*args, _stream(stream)), "dp_all_gather")
    else:
        _check(lib().dp_all_gather_ex(*args, opts, _stream(stream)), "dp_all_gather_ex")


def dp_all_gather(send, recv, n=None, s_chunks: int = 1, stream=None):
    """recv[r][c*L + j] <- send[c][j] for the valid elements of every shard."""
    _ag(send, recv, n, s_chunks, stream, None)


def dp_all_gather_ex(send, recv, n=None, s_chunks: int = 1, max_workgroups: int = 0, stream=None):
    _ag(send, recv, n, s_chunks, stream, ctypes.byref(LaunchOpts.make(max_workgroups)))


def _ar(send, recv, op, s_chunks, stream, n, opts):
    send = _tensors(send, "send")
    recv = _tensors(recv, "recv", send[0].dtype)
    k = len(send)
    n = send[0].numel() if n is None else n
    _numel_check(send, n, "send")
    _numel_check(recv, n, "recv")
    if len(recv) != k:
        raise ValueError("send and recv need one buffer per rank")
    args = (ptr_array([t.data_ptr() for t in send]), ptr_array([t.data_ptr() for t in recv]), n, k,
            _dt(send[0]), _OPS[op], s_chunks)
    if opts is None:
        _check(lib().dp_all_reduce(*args, _stream(stream)), "dp_all_reduce")
    else:
        _check(lib().dp_all_reduce_ex(*args, opts, _stream(stream)), "dp_all_reduce_ex")


def dp_all_reduce(send, recv, op: str = "sum", s_chunks: int = 1, stream=None, n=None):
    _ar(send, recv, op, s_chunks, stream, n, None)


def dp_all_reduce_ex(send, recv, op: str = "sum", s_chunks: int = 1, max_workgroups: int = 0,
                     two_phase: bool = False, stream=None, n=None, lean: bool = False):
    """dp_all_reduce with launch options; two_phase runs ReduceScatter then
    AllGather instead of the one-pass kernel, lean the 64-VGPR kernel variant
    (same results either way)."""
    _ar(send, recv, op, s_chunks, stream, n,
        ctypes.byref(LaunchOpts.make(max_workgroups, two_phase=two_phase, lean=lean)))


def _wr(send, recv, tokens, s_chunks, stream, n, opts):
    send = _tensors(send, "send")
    recv = _tensors(recv, "recv", send[0].dtype)
    k = len(send)
    n = send[0].numel() if n is None else n
    _numel_check(send, n, "send")
    _numel_check(recv, n, "recv")
    if len(recv) != k or len(tokens) != k:
        raise ValueError("send, recv and tokens need one entry per rank")
    toks = (ctypes.c_int64 * k)(*[int(t) for t in tokens])
    args = (ptr_array([t.data_ptr() for t in send]), ptr_array([t.data_ptr() for t in recv]), toks,
            n, k, _dt(send[0]), s_chunks)
    if opts is None:
        _check(lib().dp_weighted_reduce(*args, _stream(stream)), "dp_weighted_reduce")
    else:
        _check(lib().dp_weighted_reduce_ex(*args, opts, _stream(stream)), "dp_weighted_reduce_ex")


def dp_weighted_reduce(send, recv, tokens, s_chunks: int = 1, stream=None, n=None):
    """recv[r] <- sum_r f32(t_r) send[r] / f32(sum_r t_r), on every rank."""
    _wr(send, recv, tokens, s_chunks, stream, n, None)


def dp_weighted_reduce_ex(send, recv, tokens, s_chunks: int = 1, max_workgroups: int = 0,
                          two_phase: bool = False, stream=None, n=None, lean: bool = False):
    _wr(send, recv, tokens, s_chunks, stream, n,
        ctypes.byref(LaunchOpts.make(max_workgroups, two_phase=two_phase, lean=lean)))


def dp_fsdp_layer(x_local, w_shard, dy_local, w_full, y_local, dw_full=None, dw_shard=None,
                  stream=None, dx_local=None):
    """FSDP layer step over K ranks (fp32): gather W, y = x W, dW = x^T dy, RS(dW);
    with dx_local (needs dy_local) also the input gradient dx = dy W^T."""
    f32 = torch.float32
    x_local = _tensors(x_local, "x_local", f32)
    w_shard = _tensors(w_shard, "w_shard", f32)
    w_full = _tensors(w_full, "w_full", f32)
    y_local = _tensors(y_local, "y_local", f32)
    k = len(x_local)
    m_local, d = x_local[0].shape
    f = w_full[0].shape[1]
    bwd = dy_local is not None
    if bwd:
        dy_local = _tensors(dy_local, "dy_local", f32)
        dw_full = _tensors(dw_full, "dw_full", f32)
        dw_shard = _tensors(dw_shard, "dw_shard", f32)
    want_dx = dx_local is not None
    if want_dx:
        if not bwd:
            raise ValueError("dx_local needs dy_local")
        dx_local = _tensors(dx_local, "dx_local", f32)
    R = dp_shard_len(d, k)
    for name, ts, shape in ((("dx_local", dx_local, (m_local, d)),) if want_dx else ()) + (
            ("x_local", x_local, (m_local, d)), ("w_shard", w_shard, (R, f)),
                            ("w_full", w_full, (d, f)), ("y_local", y_local, (m_local, f))) + (
            (("dy_local", dy_local, (m_local, f)), ("dw_full", dw_full, (d, f)),
             ("dw_shard", dw_shard, (R, f))) if bwd else ()):
        if len(ts) != k or any(tuple(t.shape) != shape for t in ts):
            raise ValueError(f"{name}: expected {k} tensors of shape {shape}")
    P = lambda ts: ptr_array([t.data_ptr() for t in ts])
    if want_dx:
        _check(lib().dp_fsdp_layer_ex(k, m_local, d, f, P(x_local), P(w_shard), P(dy_local),
                                      P(w_full), P(y_local), P(dx_local), P(dw_full),
                                      P(dw_shard), _stream(stream)), "dp_fsdp_layer_ex")
        return
    _check(lib().dp_fsdp_layer(k, m_local, d, f, P(x_local), P(w_shard),
                               P(dy_local) if bwd else None, P(w_full), P(y_local),
                               P(dw_full) if bwd else None, P(dw_shard) if bwd else None,
                               _stream(stream)), "dp_fsdp_layer")


def dp_fsdp_layer_static(x_local, w_shard, dy_local, y_local, dw_shard=None, dx_local=None,
                         stream=None):
    """dp_fsdp_layer (with dx_local: dp_fsdp_layer_ex) without caller
    workspaces: the gathered W and the per-rank dW live in the library's
    static device buffer, so the call allocates nothing. Calls on one GPU that
    can overlap race on that buffer."""
    f32 = torch.float32
    x_local = _tensors(x_local, "x_local", f32)
    w_shard = _tensors(w_shard, "w_shard", f32)
    y_local = _tensors(y_local, "y_local", f32)
    k = len(x_local)
    m_local, d = x_local[0].shape
    f = y_local[0].shape[1]
    bwd = dy_local is not None
    if bwd:
        dy_local = _tensors(dy_local, "dy_local", f32)
        dw_shard = _tensors(dw_shard, "dw_shard", f32)
    if dx_local is not None:
        dx_local = _tensors(dx_local, "dx_local", f32)
    R = dp_shard_len(d, k)
    shapes = [("x_local", x_local, (m_local, d)), ("w_shard", w_shard, (R, f)),
              ("y_local", y_local, (m_local, f))]
    if bwd:
        shapes += [("dy_local", dy_local, (m_local, f)), ("dw_shard", dw_shard, (R, f))]
    if dx_local is not None:
        shapes.append(("dx_local", dx_local, (m_local, d)))
    for name, ts, shape in shapes:
        if len(ts) != k or any(tuple(t.shape) != shape for t in ts):
            raise ValueError(f"{name}: expected {k} tensors of shape {shape}")
    P = lambda ts: ptr_array([t.data_ptr() for t in ts]) if ts is not None else None
    _check(lib().dp_fsdp_layer_static(k, m_local, d, f, P(x_local), P(w_shard), P(dy_local),
                                      P(y_local), P(dx_local), P(dw_shard), _stream(stream)),
           "dp_fsdp_layer_static")


def _gemm(a, b, c, stream, opts, b_nk=False):
    for name, t in (("a", a), ("b", b), ("c", c)):
        _tensors([t], name, torch.bfloat16)
    m, kk = a.shape
    n = b.shape[0] if b_nk else b.shape[1]
    if (b.shape[1] if b_nk else b.shape[0]) != kk or tuple(c.shape) != (m, n):
        raise ValueError("dp_gemm_bf16: shapes must be a[m,k], " +
                         ("b[n,k]" if b_nk else "b[k,n]") + ", c[m,n]")
    if opts is None:
        _check(lib().dp_gemm_bf16(a.data_ptr(), b.data_ptr(), c.data_ptr(), m, n, kk,
                                  _stream(stream)), "dp_gemm_bf16")
    else:
        _check(lib().dp_gemm_bf16_ex(a.data_ptr(), b.data_ptr(), c.data_ptr(), m, n, kk, opts,
                                     _stream(stream)), "dp_gemm_bf16_ex")


def dp_gemm_bf16(a, b, c, stream=None):
    """c[m,n] = a[m,kk] @ b[kk,n] in bf16 with fp32 accumulation."""
    _gemm(a, b, c, stream, None)


def dp_gemm_bf16_ex(a, b, c, share_cu: bool = False, stream=None, lean: bool = False,
                    b_layout: str = "kn"):
    """dp_gemm_bf16 with a variant choice and B's layout: b_layout "kn" (b is
    [kk,n], c = a @ b) or "nk" (b is [n,kk], c = a @ b.T). share_cu selects
    the variant that leaves room for a default sync workgroup on every CU,
    lean the one beside which a lean sync workgroup fits; neither, the fastest
    (same bits)."""
    if b_layout not in ("kn", "nk"):
        raise ValueError("b_layout must be 'kn' or 'nk'")
    b_nk = b_layout == "nk"
    o = LaunchOpts.make(0, share_cu, lean=lean)
    if b_nk:
        o.flags |= DP_LAUNCH_B_NK
    _gemm(a, b, c, stream, ctypes.byref(o), b_nk)


def dp_scatter_accumulate(grads, acc, stream=None, n=None):
    """Apply the pushes `grads` (one tensor or a list, in push order) to the K
    owners' fp32 accumulators: acc[c][j] += f32(g[c*L + j]) for each g in turn
    (ODC scatter-accumulate)."""
    if isinstance(grads, torch.Tensor):
        grads = [grads]
    grads = _tensors(grads, "grads")
    acc = _tensors(acc, "acc", torch.float32)
    k = len(acc)
    n = grads[0].numel() if n is None else n
    _numel_check(grads, n, "grads")
    _numel_check(acc, dp_shard_len(n, k), "acc")
    if grads[0].dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("grads must be float32 or bfloat16")
    _check(lib().dp_scatter_accumulate(ptr_array([t.data_ptr() for t in grads]), len(grads),
                                       _dt(grads[0]), ptr_array([t.data_ptr() for t in acc]), n, k,
                                       _stream(stream)), "dp_scatter_accumulate")


def dp_settle(acc, out, n, divisor: float = 1.0, reset: bool = False, stream=None):
    """out[c][j] = cast(acc[c][j] / divisor), pads zero; optionally zero the
    accumulators afterwards (ODC per-minibatch settle)."""
    acc = _tensors(acc, "acc", torch.float32)
    out = _tensors(out, "out")
    k = len(acc)
    if len(out) != k:
        raise ValueError("acc and out need one buffer per owner")
    L = dp_shard_len(n, k)
    _numel_check(acc, L, "acc")
    _numel_check(out, L, "out")
    if out[0].dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _check(lib().dp_settle(ptr_array([t.data_ptr() for t in acc]),
                           ptr_array([t.data_ptr() for t in out]), n, k, _dt(out[0]),
                           float(divisor), 1 if reset else 0, _stream(stream)), "dp_settle")


def dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, bucket_elems, op="avg",
                                  compute_stream=None, comm_stream=None, events=None,
                                  max_workgroups=0, share_cu=False, two_phase=False, lean=False):
    """Backward weight gradients (bf16 GEMMs, piece by piece for every rank) on
    compute_stream, with each bucket AllReduced on comm_stream as soon as it is
    complete. pieces: list of (offset, m, n); dy, x: lists indexed [g*k + r] of
    [m, t] / [n, t] bf16 tensors; grad, out: K flat bf16 vectors. With
    comm_stream equal to compute_stream (the default: both the current
    stream) the whole pass runs on one stream."""
    grad = _tensors(grad, "grad", torch.bfloat16)
    out = _tensors(out, "out", torch.bfloat16)
    k = len(grad)
    total = grad[0].numel()
    _numel_check(out, total, "out")
    n_pieces = len(pieces)
    dy = _tensors(dy, "dy", torch.bfloat16)
    x = _tensors(x, "x", torch.bfloat16)
    if len(dy) != n_pieces * k or len(x) != n_pieces * k or len(out) != k:
        raise ValueError("need one dy and one x per (piece, rank) and one out per rank")
    for g, (_, m, n) in enumerate(pieces):
        for r in range(k):
            _numel_check([dy[g * k + r]], m * t, "dy")
            _numel_check([x[g * k + r]], n * t, "x")
    arr = (GradPiece * n_pieces)(*[GradPiece(o, m, n) for o, m, n in pieces])
    cs = _stream(compute_stream)
    ms = _stream(comm_stream) if comm_stream is not None else cs
    ev = events.array if events is not None else None
    nev = len(events) if events is not None else 0
    opts = LaunchOpts.make(max_workgroups, share_cu=share_cu, two_phase=two_phase, lean=lean)
    _check(lib().dp_backward_allreduce_overlap(
        k, n_pieces, arr, t, ptr_array([a.data_ptr() for a in dy]),
        ptr_array([b.data_ptr() for b in x]), ptr_array([g.data_ptr() for g in grad]),
        ptr_array([o.data_ptr() for o in out]), total, bucket_elems, _OPS[op],
        ctypes.byref(opts), cs, ms, ev, nev), "dp_backward_allreduce_overlap")


def dp_reduce_scatter_all_gather(rs_send, rs_recv, ag_send, ag_recv, op: str = "sum",
                                 rs_n=None, ag_n=None, s_chunks: int = 1, stream=None):
    """ReduceScatter of (rs_send -> rs_recv) and AllGather of (ag_send ->
    ag_recv) in one launch; the two buffer sets must be disjoint."""
    rs_send = _tensors(rs_send, "rs_send")
    dt = rs_send[0].dtype
    rs_recv = _tensors(rs_recv, "rs_recv", dt)
    ag_send = _tensors(ag_send, "ag_send", dt)
    ag_recv = _tensors(ag_recv, "ag_recv", dt)
    k = len(rs_send)
    if not (len(rs_recv) == len(ag_send) == len(ag_recv) == k):
        raise ValueError("every buffer set needs one tensor per rank")
    rs_n = rs_send[0].numel() if rs_n is None else rs_n
    ag_n = ag_recv[0].numel() if ag_n is None else ag_n
    _numel_check(rs_send, rs_n, "rs_send")
    _numel_check(rs_recv, dp_shard_len(rs_n, k), "rs_recv")
    _numel_check(ag_send, dp_shard_len(ag_n, k), "ag_send")
    _numel_check(ag_recv, ag_n, "ag_recv")
    P = lambda ts: ptr_array([t.data_ptr() for t in ts])
    _check(lib().dp_reduce_scatter_all_gather(P(rs_send), P(rs_recv), rs_n, P(ag_send),
                                              P(ag_recv), ag_n, k, _dt(rs_send[0]), _OPS[op],
                                              s_chunks, _stream(stream)),
           "dp_reduce_scatter_all_gather")
