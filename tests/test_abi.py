"""The C-ABI library loads, exports every symbol include/dpsync.h declares, and
rejects invalid arguments before enqueuing anything. CPU only: every call
below fails validation (or is a no-op), so no device memory is touched and no
kernel is launched."""
import ctypes
import os
import re

import pytest

import gradient_sync_amd as dps
from gradient_sync_amd.buckets import bucket_plan, rank_buffers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dpsync.h")

OK, INVALID, UNSUPPORTED, ALIAS = 0, 1, 2, 3
F32, BF16, I32 = 0, 1, 2
SUM, AVG = 0, 1
P = dps.ptr_array
MB = 1 << 20


def fake(k, base=1 << 40, stride=MB):
    """k distinct, 256-byte aligned, non-overlapping fake device addresses."""
    return [base + i * stride for i in range(k)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dp_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(dps.EXPORTS)
    L = dps.lib()
    for n in names:
        assert hasattr(L, n), n
    assert dps.dp_version() == 100


def test_shard_len_and_strings():
    assert dps.dp_shard_len(0, 8) == 0
    assert dps.dp_shard_len(10_000_019, 8) == 1_250_003
    assert dps.dp_shard_len(1_048_576, 4) == 262_144
    assert dps.dp_shard_len(5, 0) == 0
    for code in range(6):
        assert dps.dp_status_string(code).startswith("DP_")
    assert "unknown" in dps.dp_status_string(99)
    assert dps.dp_last_hip_error() == 0


def rs(send, recv, n, k, dt=F32, op=SUM, s=1):
    return dps.lib().dp_reduce_scatter(P(send), P(recv), n, k, dt, op, s, None)


def ag(send, recv, n, k, dt=F32, s=1):
    return dps.lib().dp_all_gather(P(send), P(recv), n, k, dt, s, None)


def ar(send, recv, n, k, dt=F32, op=SUM, s=1):
    return dps.lib().dp_all_reduce(P(send), P(recv), n, k, dt, op, s, None)


def wr(send, recv, toks, n, k, dt=F32, s=1):
    t = (ctypes.c_int64 * len(toks))(*toks)
    return dps.lib().dp_weighted_reduce(P(send), P(recv), t, n, k, dt, s, None)


def test_rank_count_and_chunks():
    a, b = fake(65), fake(65, base=1 << 41)
    assert rs(a[:2], b[:2], 100, 0) == INVALID
    assert rs(a, b, 100, 65) == INVALID
    assert rs(a[:2], b[:2], 100, 2, s=0) == INVALID
    assert ag(a[:2], b[:2], 100, 2, s=-1) == INVALID
    assert ar(a[:2], b[:2], 100, 2, s=0) == INVALID


def test_null_and_misaligned_pointers():
    L = dps.lib()
    a, b = fake(4), fake(4, base=1 << 41)
    assert L.dp_reduce_scatter(None, P(b), 100, 4, F32, SUM, 1, None) == INVALID
    assert L.dp_all_gather(P(a), None, 100, 4, F32, 1, None) == INVALID
    assert rs([a[0], 0, a[2], a[3]], b, 100, 4) == INVALID
    assert rs([a[0] + 2] + a[1:], b, 100, 4, dt=F32) == INVALID       # 2-byte aligned f32
    assert rs(a, [b[0] + 1] + b[1:], 100, 4, dt=BF16) == INVALID      # odd address bf16
    assert rs(a, b, 1 << 62, 4) == INVALID                            # size overflow


def test_unsupported_dtype_and_op():
    a, b = fake(4), fake(4, base=1 << 41)
    assert rs(a, b, 100, 4, dt=7) == UNSUPPORTED
    assert rs(a, b, 100, 4, op=9) == UNSUPPORTED
    assert rs(a, b, 100, 4, dt=I32, op=AVG) == UNSUPPORTED
    assert ar(a, b, 100, 4, dt=I32, op=AVG) == UNSUPPORTED
    assert wr(a, b, [1, 1, 1, 1], 100, 4, dt=I32) == UNSUPPORTED


def test_token_validation():
    a, b = fake(4), fake(4, base=1 << 41)
    assert wr(a, b, [0, 0, 0, 0], 100, 4) == INVALID
    assert wr(a, b, [5, -1, 0, 0], 100, 4) == INVALID
    assert dps.lib().dp_weighted_reduce(P(a), P(b), None, 100, 4, F32, 1, None) == INVALID
    assert wr(a, b, [1, 2, 3, 4], 0, 4) == OK                         # n == 0 is a no-op


def test_alias_rules():
    a = fake(4)
    # recv overlapping a send buffer
    assert rs(a, [a[1] + 64] + fake(3, base=1 << 41), 1000, 4) == ALIAS
    # recv buffers overlapping each other
    assert rs(a, [1 << 41, (1 << 41) + 16, 1 << 42, 1 << 43], 1000, 4) == ALIAS
    # AllGather outputs overlapping each other
    assert ag(fake(4, base=1 << 41), [a[0], a[0] + 400, a[2], a[3]], 1000, 4) == ALIAS
    # AllGather source shard inside an output, not at the in-place position
    assert ag([a[0] + 8, a[1], a[2], a[3]], fake(4, base=a[0]), 1000, 4) == ALIAS
    # AllReduce: recv[r] may be send[r], but not overlap another send
    assert ar(a, [a[1]] + fake(3, base=1 << 41), 1000, 4) == ALIAS
    # ReduceScatter in-place form requires n == k*L
    n = 1001
    L = dps.dp_shard_len(n, 4)
    assert rs(a, [a[c] + c * L * 4 for c in range(4)], n, 4) == ALIAS


def test_zero_length_is_noop():
    a, b = fake(3), fake(3, base=1 << 41)
    assert rs(a, b, 0, 3) == OK
    assert ag(a, b, 0, 3) == OK
    assert ar(a, b, 0, 3, op=AVG) == OK


def test_fsdp_validation():
    L = dps.lib()
    k = 2
    x, ws, dy = fake(k, 1 << 40), fake(k, 1 << 41), fake(k, 1 << 42)
    wf, y, dwf, dws = fake(k, 1 << 43), fake(k, 1 << 44), fake(k, 1 << 45), fake(k, 1 << 46)

    def call(k_=k, m=8, d=8, f=8, x_=x, wf_=wf, y_=y, dy_=dy):
        return L.dp_fsdp_layer(k_, m, d, f, P(x_), P(ws), P(dy_) if dy_ else None, P(wf_), P(y_),
                               P(dwf), P(dws), None)
    assert call(k_=0) == INVALID
    assert call(m=0) == INVALID
    assert call(d=-1) == INVALID
    assert call(x_=[x[0], 0]) == INVALID
    assert call(y_=[x[0], y[1]]) == ALIAS             # output on top of an input
    assert call(wf_=[wf[0], wf[0] + 4]) == ALIAS      # outputs overlap each other
    dx = fake(k, 1 << 47)

    def call_ex(dx_=dx, dy_=dy, x_=x):
        return L.dp_fsdp_layer_ex(k, 8, 8, 8, P(x_), P(ws), P(dy_) if dy_ else None, P(wf), P(y),
                                  P(dx_) if dx_ else None, P(dwf), P(dws), None)
    assert call_ex(dy_=None) == INVALID                # dx needs the backward pass
    assert call_ex(dx_=[dx[0], 0]) == INVALID
    assert call_ex(dx_=[dx[0], x[1] + 8]) == ALIAS     # dx on top of an input
    assert call_ex(dx_=[dx[0], dwf[0]]) == ALIAS       # dx on top of another output


def test_fsdp_static_validation():
    """The allocation-free FSDP step checks the caller's buffers like
    dp_fsdp_layer_ex and rejects workspaces beyond the static buffer, all
    before it touches the device."""
    L = dps.lib()
    k = 8
    x, ws, dy = fake(k, 1 << 40), fake(k, 1 << 41), fake(k, 1 << 42)
    y, dws, dx = fake(k, 1 << 44), fake(k, 1 << 46), fake(k, 1 << 47)

    def call(k_=k, m=64, d=64, f=64, x_=x, y_=y, dy_=dy, dx_=None):
        return L.dp_fsdp_layer_static(k_, m, d, f, P(x_[:k_]), P(ws[:k_]),
                                      P(dy_[:k_]) if dy_ else None, P(y_[:k_]),
                                      P(dx_[:k_]) if dx_ else None, P(dws[:k_]), None)
    assert call(k_=0) == INVALID
    assert call(m=0) == INVALID
    assert call(x_=[x[0], 0] + x[2:]) == INVALID
    assert call(y_=[x[0]] + y[1:]) == ALIAS
    assert call(dy_=None, dx_=dx) == INVALID            # dx needs the backward pass
    # 2 * K * d * f * 4 bytes against the 32 MiB buffer
    assert call(d=1024, f=1024) == dps.DP_ERR_SCRATCH
    # just over the limit with K = 2 (each region rounded up to 256 bytes)
    big = [fake(2, 1 << 40 + i, stride=64 * MB) for i in range(5)]
    assert L.dp_fsdp_layer_static(2, 64, 2048, 1025, P(big[0]), P(big[1]), P(big[2]), P(big[3]),
                                  None, P(big[4]), None) == dps.DP_ERR_SCRATCH
    assert dps.DP_STATIC_SCRATCH_BYTES == 32 << 20


def test_gemm_validation():
    L = dps.lib()
    a, b, c = 1 << 40, 1 << 41, 1 << 42
    assert L.dp_gemm_bf16(a, b, c, 0, 8, 8, None) == INVALID
    assert L.dp_gemm_bf16(None, b, c, 8, 8, 8, None) == INVALID
    assert L.dp_gemm_bf16(a + 1, b, c, 8, 8, 8, None) == INVALID      # not element-aligned
    assert L.dp_gemm_bf16(a, b, c + 3, 8, 8, 12, None) == INVALID
    assert L.dp_gemm_bf16(a, b, a + 16, 8, 8, 8, None) == ALIAS
    assert L.dp_gemm_bf16(a, b, c, 1 << 25, 8, 8, None) == INVALID


def test_bucket_plan():
    plan = bucket_plan(218_103_808, 25_000_000)
    assert len(plan) == 9
    assert plan[-1] == (200_000_000, 18_103_808)
    assert sum(n for _, n in plan) == 218_103_808
    assert all(o == i * 25_000_000 for i, (o, _) in enumerate(plan))
    assert bucket_plan(0, 10) == []
    with pytest.raises(ValueError):
        bucket_plan(10, 0)


def test_rank_buffers_layout():
    import torch
    for dt, n, st in ((torch.bfloat16, 1001, 131072), (torch.float32, 64, 0), (torch.int32, 3, 256)):
        bufs = rank_buffers(3, n, dt, device="cpu", stagger=st)
        es = bufs[0].element_size()
        stride = (-(-n * es // 256) * 256 + st)
        base = bufs[0].data_ptr()
        for r, b in enumerate(bufs):
            assert b.numel() == n and b.is_contiguous() and b.dtype == dt
            assert b.data_ptr() - base == r * stride
            assert (b.data_ptr() - base) % 256 == 0
        for b in bufs:
            b.zero_()
        bufs[1].fill_(1)                              # no overlap between ranks
        assert bufs[0].eq(0).all() and bufs[2].eq(0).all()
    assert [b.numel() for b in rank_buffers(2, 0, device="cpu")] == [0, 0]
    with pytest.raises(ValueError):
        rank_buffers(2, 10, stagger=100)


def test_binding_rejects_host_tensors():
    import torch
    t = [torch.zeros(10) for _ in range(2)]
    with pytest.raises(ValueError):
        dps.dp_all_reduce(t, t)


def test_launch_options_validation():
    L = dps.lib()
    a, b = fake(4), fake(4, base=1 << 41)
    bad = [dps.LaunchOpts(-1, 0, (ctypes.c_int * 2)(0, 0)),
           dps.LaunchOpts(0, 16, (ctypes.c_int * 2)(0, 0)),
           dps.LaunchOpts(0, 0, (ctypes.c_int * 2)(1, 0))]
    for o in bad:
        r = ctypes.byref(o)
        assert L.dp_reduce_scatter_ex(P(a), P(b), 100, 4, F32, SUM, 1, r, None) == INVALID
        assert L.dp_all_gather_ex(P(a), P(b), 100, 4, F32, 1, r, None) == INVALID
        assert L.dp_all_reduce_ex(P(a), P(b), 100, 4, F32, SUM, 1, r, None) == INVALID
        assert L.dp_gemm_bf16_ex(1 << 40, 1 << 41, 1 << 42, 8, 8, 8, r, None) == INVALID
    ok = ctypes.byref(dps.LaunchOpts.make(16, True))
    # valid options, still rejected for the usual reasons (nothing is launched)
    assert L.dp_reduce_scatter_ex(P(a), P(b), 100, 0, F32, SUM, 1, ok, None) == INVALID
    assert L.dp_all_reduce_ex(P(a), P(b), 0, 4, F32, SUM, 1, ok, None) == OK
    assert L.dp_gemm_bf16_ex(1 << 40, (1 << 41) + 1, 1 << 42, 8, 8, 12, ok, None) == INVALID
    nk = ctypes.byref(dps.LaunchOpts(0, dps.DP_LAUNCH_B_NK, (ctypes.c_int * 2)(0, 0)))
    assert L.dp_gemm_bf16_ex(1 << 40, 1 << 41, (1 << 41) + 2, 8, 8, 8, nk, None) == ALIAS
    assert L.dp_reduce_scatter_ex(P(a), P(b), 0, 4, F32, SUM, 1, None, None) == OK


def test_odc_validation():
    L = dps.lib()
    g, acc, out = 1 << 40, fake(4, base=1 << 41), fake(4, base=1 << 42)
    sa = L.dp_scatter_accumulate
    gs = [g, g + 4096]
    assert sa(P(gs), 2, F32, P(acc), 1000, 0, None) == INVALID           # k out of range
    assert sa(P(gs), 0, F32, P(acc), 1000, 4, None) == INVALID           # no push
    assert sa(P(gs), 65, F32, P(acc), 1000, 4, None) == INVALID
    assert sa(P(gs), 2, I32, P(acc), 1000, 4, None) == UNSUPPORTED
    assert sa(P([g, 0]), 2, F32, P(acc), 1000, 4, None) == INVALID
    assert sa(None, 1, F32, P(acc), 1000, 4, None) == INVALID
    assert sa(P([g + 1]), 1, BF16, P(acc), 1000, 4, None) == INVALID    # misaligned gradient
    assert sa(P(gs), 2, F32, P([acc[0] + 2] + acc[1:]), 1000, 4, None) == INVALID
    assert sa(P(gs), 2, F32, P([g + 6000] + acc[1:]), 1000, 4, None) == ALIAS   # inside grad 1
    assert sa(P(gs), 2, F32, P([acc[0], acc[0] + 16] + acc[2:]), 1000, 4, None) == ALIAS
    assert sa(P(gs), 2, BF16, P(acc), 0, 4, None) == OK                 # n == 0 is a no-op
    st = L.dp_settle
    assert st(P(acc), P(out), 1000, 4, F32, 0.0, 0, None) == INVALID  # zero divisor
    assert st(P(acc), P(out), 1000, 4, F32, float("inf"), 0, None) == INVALID
    assert st(P(acc), P(out), 1000, 4, F32, float("nan"), 0, None) == INVALID
    assert st(P(acc), P(out), 1000, 4, I32, 1.0, 0, None) == UNSUPPORTED
    assert st(P(acc), P([out[0] + 1] + out[1:]), 1000, 4, BF16, 1.0, 0, None) == INVALID
    assert st(P(acc), P([acc[1]] + out[1:]), 1000, 4, F32, 1.0, 0, None) == ALIAS
    # in place is allowed only for fp32 output without reset
    assert st(P(acc), P(acc), 0, 4, F32, 1.0, 0, None) == OK
    assert st(P(acc), P(acc), 1000, 4, F32, 1.0, 1, None) == ALIAS
    assert st(P(acc), P(acc), 1000, 4, BF16, 1.0, 0, None) == ALIAS
    assert st(P(acc), P([out[0], out[0] + 8] + out[2:]), 1000, 4, F32, 1.0, 0, None) == ALIAS
    assert st(P(acc), P(out), 0, 4, BF16, 3.0, 1, None) == OK


def test_overlap_validation():
    L = dps.lib()
    k, t = 2, 16
    pieces = [(0, 32, 32), (1024, 16, 8)]
    total = 1024 + 128
    arr = (dps.GradPiece * 2)(*[dps.GradPiece(*p) for p in pieces])
    dy, x = fake(4, base=1 << 40), fake(4, base=1 << 41)
    grad, out = fake(k, base=1 << 42), fake(k, base=1 << 43)
    ev = P(fake(2, base=1 << 44))
    o = ctypes.byref(dps.LaunchOpts.make())
    s1, s2 = 1 << 20, 2 << 20            # two distinct (fake) streams

    def call(k_=k, n_p=2, arr_=arr, t_=t, dy_=dy, x_=x, grad_=grad, out_=out, total_=total,
             bucket=500, op=AVG, opts=o, cs=s1, ms=s2, ev_=ev, nev=3):
        return L.dp_backward_allreduce_overlap(k_, n_p, arr_, t_, P(dy_), P(x_), P(grad_),
                                               P(out_), total_, bucket, op, opts, cs, ms, ev_, nev)
    assert call(k_=0) == INVALID
    assert call(n_p=0) == INVALID
    assert call(t_=12) == UNSUPPORTED                       # tokens not a multiple of 8
    assert call(op=7) == UNSUPPORTED
    assert call(total_=total + 1) == INVALID                # pieces do not tile the vector
    bad = (dps.GradPiece * 2)(dps.GradPiece(0, 32, 32), dps.GradPiece(1000, 16, 8))
    assert call(arr_=bad) == INVALID                        # gap / overlap between pieces
    assert call(dy_=[dy[0] + 8] + dy[1:]) == UNSUPPORTED     # operand not 16-byte aligned
    assert call(dy_=[0] + dy[1:]) == INVALID
    assert call(grad_=[grad[0], grad[0] + 64]) == ALIAS     # gradient vectors overlap
    assert call(out_=[grad[1], out[1]]) == ALIAS            # output on another rank's gradient
    assert call(x_=[grad[0]] + x[1:]) == ALIAS              # operand inside a gradient
    assert call(nev=2) == INVALID                           # 3 buckets need 3 events
    assert call(ev_=None, nev=0) == INVALID
    assert call(bucket=0) == INVALID
    bad_opts = dps.LaunchOpts(0, 16, (ctypes.c_int * 2)(0, 0))
    assert call(opts=ctypes.byref(bad_opts)) == INVALID


def test_fused_rs_ag_validation():
    L = dps.lib()
    k, n = 4, 1000
    Lk = dps.dp_shard_len(n, k)
    rs_s, rs_r = fake(k, base=1 << 40), fake(k, base=1 << 41)
    ag_s, ag_r = fake(k, base=1 << 42), fake(k, base=1 << 43)

    def call(a=rs_s, b=rs_r, na=n, c=ag_s, d=ag_r, nb=n, k_=k, dt=F32, op=SUM, s=1):
        return L.dp_reduce_scatter_all_gather(P(a), P(b), na, P(c), P(d), nb, k_, dt, op, s, None)
    assert call(k_=0) == INVALID
    assert call(s=0) == INVALID
    assert call(dt=7) == UNSUPPORTED
    assert call(dt=I32, op=AVG) == UNSUPPORTED
    assert call(b=[rs_s[1] + 64] + rs_r[1:]) == ALIAS          # RS output inside an RS input
    assert call(d=[ag_r[0], ag_r[0] + 400] + ag_r[2:]) == ALIAS  # AG outputs overlap
    assert call(c=[rs_s[0]] + ag_s[1:]) == ALIAS               # AG input inside an RS input
    assert call(d=[rs_r[2]] + ag_r[1:]) == ALIAS               # AG output on an RS shard
    assert call(na=0, nb=0) == OK
    assert Lk == 250
