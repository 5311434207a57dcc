"""GPU parity on IEEE special values, through every sync kernel.

The ReduceScatter fold is a plain fp32 sum in ring order (CMU 11-868 L14-L15
notes, "Ring AllReduce: ReduceScatter, then AllGather"), so its corner cases
are those of IEEE binary32 addition: the first operand of the fold is taken
as it is (a fold of -0.0 values stays -0.0), infinities propagate, Inf - Inf
and 0 * Inf give NaN, subnormals are kept, and bf16 results are rounded once
to nearest even, overflowing to Inf where the fp32 value lies at or beyond
the halfway point above the largest bf16. These tests plant such values at
every position kind of the kernels (vector bodies, scalar heads of misaligned
shards, tails) and compare with the oracle.

Comparison rule: where the oracle's result is a NaN, the GPU's must be a NaN
of the same width (any sign and payload: IEEE 754 does not fix which payload
an operation on two NaN operands returns, nor the sign of the NaN that 0*Inf
or Inf-Inf creates, and x86 and the GPU differ there); every other element
must be equal bit for bit, the sign of zero included. The AllGather moves bits
without arithmetic, so there NaNs, signalling ones included, must match bit
for bit too.
"""
import numpy as np
import pytest
import torch

import gradient_sync_amd as dps
import oracle
from tests.helpers import say, to_np
from tests.special_values import special_equal, special_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _to_dev(bits_list, dtype, off):
    """Device tensors holding the given bit patterns, each at element offset off
    inside its own allocation (off > 0 makes the shards start misaligned)."""
    out = []
    for b in bits_list:
        full = torch.zeros(b.size + off, dtype=dtype, device=DEV)
        if dtype == torch.bfloat16:
            full.view(torch.int16)[off:].copy_(torch.from_numpy(b.view(np.int16)))
        else:
            full.view(torch.int32)[off:].copy_(torch.from_numpy(b.view(np.int32)))
        out.append(full[off:])
    return out


def _host(bits, dtype):
    """The oracle's view: bf16 as uint16 bits, fp32 as float32."""
    return bits if dtype == torch.bfloat16 else bits.view(np.float32)


DTYPES = [torch.float32, torch.bfloat16]
# K = 8 averages by multiplying with the exact 1/8, K = 6 by dividing
SHAPES = [(8, 8 * 2048 * 3 + 37), (6, 6 * 1024 + 5), (8, 13)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,n", SHAPES)
def test_special_reduce_scatter(dtype, k, n):
    L = dps.dp_shard_len(n, k)
    for off in (0, 1):
        bits = special_inputs(dtype, k, n, seed=100 + k + off)
        xs = _to_dev(bits, dtype, off)
        hx = [_host(b, dtype) for b in bits]
        for op in ("sum", "avg"):
            want = oracle.reduce_scatter(hx, op=op)
            for s in (1, 3):
                say(f"special rs {dtype} k={k} n={n} off={off} {op} S={s}")
                outs = [torch.empty(L, dtype=dtype, device=DEV) for _ in range(k)]
                dps.dp_reduce_scatter(xs, outs, op=op, s_chunks=s)
                torch.cuda.synchronize()
                for c in range(k):
                    assert special_equal(to_np(outs[c]), want[c]), (off, op, s, c)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,n", SHAPES)
def test_special_all_gather_moves_bits(dtype, k, n):
    L = dps.dp_shard_len(n, k)
    for sh_off in (0, 1):
        bits = special_inputs(dtype, k, k * L, seed=200 + k + sh_off)
        shards = _to_dev([b[:L].copy() for b in bits], dtype, sh_off)
        say(f"special ag {dtype} k={k} n={n} sh_off={sh_off}")
        outs = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
        dps.dp_all_gather(shards, outs, n=n)
        torch.cuda.synchronize()
        want = oracle.all_gather([_host(b[:L].copy(), dtype) for b in bits], n)
        for r in range(k):
            assert to_np(outs[r]).tobytes() == want[r].tobytes(), (sh_off, r)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,n", SHAPES)
def test_special_all_reduce_one_pass_and_two_phase(dtype, k, n):
    for off in (0, 1):
        bits = special_inputs(dtype, k, n, seed=300 + k + off)
        xs = _to_dev(bits, dtype, off)
        hx = [_host(b, dtype) for b in bits]
        for op in ("sum", "avg"):
            want = oracle.all_reduce(hx, op=op)
            for two_phase in (False, True):
                say(f"special ar {dtype} k={k} n={n} off={off} {op} two_phase={two_phase}")
                outs = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
                dps.dp_all_reduce_ex(xs, outs, op=op, two_phase=two_phase, s_chunks=2)
                torch.cuda.synchronize()
                for r in range(k):
                    assert special_equal(to_np(outs[r]), want[r]), (off, op, two_phase, r)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k,n", SHAPES)
def test_special_weighted_with_zero_tokens(dtype, k, n):
    """Token counts with zeros: a zero weight times an infinity or a NaN is a
    NaN that enters the fold; a zero weight times -0.0 or a finite value is a
    signed zero."""
    tokens = {8: [0, 1500, 0, 800, 3, 0, 77, 1024], 6: [0, 5, 1000, 0, 3, 2]}[k]
    for off in (0, 1):
        bits = special_inputs(dtype, k, n, seed=400 + k + off)
        xs = _to_dev(bits, dtype, off)
        hx = [_host(b, dtype) for b in bits]
        want = oracle.weighted_all_reduce(hx, tokens)
        for two_phase in (False, True):
            say(f"special weighted {dtype} k={k} n={n} off={off} two_phase={two_phase}")
            outs = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
            dps.dp_weighted_reduce_ex(xs, outs, tokens, two_phase=two_phase)
            torch.cuda.synchronize()
            for r in range(k):
                assert special_equal(to_np(outs[r]), want[r]), (off, two_phase, r)


@pytest.mark.parametrize("dtype", DTYPES)
def test_special_fused_reduce_scatter_all_gather(dtype):
    k, n_rs, n_ag = 8, 8 * 2048 * 2 + 9, 8 * 2048 + 3
    rb = special_inputs(dtype, k, n_rs, seed=500)
    La = dps.dp_shard_len(n_ag, k)
    ab = special_inputs(dtype, k, k * La, seed=501)
    rs_send = _to_dev(rb, dtype, 0)
    rs_recv = [torch.empty(dps.dp_shard_len(n_rs, k), dtype=dtype, device=DEV) for _ in range(k)]
    ag_send = _to_dev([b[:La].copy() for b in ab], dtype, 1)
    ag_recv = [torch.empty(n_ag, dtype=dtype, device=DEV) for _ in range(k)]
    say(f"special rsag {dtype}")
    dps.dp_reduce_scatter_all_gather(rs_send, rs_recv, ag_send, ag_recv, op="avg", ag_n=n_ag)
    torch.cuda.synchronize()
    want_rs = oracle.reduce_scatter([_host(b, dtype) for b in rb], op="avg")
    want_ag = oracle.all_gather([_host(b[:La].copy(), dtype) for b in ab], n_ag)
    for c in range(k):
        assert special_equal(to_np(rs_recv[c]), want_rs[c]), c
        assert to_np(ag_recv[c]).tobytes() == want_ag[c].tobytes(), c


@pytest.mark.parametrize("gdtype", DTYPES)
@pytest.mark.parametrize("odtype", DTYPES)
def test_special_scatter_accumulate_and_settle(gdtype, odtype):
    """ODC pushes of gradients full of special values into fp32 accumulators,
    then settles by a power-of-two divisor (multiplied by its reciprocal) and
    by 3 (divided)."""
    k, n, np_ = 8, 8 * 1024 * 3 + 11, 3
    L = dps.dp_shard_len(n, k)
    g_bits = special_inputs(gdtype, np_, n, seed=600)
    grads = _to_dev(g_bits, gdtype, 1)
    for divisor in (8.0, 3.0):
        say(f"special odc {gdtype}->{odtype} divisor={divisor}")
        acc = [torch.zeros(L, dtype=torch.float32, device=DEV) for _ in range(k)]
        out = [torch.empty(L, dtype=odtype, device=DEV) for _ in range(k)]
        dps.dp_scatter_accumulate(grads, acc)
        dps.dp_settle(acc, out, n, divisor=divisor)
        torch.cuda.synchronize()
        h_acc = [np.zeros(L, np.float32) for _ in range(k)]
        for b in g_bits:
            oracle.scatter_accumulate(_host(b, gdtype), h_acc, k)
        for c in range(k):
            assert special_equal(to_np(acc[c]), h_acc[c]), c
        want = oracle.settle(h_acc, n, k, dtype=np.uint16 if odtype == torch.bfloat16 else np.float32,
                             divisor=divisor)
        for c in range(k):
            assert special_equal(to_np(out[c]), want[c]), (divisor, c)
