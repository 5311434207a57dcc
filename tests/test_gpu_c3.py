"""The concurrency workload run concurrently, checked: K=8 ranks of 268,435,456
fp32 (1 GiB each) ReduceScatter (sum) + AllGather on one stream, beside a bf16
8192^3 GEMM on another ("Optimizing ML Concurrent Computation and
Communication with GPU DMA Engines", section "Problem Formulation": the two
kernels share the GPU and have no data dependence, so running them together
must leave both results unchanged).

Schedules: the base one (default grids, GEMM enqueued first), schedule
prioritisation (collective first, at most 128 resident workgroups) and
resource partitioning (collective on 176 CUs, GEMM on the other 80, through
CU-masked streams).

Checks after each concurrent run:
  - collective: every shard element bit-exact against the oracle's full
    ReduceScatter of the same inputs (fp64 per-shard checksums of both are
    compared as well, as a summary), every AllGather output equal to output 0
    on the device, and output 0 bit-exact against the oracle's AllGather;
  - GEMM (C = A B, both operands [8192, 8192] row-major): bit-identical to
    the same GEMM run alone, which is itself checked at sampled entries within
    the fp32 summation bound of the fp64 product.
"""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
import oracle
from gradient_sync_amd.buckets import rank_buffers
from gradient_sync_amd.concurrency import SCHEDULES, C3Pair
from tests.helpers import say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
K, N, MNK = 8, 268_435_456, 8192
U24, U_BF16 = 2.0 ** -24, 2.0 ** -8


def _gamma(m):
    return m * U24 / (1 - m * U24)


@pytest.fixture(scope="module")
def workload():
    say("c3: generating 8 x 1 GiB fp32 and 2 x 8192^2 bf16")
    xs = rank_buffers(K, N, torch.float32)
    for r in range(K):          # the cfg-5 inputs, one rank at a time (tensor id 0)
        xs[r].copy_(gen.uniform_pm1(5, 0, r, N, device=DEV))
    L = dps.dp_shard_len(N, K)
    sh = rank_buffers(K, L, torch.float32)
    out = rank_buffers(K, N, torch.float32)
    a, b = gen.gemm_bf16_inputs(5, MNK, MNK, MNK, device=DEV)
    c = torch.empty(MNK, MNK, dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    say("c3: oracle ReduceScatter of the host copies")
    hx = [x.cpu().numpy() for x in xs]
    want_sh = oracle.reduce_scatter(hx, op="sum", nthreads=16)
    del hx
    say("c3: GEMM alone")
    c_alone = torch.empty_like(c)
    dps.dp_gemm_bf16(a, b, c_alone)
    torch.cuda.synchronize()
    yield dict(xs=xs, sh=sh, out=out, a=a, b=b, c=c, c_alone=c_alone, want_sh=want_sh, L=L)


def test_c3_gemm_alone_sampled(workload):
    """The reference GEMM result (run alone) at sampled entries, corners and
    tile edges included, within |c - r64| <= u_bf16 (|r64| + g) + g with
    g = gamma_{k+1} sum_p |a_ip| |b_pj| (bf16 products are exact in fp32)."""
    w = workload
    rng = np.random.default_rng(3)
    rows = np.concatenate([rng.integers(0, MNK, 2000), [0, 0, MNK - 1, MNK - 1, 255, 256]])
    cols = np.concatenate([rng.integers(0, MNK, 2000), [0, MNK - 1, 0, MNK - 1, 256, 255]])
    rows, cols = rows.astype(np.int64), cols.astype(np.int64)
    ref, absr = oracle.gemm_bf16_at(to_np(w["a"]), to_np(w["b"]), rows, cols, nthreads=16)
    got = oracle.bf16_to_f32(to_np(w["c_alone"])[rows, cols]).astype(np.float64)
    g = _gamma(MNK + 1) * absr
    assert np.all(np.abs(got - ref) <= U_BF16 * (np.abs(ref) + g) + g)


@pytest.mark.parametrize("name", ["base", "sp_cap128", "rp_comm176"])
def test_c3_concurrent_results(workload, name):
    w = workload
    sched = SCHEDULES[name]
    pair = C3Pair(w["xs"], w["sh"], w["out"], w["a"], w["b"], w["c"])
    # poison every output so that a skipped write cannot pass
    for t in list(w["sh"]) + list(w["out"]) + [w["c"]]:
        t.view(torch.int16).fill_(-1)                    # NaN bit patterns
    torch.cuda.synchronize()
    sc, sg, closers = pair.streams(sched)
    try:
        say(f"c3 concurrent {name}")
        start, done_c, done_g = pair.launch(sched, sc, sg)
        torch.cuda.synchronize()
        t_c, t_g = start.elapsed_time(done_c), start.elapsed_time(done_g)
        say(f"c3 {name}: collective done at {t_c:.3f} ms, GEMM at {t_g:.3f} ms")
    finally:
        for s in closers:
            s.close()
    # the GEMM beside the collective gives the same bits as alone
    assert torch.equal(w["c"].view(torch.int16), w["c_alone"].view(torch.int16))
    # every shard element against the oracle, plus fp64 checksums
    L = w["L"]
    for c in range(K):
        got = to_np(w["sh"][c])
        assert got.tobytes() == w["want_sh"][c].tobytes(), (name, c)
        assert np.sum(got, dtype=np.float64) == np.sum(w["want_sh"][c], dtype=np.float64)
    # all outputs equal, and output 0 is the gathered shards
    for r in range(1, K):
        assert torch.equal(w["out"][r].view(torch.int32), w["out"][0].view(torch.int32)), (name, r)
    o0 = to_np(w["out"][0])
    for c in range(K):
        assert o0[c * L:(c + 1) * L].tobytes() == w["want_sh"][c].tobytes(), (name, c)
