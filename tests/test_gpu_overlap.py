"""GPU checks of the backward pass with bucketed AllReduce overlap
(dp_backward_allreduce_overlap), through the C ABI.

The gradients are bf16 GEMMs, checked against the oracle's fp64 products within
the recursive-summation bound (bit-exact for small-integer inputs); the
AllReduced outputs are checked bit-exactly against the oracle's AllReduce of
those same gradients, and the overlapped schedule against the one-stream
schedule.
"""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
import oracle
from tests.helpers import bits_equal, say, to_np
from tests.test_gpu_fsdp_gemm import U_BF16, gamma
from tests.test_gpu_sync import DEV

pytestmark = pytest.mark.gpu


def make_pieces(shapes):
    out, off = [], 0
    for m, n in shapes:
        out.append((off, m, n))
        off += m * n
    return out, off


def run(pieces, total, t, dy, x, k, bucket, op, overlap, in_place=False, **opts):
    grad = [torch.full((total,), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    out = grad if in_place else [torch.full((total,), float("nan"), dtype=torch.bfloat16,
                                            device=DEV) for _ in range(k)]
    cur = torch.cuda.current_stream()
    if overlap:
        comm = torch.cuda.Stream()
        ev = dps.HipEvents(-(-total // bucket))
        dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, bucket, op=op,
                                          compute_stream=cur, comm_stream=comm, events=ev, **opts)
        torch.cuda.synchronize()
        ev.close()
    else:
        dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, bucket, op=op, **opts)
        torch.cuda.synchronize()
    return grad, out


def check_pieces(pieces, t, dy, x, grad_host, k, ranks, samples=None, exact=False):
    """Gradient pieces of the given ranks against the oracle's fp64 products."""
    rng = np.random.default_rng(0)
    for g, (off, m, n) in enumerate(pieces):
        for r in ranks:
            if samples is None:
                rows, cols = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
                rows, cols = rows.ravel(), cols.ravel()
            else:
                rows = np.concatenate([rng.integers(0, m, samples), [0, m - 1, 0, m - 1]])
                cols = np.concatenate([rng.integers(0, n, samples), [0, n - 1, n - 1, 0]])
            # dW = dY X^T with X stored [n, t]: the [n, kk] layout of B
            ref, absr = oracle.gemm_bf16_at(to_np(dy[g * k + r]), to_np(x[g * k + r]),
                                            rows.astype(np.int64), cols.astype(np.int64),
                                            nthreads=16, b_layout="nk")
            got = oracle.bf16_to_f32(grad_host[r][off:off + m * n].reshape(m, n)[rows, cols])
            got = got.astype(np.float64)
            if exact:
                assert np.array_equal(got, ref), (g, r)
                continue
            gm = gamma(t + 1)
            bound = U_BF16 * (np.abs(ref) + gm * absr) + gm * absr
            assert np.all(np.abs(got - ref) <= bound), (g, r)


def oracle_bucketed_all_reduce(gh, bucket, op):
    """Each bucket AllReduced on its own (its own shards and ring order), as
    the call defines it."""
    total = gh[0].size
    outs = [np.empty(total, dtype=gh[0].dtype) for _ in gh]
    for b0 in range(0, total, bucket):
        part = oracle.all_reduce([np.ascontiguousarray(g[b0:b0 + bucket]) for g in gh], op=op,
                                 nthreads=16)
        for o, p in zip(outs, part):
            o[b0:b0 + p.size] = p
    return outs


def int_operands(k, pieces, t, seed):
    g = torch.Generator().manual_seed(seed)
    dy, x = [], []
    for _, m, n in pieces:
        for _ in range(k):
            dy.append(torch.randint(-2, 3, (m, t), generator=g).to(torch.bfloat16).to(DEV))
            x.append(torch.randint(-2, 3, (n, t), generator=g).to(torch.bfloat16).to(DEV))
    return dy, x


@pytest.mark.parametrize("k", [1, 2, 3, 8])
@pytest.mark.parametrize("integer", [False, True])
def test_small_pieces_all_schedules(k, integer):
    pieces, total = make_pieces([(100, 72), (64, 40), (300, 8), (257, 129)])
    t = 40
    if integer:
        dy, x = int_operands(k, pieces, t, seed=k)
    else:
        dy, x = gen.backward_operands(11 + k, k, pieces, t, device=DEV, dy_std=1.0)
    for bucket in (1000, 7000, total, 10 ** 6):
        for op in ("sum", "avg"):
            say(f"overlap small k={k} int={integer} bucket={bucket} op={op}")
            g1, o1 = run(pieces, total, t, dy, x, k, bucket, op, overlap=False)
            g2, o2 = run(pieces, total, t, dy, x, k, bucket, op, overlap=True)
            gh = [to_np(a) for a in g1]
            for r in range(k):
                assert bits_equal(to_np(g2[r]), gh[r])
                assert bits_equal(to_np(o1[r]), to_np(o2[r]))
            want = oracle_bucketed_all_reduce(gh, bucket, op)
            for r in range(k):
                assert bits_equal(to_np(o1[r]), want[r]), (r, bucket, op)
    check_pieces(pieces, t, dy, x, gh, k, range(k), exact=integer)


def test_in_place_and_launch_options():
    k, t = 4, 64
    pieces, total = make_pieces([(512, 256), (128, 1000), (256, 256)])
    dy, x = gen.backward_operands(5, k, pieces, t, device=DEV, dy_std=1.0)
    for opts in ({}, {"max_workgroups": 256}, {"share_cu": True}, {"two_phase": True},
                 {"share_cu": True, "max_workgroups": 64}):
        for in_place in (False, True):
            say(f"overlap opts={opts} in_place={in_place}")
            grad, out = run(pieces, total, t, dy, x, k, 100_000, "avg", overlap=True,
                            in_place=in_place, **opts)
            if in_place:
                # the gradients were overwritten; recompute them on one stream
                g_ref, _ = run(pieces, total, t, dy, x, k, 100_000, "avg", overlap=False,
                               share_cu=opts.get("share_cu", False))
                gh = [to_np(a) for a in g_ref]
            else:
                gh = [to_np(a) for a in grad]
                check_pieces(pieces, t, dy, x, gh, k, [0, k - 1], samples=500)
            want = oracle_bucketed_all_reduce(gh, 100_000, "avg")
            for r in range(k):
                assert bits_equal(to_np(out[r]), want[r]), (opts, in_place, r)


def test_errors():
    k, t = 2, 16
    pieces, total = make_pieces([(32, 32)])
    dy, x = gen.backward_operands(1, k, pieces, t, device=DEV)
    grad = [torch.zeros(total, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    with pytest.raises(dps.DpsyncError):      # pieces do not tile the vector
        dps.dp_backward_allreduce_overlap([(8, 32, 32)], t, dy, x, grad, grad, 100)
    with pytest.raises(dps.DpsyncError):      # two streams without events
        dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, grad, 100,
                                          comm_stream=torch.cuda.Stream())
    ev = dps.HipEvents(2)
    with pytest.raises(dps.DpsyncError):      # too few events for 11 buckets
        dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, grad, 100,
                                          comm_stream=torch.cuda.Stream(), events=ev)
    ev.close()


def test_layer_k8_full_size():
    """The bench workload: K=8, one layer's 7 weight gradients (218,103,808 per
    rank) from t=128 tokens per rank, 25,000,000-element buckets, averaged,
    overlapped with CU sharing; AllReduce checked over every element, the
    gradients at sampled entries of ranks 0 and 7."""
    k, t = 8, 128
    pieces = gen.layer_backward_pieces()
    total = gen.LAYER_PARAMS
    say(f"overlap layer k={k} t={t}")
    dy, x = gen.backward_operands(6, k, pieces, t, device=DEV)
    grad, out = run(pieces, total, t, dy, x, k, gen.BUCKET_ELEMS, "avg", overlap=True,
                    share_cu=True, max_workgroups=256)
    gh = [to_np(a) for a in grad]
    check_pieces(pieces, t, dy, x, gh, k, [0, k - 1], samples=400)
    want = oracle_bucketed_all_reduce(gh, gen.BUCKET_ELEMS, "avg")
    for r in range(k):
        assert bits_equal(to_np(out[r]), want[r]), r
