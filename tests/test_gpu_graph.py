"""The entry points under stream capture: every call only enqueues kernels on
the caller's stream (no allocation, memset, copy or host synchronisation), so a
caller can record a whole step into a HIP graph and replay it.

Each graph is replayed several times on fresh inputs, with eager work and
synchronisations between the replays, and every replay is compared bit for
bit with the same calls run eagerly on the same inputs (whose parity with the
oracle the other GPU tests establish).
"""
import pytest
import torch

import gen
import gradient_sync_amd as dps
from gradient_sync_amd.buckets import BucketedSync
from tests.helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 4


def _capture(fn):
    """fn recorded into a graph on a side stream (torch's capture protocol)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_matches_eager(fn, inputs, outputs, fresh_inputs):
    """Capture fn once; for each replay, load a fresh input set, poison the
    outputs, replay, and compare with fn run eagerly on the same inputs."""
    g = _capture(fn)
    for i in range(REPLAYS):
        new = fresh_inputs(i)
        for dst, src in zip(inputs, new):
            dst.copy_(src)
        for o in outputs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outputs]
        # eager work between replays: the same step, on the same inputs
        for o in outputs:
            o.fill_(float("nan"))
        fn()
        torch.cuda.synchronize()
        for r, (a, b) in enumerate(zip(got, outputs)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), (i, r)
    return g


def test_graph_pipelined_bucket_step():
    k, total, cap = 8, 2_500_003, 1_000_003          # 3 buckets, ragged tails
    say("graph: pipelined bucket step")
    sets = [gen.ring_uniform_inputs(40 + i, k, total, device=DEV) for i in range(REPLAYS)]
    grads = [torch.empty(total, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    out = [torch.empty(total, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    sync = BucketedSync(grads, out, cap, op="avg")
    _replay_matches_eager(sync.step_pipelined, grads, out,
                          lambda i: [x.to(torch.bfloat16) for x in sets[i]])


def test_graph_one_pass_step_and_weighted():
    k, total, cap = 8, 2_500_003, 1_000_003
    say("graph: one-pass AllReduce step")
    sets = [gen.ring_uniform_inputs(50 + i, k, total, device=DEV) for i in range(REPLAYS)]
    grads = [torch.empty(total, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    out = [torch.empty(total, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    sync = BucketedSync(grads, out, cap, op="sum")
    _replay_matches_eager(sync.step_all_reduce, grads, out,
                          lambda i: [x.to(torch.bfloat16) for x in sets[i]])

    say("graph: token-weighted AllReduce")
    n = 1_000_019
    xs = [torch.empty(n, device=DEV) for _ in range(k)]
    ys = [torch.empty(n, device=DEV) for _ in range(k)]
    toks = gen.token_counts(4, k)
    fsets = [gen.ring_uniform_inputs(60 + i, k, n, device=DEV) for i in range(REPLAYS)]
    _replay_matches_eager(lambda: dps.dp_weighted_reduce(xs, ys, toks), xs, ys, lambda i: fsets[i])


@pytest.mark.parametrize("with_dx", [False, True])
def test_graph_fsdp_step(with_dx):
    k, ml, d, f = 8, 128, 512, 512
    R = d // k
    say(f"graph: FSDP step with_dx={with_dx}")
    x = [torch.empty(ml, d, device=DEV) for _ in range(k)]
    ws = [torch.empty(R, f, device=DEV) for _ in range(k)]
    dy = [torch.empty(ml, f, device=DEV) for _ in range(k)]
    wf = [torch.empty(d, f, device=DEV) for _ in range(k)]
    y = [torch.empty(ml, f, device=DEV) for _ in range(k)]
    dwf = [torch.empty(d, f, device=DEV) for _ in range(k)]
    dws = [torch.empty(R, f, device=DEV) for _ in range(k)]
    dx = [torch.empty(ml, d, device=DEV) for _ in range(k)]
    kw = {"dx_local": dx} if with_dx else {}

    def fresh(i):
        fx = gen.fsdp_fixture(seed=70 + i, k=k, device=DEV)
        return ([fx["x"][r * ml:(r + 1) * ml] for r in range(k)] +
                [fx["w"][c * R:(c + 1) * R] for c in range(k)] +
                [fx["dy"][r * ml:(r + 1) * ml] for r in range(k)])

    outs = wf + y + dwf + dws + (dx if with_dx else [])
    _replay_matches_eager(lambda: dps.dp_fsdp_layer(x, ws, dy, wf, y, dwf, dws, **kw),
                          x + ws + dy, outs, fresh)
