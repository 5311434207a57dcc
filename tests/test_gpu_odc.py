"""GPU parity of the ODC scatter-accumulate and settle calls against the oracle,
through the C ABI.

Every comparison is bit-exact: a push is one fp32 addition per element in push
order on both sides, and the settle is one fp32 division (or the exact
power-of-two reciprocal) and one round to nearest even.
"""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
import oracle
from tests.helpers import bits_equal, say, to_np
from tests.test_gpu_sync import DEV, Guarded

pytestmark = pytest.mark.gpu


def push_order(counts):
    """Arrival order of the emulated minibatch: round m holds the m-th
    microbatch of every rank that has one, in rank order."""
    return [[(r, m) for r in range(len(counts)) if counts[r] > m] for m in range(max(counts))]


def microbatches(counts, n, dtype, seed, g_off=0):
    """Device gradients (inside canary-guarded buffers at element offset g_off)
    and their host copies, indexed [r][m]."""
    dev, host = [], []
    for r, cnt in enumerate(counts):
        dr, hr = [], []
        for m in range(cnt):
            v = gen.uniform_pm1(seed, 40 + m, r, n).to(dtype)
            g = Guarded(n, dtype, g_off)
            g.t.copy_(v.to(DEV))
            dr.append(g)
            hr.append(to_np(g.t))
        dev.append(dr)
        host.append(hr)
    return dev, host


def init_acc(k, L, seed, acc_off=0):
    """Accumulators with nonzero starting values (pads included), on both sides."""
    dev, host = [], []
    for c in range(k):
        v = gen.uniform_pm1(seed, 60, c, L)
        g = Guarded(L, torch.float32, acc_off)
        g.t.copy_(v.to(DEV))
        dev.append(g)
        host.append(v.numpy().copy())
    return dev, host


def apply_pushes(mode, rounds, dev_g, acc):
    """Issue the pushes on the GPU: one call per push, one call per round, or
    (up to 64 pushes) one call for the whole minibatch."""
    flat = [dev_g[r][m].t for rnd in rounds for r, m in rnd]
    if mode == "per_push":
        for t in flat:
            dps.dp_scatter_accumulate(t, acc)
    elif mode == "per_round":
        for rnd in rounds:
            dps.dp_scatter_accumulate([dev_g[r][m].t for r, m in rnd], acc)
    else:
        for i in range(0, len(flat), dps.DP_MAX_K):
            dps.dp_scatter_accumulate(flat[i:i + dps.DP_MAX_K], acc)


def check_acc(acc_dev, acc_host, what):
    for c, (d, h) in enumerate(zip(acc_dev, acc_host)):
        assert bits_equal(to_np(d.t), h), (what, c)
        assert d.intact(), (what, c)


def run_case(dtype, counts, n, seed, mode="per_round", g_off=0, acc_off=0):
    k = len(counts)
    L = dps.dp_shard_len(n, k)
    say(f"odc push k={k} n={n} {dtype} counts={counts} mode={mode} g_off={g_off} acc_off={acc_off}")
    dev_g, host_g = microbatches(counts, n, dtype, seed, g_off)
    acc_d, acc_h = init_acc(k, L, seed, acc_off)
    rounds = push_order(counts)
    apply_pushes(mode, rounds, dev_g, [a.t for a in acc_d])
    torch.cuda.synchronize()
    for rnd in rounds:
        for r, m in rnd:
            oracle.scatter_accumulate(host_g[r][m], acc_h, k, L=L)
    check_acc(acc_d, acc_h, (k, n, mode))
    for dev_r in dev_g:
        for g in dev_r:
            assert g.intact()
    return acc_d, acc_h


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_push_bruteforce_small(dtype):
    for k in [1, 2, 3, 5, 8, 16, 64]:
        for n in sorted({1, max(1, k - 1), k + 1, 97, 4099}):
            counts = [(r * 5 + k) % 3 for r in range(k)]
            if max(counts) == 0:
                counts[0] = 1
            run_case(dtype, counts, n, seed=300 + k * 11 + n)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", ["per_push", "per_round", "one_call"])
def test_push_modes_multi_tile_ragged(dtype, mode):
    # several 4096-element tiles per shard and a ragged last shard
    counts = [3, 2, 2, 6, 1, 4, 2, 3]
    run_case(dtype, counts, 3 * 4096 * 8 + 4093, seed=7, mode=mode)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_push_every_alignment(dtype):
    # gradient and accumulator offsets move the shards off the 16-byte path
    for g_off in range(8):
        for acc_off in (0, 1, 2, 3):
            run_case(dtype, [2, 1, 3], 3 * 5000 + 2, seed=11 + g_off, g_off=g_off,
                     acc_off=acc_off)


@pytest.mark.parametrize("npush", [1, 3, 4, 5, 9, 64])
def test_push_counts_per_call(npush):
    # np around and beyond the number of gradients loaded together
    k = 4
    counts = [npush // k + (1 if r < npush % k else 0) for r in range(k)]
    run_case(torch.bfloat16, counts, 40_000, seed=90 + npush, mode="one_call")


def settle_and_check(acc_d, acc_h, n, k, out_dtype, divisor, reset):
    L = dps.dp_shard_len(n, k)
    say(f"odc settle k={k} n={n} {out_dtype} divisor={divisor} reset={reset}")
    outs = [Guarded(L, out_dtype, off=c % 3) for c in range(k)]
    for o in outs:
        o.t.view(torch.uint8).fill_(0x77)           # pads must be overwritten with zero
    pads_before = [to_np(a.t)[max(0, min(L, n - c * L)):].copy() for c, a in enumerate(acc_d)]
    dps.dp_settle([a.t for a in acc_d], [o.t for o in outs], n, divisor=divisor, reset=reset)
    torch.cuda.synchronize()
    np_dt = np.float32 if out_dtype == torch.float32 else np.uint16
    want = oracle.settle(acc_h, n, k, dtype=np_dt, divisor=divisor, L=L)
    for c in range(k):
        assert bits_equal(to_np(outs[c].t), want[c]), (n, k, divisor, c)
        assert outs[c].intact()
        nc = max(0, min(L, n - c * L))
        a = to_np(acc_d[c].t)
        if reset:
            assert np.all(a[:nc] == 0.0) and not np.any(np.signbit(a[:nc]))
            acc_h[c][:nc] = 0.0
        else:
            assert bits_equal(a, acc_h[c])
        assert bits_equal(a[nc:], pads_before[c])     # pads are never touched
        assert acc_d[c].intact()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_settle_divisors_and_pads(out_dtype):
    for k, n in [(1, 1), (3, 7), (5, 4099), (8, 3 * 4096 * 8 + 4093), (64, 1000)]:
        counts = [1 + (r % 3) for r in range(k)]
        acc_d, acc_h = run_case(torch.bfloat16, counts, n, seed=500 + n)
        for divisor in (1.0, 8.0, 0.25, float(sum(counts)), 3.0, -2.0):
            settle_and_check(acc_d, acc_h, n, k, out_dtype, divisor, reset=False)
        settle_and_check(acc_d, acc_h, n, k, out_dtype, 2.0, reset=True)


def test_settle_in_place_fp32():
    k, n = 4, 10_001
    acc_d, acc_h = run_case(torch.float32, [1, 2, 0, 3], n, seed=41)
    L = dps.dp_shard_len(n, k)
    want = oracle.settle(acc_h, n, k, dtype=np.float32, divisor=6.0, L=L)
    dps.dp_settle([a.t for a in acc_d], [a.t for a in acc_d], n, divisor=6.0)
    torch.cuda.synchronize()
    for c in range(k):
        assert bits_equal(to_np(acc_d[c].t), want[c])


def test_two_minibatches_with_reset():
    # settle with reset, then a second minibatch accumulates from zero
    k, n = 8, 100_003
    counts = [3, 2, 2, 6, 1, 4, 2, 3]
    acc_d, acc_h = run_case(torch.bfloat16, counts, n, seed=3)
    settle_and_check(acc_d, acc_h, n, k, torch.bfloat16, float(sum(counts)), reset=True)
    dev_g, host_g = microbatches(counts[::-1], n, torch.bfloat16, seed=4)
    apply_pushes("per_round", push_order(counts[::-1]), dev_g, [a.t for a in acc_d])
    torch.cuda.synchronize()
    for rnd in push_order(counts[::-1]):
        for r, m in rnd:
            oracle.scatter_accumulate(host_g[r][m], acc_h, k)
    check_acc(acc_d, acc_h, "second minibatch")


def test_zero_length_and_errors():
    acc = [torch.zeros(4, device=DEV) for _ in range(2)]
    g = torch.zeros(0, dtype=torch.bfloat16, device=DEV)
    dps.dp_scatter_accumulate(g, acc)
    dps.dp_settle(acc, [torch.zeros(4, device=DEV) for _ in range(2)], 0)
    with pytest.raises(dps.DpsyncError):
        dps.dp_scatter_accumulate(torch.zeros(8, device=DEV), [acc[0], acc[0]])
    with pytest.raises(dps.DpsyncError):
        dps.dp_settle(acc, [torch.zeros(4, device=DEV) for _ in range(2)], 8, divisor=0.0)


def test_minibatch_k8_bf16_25m_full_size():
    """The bench workload: K=8 ranks, 25M-element bf16 gradients, uneven
    microbatch counts from the variable-length token generator, pushes drained
    per round, one bf16 settle; compared over every element."""
    k, n = 8, gen.BUCKET_ELEMS
    counts = gen.microbatch_counts(1, k)
    L = dps.dp_shard_len(n, k)
    say(f"odc full size k={k} n={n} counts={counts}")
    dev = [[gen.microbatch_grad(1, r, m, n, device=DEV) for m in range(counts[r])]
           for r in range(k)]
    acc = [torch.zeros(L, dtype=torch.float32, device=DEV) for _ in range(k)]
    for rnd in push_order(counts):
        dps.dp_scatter_accumulate([dev[r][m] for r, m in rnd], acc)
    out = [torch.empty(L, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    dps.dp_settle(acc, out, n, divisor=float(sum(counts)), reset=True)
    torch.cuda.synchronize()
    acc_h = [np.zeros(L, np.float32) for _ in range(k)]
    for rnd in push_order(counts):
        for r, m in rnd:
            oracle.scatter_accumulate(to_np(dev[r][m]), acc_h, k)
    want = oracle.settle(acc_h, n, k, dtype=np.uint16, divisor=float(sum(counts)))
    for c in range(k):
        assert bits_equal(to_np(out[c]), want[c]), c
        assert not torch.any(acc[c] != 0)


def test_beyond_2g_elements_sampled():
    """K=2 owners, two bf16 pushes of 2^31 + 7 elements (4 GiB each) and a
    bf16 settle: accumulators and settled shards checked at every shard
    boundary, around the 2^31-element mark, at the ends and at random
    positions against the oracle's push and settle of the same values."""
    from tests.test_gpu_sync import _uniform_chunked
    k, n = 2, (1 << 31) + 7
    say(f"odc beyond-2g n={n}: generating pushes")
    grads = [_uniform_chunked(31 + i, 0, n, torch.bfloat16) for i in range(2)]
    L = dps.dp_shard_len(n, k)
    acc = [torch.zeros(L, dtype=torch.float32, device=DEV) for _ in range(k)]
    out = [torch.empty(L, dtype=torch.bfloat16, device=DEV) for _ in range(k)]
    dps.dp_scatter_accumulate(grads, acc)
    dps.dp_settle(acc, out, n, divisor=2.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    idx = np.concatenate([rng.integers(0, n, 100_000), np.arange(k) * L, np.arange(1, k + 1) * L - 1,
                          np.arange(16), n - 1 - np.arange(16), np.arange((1 << 31) - 16, (1 << 31) + 7)])
    idx = np.unique(idx[(idx >= 0) & (idx < n)].astype(np.int64))
    ti = torch.from_numpy(idx).to(DEV)
    s = idx.size
    # the oracle on the compact samples: one owner holding all of them
    want_acc = oracle.scatter_accumulate(to_np(grads[0][ti]), [np.zeros(s, np.float32)], 1)
    want_acc = oracle.scatter_accumulate(to_np(grads[1][ti]), want_acc, 1)
    want_out = oracle.settle(want_acc, s, 1, dtype=np.uint16, divisor=2.0)[0]
    got_acc = np.empty(s, np.float32)
    got_out = np.empty(s, np.uint16)
    for c in range(k):
        m = (idx // L) == c
        j = torch.from_numpy(idx[m] - c * L).to(DEV)
        got_acc[m] = to_np(acc[c][j])
        got_out[m] = to_np(out[c][j])
    assert bits_equal(got_acc, want_acc[0])
    assert bits_equal(got_out, want_out)
