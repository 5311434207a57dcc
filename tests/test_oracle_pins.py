"""Pins that tie the oracle to the pages and to mathematics, not to itself.

CPU only. Each check below is independent of the oracle's own code: a literal
message-passing ring, exact integer sums, fp64 sums with a rounding-error
bound, library routines (numpy matmul, torch's bf16 rounding), closed-form
shapes and the pages' worked example. The mutation tests at the end plant
plausible mistakes in oracle outputs and check that a pin catches each one.
"""
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import ring_sim

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24          # unit roundoff of binary32


def _read_golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return [ln.split() for ln in fh if ln.strip() and not ln.startswith("#")]


def _rand_f32(k, n, seed):
    return [gen.uniform_pm1(seed, 0, r, n).numpy() for r in range(k)]


def _gamma(m):
    return m * U32 / (1 - m * U32)


# ------------------------------------------------------------------ generator

def test_splitmix64_published_outputs():
    want = [int(t[0]) for t in _read_golden("splitmix64_seed1234567.txt")]
    assert gen.splitmix64_sequence(1234567, 5) == want


def test_counter_based_generator_matches_sequential():
    key = gen.stream_key(3, 1, 2)
    seq = gen.splitmix64_sequence(key, 50)
    got = gen.raw_u64(3, 1, 2, 0, 50).numpy().view(np.uint64).tolist()
    assert got == seq
    part = gen.raw_u64(3, 1, 2, 17, 10).numpy().view(np.uint64).tolist()
    assert part == seq[17:27]


def test_uniform_and_int_copy_ranges():
    x = gen.uniform_pm1(1, 0, 0, 200_000)
    assert x.dtype == torch.float32
    assert float(x.min()) >= -1.0 and float(x.max()) <= 1.0 - 2.0 ** -23
    assert torch.equal(x, (x * 2 ** 23).round() / 2 ** 23)          # exact grid
    assert abs(float(x.mean())) < 0.01
    i = gen.int_copy(x)
    assert int(i.min()) >= -1000 and int(i.max()) <= 1000
    z = gen.normal(1, 2, 0, 200_000)
    assert abs(float(z.mean())) < 0.01 and abs(float(z.std()) - 1.0) < 0.01


def test_token_counts_lognormal():
    t = gen.token_counts(4, 8)
    assert len(t) == 8 and all(v >= 2 for v in t)
    many = gen.token_counts(4, 4000, docs_per_rank=1)
    med = float(np.median(many))
    assert 0.9 * np.exp(7) < med < 1.1 * np.exp(7)      # median of log-normal(7,1)


# ------------------------------------------------------- the pages' example

def test_worked_example_four_workers():
    rows = dict((r[0], r[1]) for r in _read_golden("ring_allreduce_4_workers.txt"))
    k = int(rows["workers"])
    after_rs, after_ag = ring_sim.symbolic_ring(k)
    # each worker holds exactly one fully reduced chunk ...
    for w in range(k):
        full = [c for c in range(k) if len(after_rs[w][c]) == k]
        assert full == [w]
        assert sorted(after_rs[w][w]) == sorted(f"{'abcd'[r]}{w}" for r in range(k))
    ex = sorted(rows["example_reduced_chunk"].split("+"))
    assert any(sorted(after_rs[w][w]) == ex for w in range(k))
    # ... and after AllGather every worker has every reduced chunk
    for w in range(k):
        for c in range(k):
            assert sorted(after_ag[w][c]) == sorted(f"{'abcd'[r]}{c}" for r in range(k))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 8])
def test_fold_order_is_the_ring_order(k):
    after_rs, _ = ring_sim.symbolic_ring(k)
    letters = "abcdefghijklmnopqrstuvwxyz"
    for c in range(k):
        want = tuple(f"{letters[oracle.fold_rank(c, m, k)]}{c}" for m in range(k))
        assert after_rs[c][c] == want


# ---------------------------------------------------------- ReduceScatter

@pytest.mark.parametrize("k", range(1, 9))
def test_rs_i32_bruteforce_exact(k):
    rng = np.random.default_rng(k)
    for n in range(0, 3 * k + 3):
        xs = [rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int64).astype(np.int32) for _ in range(k)]
        L = oracle.shard_len(n, k)
        got = oracle.reduce_scatter(xs)
        for c in range(k):
            for j in range(L):
                i = c * L + j
                if i < n:
                    s = sum(int(x[i]) for x in xs) % 2 ** 32
                    s = s - 2 ** 32 if s >= 2 ** 31 else s
                    assert int(got[c][j]) == s
                else:
                    assert int(got[c][j]) == 0


@pytest.mark.parametrize("k", range(1, 9))
def test_rs_f32_bruteforce_bound_and_ring(k):
    for n in range(0, 3 * k + 3):
        xs = _rand_f32(k, n, 100 + n)
        got = oracle.reduce_scatter(xs)
        ring = ring_sim.rs_f32(xs)
        L = oracle.shard_len(n, k)
        for c in range(k):
            nc = oracle.shard_valid(n, L, c)
            assert got[c][:nc].tobytes() == ring[c].tobytes()
            assert not got[c][nc:].any()
            ex = sum(x[c * L:c * L + nc].astype(np.float64) for x in xs)
            ab = sum(np.abs(x[c * L:c * L + nc].astype(np.float64)) for x in xs)
            assert np.all(np.abs(got[c][:nc] - ex) <= _gamma(k - 1) * ab)


@pytest.mark.parametrize("k,n,s", [(2, 1000, 1), (4, 1 << 14, 4), (8, 10007, 3),
                                   (7, 333, 5), (3, 2, 2)])
def test_rs_equals_literal_ring_any_s(k, n, s):
    xs = _rand_f32(k, n, 7)
    want = oracle.reduce_scatter(xs)
    L = oracle.shard_len(n, k)
    for sub in (1, s):
        got = ring_sim.rs_f32(xs, s=sub)
        for c in range(k):
            nc = oracle.shard_valid(n, L, c)
            assert got[c].tobytes() == want[c][:nc].tobytes()


def test_rs_f32_on_integer_values_equals_int32():
    k, n = 8, 5000
    xi = [gen.int_copy(gen.uniform_pm1(5, 0, r, n)).numpy() for r in range(k)]
    xf = [x.astype(np.float32) for x in xi]
    for order in ("ring", "rank"):
        a = oracle.reduce_scatter(xf, order=order)
        b = oracle.reduce_scatter(xi, order=order)
        for c in range(k):
            assert np.array_equal(a[c], b[c].astype(np.float32))


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_avg_power_of_two_is_exact_scaling(k):
    xs = _rand_f32(k, 4099, 11)
    s = oracle.reduce_scatter(xs, op="sum")
    a = oracle.reduce_scatter(xs, op="avg")
    for c in range(k):
        assert a[c].tobytes() == (s[c] * np.float32(1.0 / k)).tobytes()


@pytest.mark.parametrize("k", [3, 5, 6, 7])
def test_avg_is_one_correctly_rounded_division(k):
    xs = _rand_f32(k, 4099, 12)
    s = oracle.reduce_scatter(xs, op="sum")
    a = oracle.reduce_scatter(xs, op="avg")
    for c in range(k):
        # fp64 quotient of two fp32 values rounded once to fp32 is the
        # correctly rounded fp32 quotient (53 >= 2*24 + 2)
        want = (s[c].astype(np.float64) / k).astype(np.float32)
        assert a[c].tobytes() == want.tobytes()
        # and the ring model that divides at the owner agrees
        ring = ring_sim.rs_f32(xs, op="avg")
        L = oracle.shard_len(4099, k)
        assert ring[c].tobytes() == a[c][:oracle.shard_valid(4099, L, c)].tobytes()


# ------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_library():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(1e-3),
        rng.uniform(-1e30, 1e30, 500).astype(np.float32),
        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.3895314e38,
                  3.4028235e38, 1e-40, -1e-42, 0.0, -0.0, np.inf, -np.inf], np.float32),
    ])
    got = oracle.bf16_from_f32(vals)
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # ties to even, by hand: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert got[3000 + 500] == 0x3F80 and got[3000 + 501] == 0x3F80
    assert got[3000 + 502] == 0x3F82
    nan = oracle.bf16_from_f32(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


@pytest.mark.parametrize("k,n", [(8, 3001), (3, 20), (1, 5)])
def test_rs_bf16_avg_matches_ring_then_library_rounding(k, n):
    xb = [gen.bf16_normal(6, 3, r, n, 1e-3).view(torch.int16).numpy().view(np.uint16)
          for r in range(k)]
    xf = [oracle.bf16_to_f32(x) for x in xb]
    ring = ring_sim.rs_f32(xf, op="avg")
    got = oracle.reduce_scatter(xb, op="avg")
    L = oracle.shard_len(n, k)
    for c in range(k):
        nc = oracle.shard_valid(n, L, c)
        want = torch.from_numpy(ring[c]).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(got[c][:nc], want.view(np.uint16))
        assert not got[c][nc:].any()


# --------------------------------------------------------------- weighted

def test_weighted_unit_tokens_equals_avg():
    k, n = 8, 3333
    xs = _rand_f32(k, n, 13)
    for t in ([1] * k, [4] * k):
        w = oracle.weighted_reduce_scatter(xs, t)
        a = oracle.reduce_scatter(xs, op="avg")
        for c in range(k):
            assert w[c].tobytes() == a[c].tobytes()


def test_weighted_one_hot_returns_that_rank():
    k, n = 8, 1001
    xs = _rand_f32(k, n, 14)
    for j in range(k):
        t = [0] * k
        t[j] = 16
        w = oracle.weighted_reduce_scatter(xs, t)
        L = oracle.shard_len(n, k)
        full = np.concatenate([w[c][:oracle.shard_valid(n, L, c)] for c in range(k)])
        assert np.array_equal(np.abs(full), np.abs(xs[j]))   # +0 vs -0 may differ


def test_weighted_general_bound_and_ring():
    k, n = 8, 10_019
    xs = _rand_f32(k, n, 15)
    t = gen.token_counts(4, k)
    got = oracle.weighted_reduce_scatter(xs, t)
    L = oracle.shard_len(n, k)
    wf = np.array(t, dtype=np.float32)
    total = np.float32(sum(t))
    ring = ring_sim.rs_f32(xs, weights=wf, total=total)
    for c in range(k):
        nc = oracle.shard_valid(n, L, c)
        assert got[c][:nc].tobytes() == ring[c].tobytes()
        seg = slice(c * L, c * L + nc)
        ex = sum(np.float64(t[r]) * xs[r][seg].astype(np.float64) for r in range(k)) / sum(t)
        ab = sum(np.float64(t[r]) * np.abs(xs[r][seg].astype(np.float64)) for r in range(k)) / sum(t)
        # k products, k-1 additions, one division, token rounding to fp32
        assert np.all(np.abs(got[c][:nc] - ex) <= _gamma(k + 2) * ab + U32 * np.abs(ex))


def test_weighted_rejects_bad_tokens():
    xs = _rand_f32(2, 10, 1)
    with pytest.raises(ValueError):
        oracle.weighted_reduce_scatter(xs, [0, 0])
    with pytest.raises(ValueError):
        oracle.weighted_reduce_scatter(xs, [-1, 5])


# ---------------------------------------------------------- bf16 weighted
# The bf16 token-weighted reduction widens each bf16 gradient exactly to fp32,
# multiplies by f32(t_r), folds the products in ring order in fp32 and rounds
# once to bf16 after one division by f32(sum t). The pins below reach that
# value without the oracle: the literal ring on the widened inputs, then
# torch's round-to-nearest-even conversion; special token sets that reduce to
# the average or to one rank's gradient; and an fp64 bound.

def _bf16_grads(k, n, seed, std=1e-3):
    return [gen.bf16_normal(seed, 7, r, n, std).view(torch.int16).numpy().view(np.uint16)
            for r in range(k)]


def _widen(b):
    """bf16 bits -> fp32, exactly (the bf16 pattern is the top half of the fp32 one)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _torch_bf16_bits(f32):
    return torch.from_numpy(np.ascontiguousarray(f32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _ring_weighted_bf16(xb, tokens):
    """Independent value of the bf16 weighted ReduceScatter: literal ring over
    f32(t_r) * widened g_r, division by f32(sum t) at the owner, library RNE."""
    wf = np.array(tokens, dtype=np.float32)
    ring = ring_sim.rs_f32([_widen(x) for x in xb], weights=wf, total=np.float32(sum(tokens)))
    return [_torch_bf16_bits(r) for r in ring]


@pytest.mark.parametrize("k,n", [(8, 3001), (3, 200), (5, 41)])
def test_weighted_bf16_constant_power_of_two_tokens_equal_avg(k, n):
    xb = _bf16_grads(k, n, 60 + k)
    avg = oracle.reduce_scatter(xb, op="avg")
    for c_tok in (1, 4, 64):
        w = oracle.weighted_reduce_scatter(xb, [c_tok] * k)
        for c in range(k):
            assert w[c].tobytes() == avg[c].tobytes(), (k, c_tok, c)


def test_weighted_bf16_one_hot_returns_that_ranks_bits():
    k, n = 8, 2001
    xb = _bf16_grads(k, n, 61, std=1.0)
    L = oracle.shard_len(n, k)
    for j in range(k):
        for m in (0, 3, 10):
            t = [0] * k
            t[j] = 2 ** m
            w = oracle.weighted_reduce_scatter(xb, t)
            full = np.concatenate([w[c][:oracle.shard_valid(n, L, c)] for c in range(k)])
            nz = (xb[j] & 0x7FFF) != 0
            assert np.array_equal(full[nz], xb[j][nz]), (j, m)
            assert not (full[~nz] & 0x7FFF).any()            # zeros stay zero (sign may differ)


@pytest.mark.parametrize("k,n,seed", [(8, 10_019, 62), (6, 4097, 63), (2, 999, 64)])
def test_weighted_bf16_general_tokens_ring_then_library_rounding(k, n, seed):
    xb = _bf16_grads(k, n, seed)
    t = gen.token_counts(seed, k)
    got = oracle.weighted_reduce_scatter(xb, t)
    want = _ring_weighted_bf16(xb, t)
    L = oracle.shard_len(n, k)
    for c in range(k):
        nc = oracle.shard_valid(n, L, c)
        assert np.array_equal(got[c][:nc], want[c]), c
        assert not got[c][nc:].any()
        # within the fp32 accumulation bound plus one bf16 rounding of the result
        seg = slice(c * L, c * L + nc)
        xs = [_widen(x[seg]).astype(np.float64) for x in xb]
        ex = sum(np.float64(t[r]) * xs[r] for r in range(k)) / sum(t)
        ab = sum(np.float64(t[r]) * np.abs(xs[r]) for r in range(k)) / sum(t)
        g = _widen(got[c][:nc]).astype(np.float64)
        assert np.all(np.abs(g - ex) <= _gamma(k + 2) * ab + 2.0 ** -8 * np.abs(ex))


def test_weighted_bf16_all_reduce_is_rs_then_ag():
    k, n = 8, 5003
    xb = _bf16_grads(k, n, 65)
    t = gen.token_counts(65, k)
    ar = oracle.weighted_all_reduce(xb, t)
    ag = oracle.all_gather(oracle.weighted_reduce_scatter(xb, t), n)
    want = np.concatenate(_ring_weighted_bf16(xb, t))
    for r in range(k):
        assert ar[r].tobytes() == ag[r].tobytes() == want.tobytes()


# Planted mistakes in the bf16 weighted reduction, each computed here in numpy
# from the widened inputs; the ring-then-library pin above must reject every
# one of them and accept the oracle.

def _mutant_weighted_bf16(xb, tokens, kind):
    k = len(xb)
    n = xb[0].size
    L = oracle.shard_len(n, k)
    wf = np.array(tokens, dtype=np.float32)
    total = np.float32(sum(tokens))
    out = []
    for c in range(k):
        seg = slice(c * L, c * L + oracle.shard_valid(n, L, c))
        order = [oracle.fold_rank(c, m, k, "rank" if kind == "rank_order" else "ring")
                 for m in range(k)]
        acc = None
        for r in order:
            g = _widen(xb[r][seg])
            if kind == "product_rounded_to_bf16":
                p = _widen(_torch_bf16_bits(wf[r] * g))
            elif kind == "divide_before_fold":
                p = (wf[r] / total) * g
            else:
                p = wf[r] * g
            acc = p if acc is None else (acc + p).astype(np.float32)
        if kind != "divide_before_fold":
            acc = (acc / total).astype(np.float32)
        out.append(_torch_bf16_bits(acc))
    return out


def _cancelling_bf16(k, n, seed):
    """bf16 gradients in which, at every index, two ranks hold +2^30 and -2^30
    and the others values in [-1, 1): the fp32 fold then depends on the order
    far beyond its last bit (what is added before the pair cancels is lost)."""
    rng = np.random.default_rng(seed)
    small = [_torch_bf16_bits(rng.uniform(-1, 1, n).astype(np.float32)) for _ in range(k)]
    big = np.uint16(0x4E80)                                  # 2^30
    for i in range(n):
        p, q = rng.choice(k, 2, replace=False)
        small[p][i] = big
        small[q][i] = big | np.uint16(0x8000)
    return small


@pytest.mark.parametrize("kind", ["product_rounded_to_bf16", "divide_before_fold", "rank_order"])
def test_mutant_weighted_bf16_is_caught(kind):
    k, n = 8, 20_011
    if kind == "rank_order":
        # equal tokens keep each cancelling pair's products equal and opposite
        xb, t = _cancelling_bf16(k, n, 66), [5] * k
    else:
        xb, t = _bf16_grads(k, n, 66, std=1.0), gen.token_counts(66, k)
    want = _ring_weighted_bf16(xb, t)
    L = oracle.shard_len(n, k)
    got = oracle.weighted_reduce_scatter(xb, t)
    assert all(np.array_equal(got[c][:oracle.shard_valid(n, L, c)], want[c]) for c in range(k))
    bad = _mutant_weighted_bf16(xb, t, kind)
    assert not all(np.array_equal(bad[c], want[c]) for c in range(k))
    # the correct computation written the same way passes the pin
    good = _mutant_weighted_bf16(xb, t, "none")
    assert all(np.array_equal(good[c], want[c]) for c in range(k))


# ------------------------------------------------------ IEEE special values
# The oracle's folds on the special-value scenarios that the GPU parity tests
# use, against what IEEE binary32 arithmetic and round-to-nearest-even fix for
# each scenario, whatever the fold order.

def _special_case(dtype, k, n, seed, op):
    from tests.special_values import scenarios, special_inputs
    bits = special_inputs(dtype, k, n, seed)
    host = [b if dtype == torch.bfloat16 else b.view(np.float32) for b in bits]
    out = np.concatenate(oracle.reduce_scatter(host, op=op))[:n]
    return bits, scenarios(n, seed), (out if dtype == torch.bfloat16 else out.view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k,op", [(8, "sum"), (8, "avg"), (6, "avg")])
def test_oracle_on_special_values(dtype, k, op):
    from tests.special_values import BF16, F32, _is_nan
    bf = dtype == torch.bfloat16
    S = BF16 if bf else F32
    n = 40_000
    bits, scen, out = _special_case(dtype, k, n, 7, op)
    mag = out & (0x7FFF if bf else 0x7FFFFFFF)
    inf = mag == (S["pinf"])
    nan = _is_nan(out, out.dtype)
    sign = (out >> (15 if bf else 31)) & 1
    # every rank -0.0: the fold keeps -0.0 (no +0.0 seed), and so does 1/K
    assert np.all(out[scen == 4] == S["nz"])
    # +Inf with -Inf, or any NaN operand: NaN
    assert np.all(nan[scen == 7]) and np.all(nan[scen == 8]) and np.all(nan[scen == 9])
    # one infinity among finite values: that infinity
    assert np.all(inf[scen == 6])
    # all subnormal operands: the exact sum is a subnormal or the smallest
    # normals, never zero unless it cancels, and never NaN or Inf
    assert not np.any(nan[scen == 10] | inf[scen == 10])
    if op == "sum":
        if bf:
            # max + 2^119 is the tie above max: rounds to even, i.e. to Inf;
            # max + 2^118 stays max
            assert np.all(inf[scen == 12]) and np.all(mag[scen == 13] == S["max"])
            # 1 + 2^-8 -> 1, (1 + 2^-7) + 2^-8 -> 1 + 2^-6 (ties to even)
            t = mag[scen == 14]
            assert np.all((t == 0x3F80) | (t == 0x3F82))
        else:
            assert np.all(inf[(scen == 12) | (scen == 13)])
            t = mag[scen == 14]
            # 1 + 2^-24 -> 1, (1 + 2^-23) + 2^-24 -> 1 + 2^-22
            assert np.all((t == 0x3F800000) | (t == 0x3F800002))
    # the sign of a tie or overflow follows its operands' common sign
    for sc in (12, 13, 14):
        m = scen == sc
        src_sign = np.zeros(n, np.int64)
        for b in bits:
            v = b & (0x7FFF if bf else 0x7FFFFFFF)
            src_sign = np.where(v != 0, (b >> (15 if bf else 31)) & 1, src_sign)
        assert np.array_equal(sign[m], src_sign[m])


# -------------------------------------------------- AllGather / AllReduce

@pytest.mark.parametrize("k,n", [(1, 7), (3, 10), (4, 1 << 12), (8, 8 * 33 + 5), (8, 3)])
def test_all_gather_slices_back(k, n):
    L = oracle.shard_len(n, k)
    shards = [np.arange(c * 1000, c * 1000 + L, dtype=np.int32) for c in range(k)]
    outs = oracle.all_gather(shards, n)
    for r in range(k):
        assert outs[r].tobytes() == outs[0].tobytes()
    for c in range(k):
        nc = oracle.shard_valid(n, L, c)
        assert np.array_equal(outs[0][c * L:c * L + nc], shards[c][:nc])


@pytest.mark.parametrize("k,n,op", [(4, 1 << 12, "sum"), (4, 1 << 12, "avg"), (8, 1003, "avg"),
                                    (5, 17, "sum"), (1, 9, "avg")])
def test_all_reduce_is_rs_then_ag_and_literal_ring(k, n, op):
    xs = _rand_f32(k, n, 21)
    ar = oracle.all_reduce(xs, op=op)
    ag = oracle.all_gather(oracle.reduce_scatter(xs, op=op), n)
    ring = ring_sim.ar_f32(xs, s=3, op=op)
    for r in range(k):
        assert ar[r].tobytes() == ag[r].tobytes() == ring[r].tobytes()


def test_weighted_all_reduce_is_rs_then_ag():
    k, n = 8, 10_019
    xs = _rand_f32(k, n, 22)
    t = gen.token_counts(4, k)
    ar = oracle.weighted_all_reduce(xs, t)
    ag = oracle.all_gather(oracle.weighted_reduce_scatter(xs, t), n)
    for r in range(k):
        assert ar[r].tobytes() == ag[r].tobytes()


def test_rs_at_matches_full():
    k, n = 8, 20_011
    xb = [gen.bf16_normal(6, 3, r, n, 1e-3).view(torch.int16).numpy().view(np.uint16)
          for r in range(k)]
    full = oracle.reduce_scatter(xb, op="avg")
    idx = np.array([0, 1, 2500, 2501, 19_999, 20_010, 7777], np.int64)
    L = oracle.shard_len(n, k)
    got = oracle.rs_at(xb, idx, op="avg")
    for s, i in enumerate(idx):
        assert got[s] == full[i // L][i % L]


def test_fold_at_matches_full():
    k, n = 8, 4001
    xs = _rand_f32(k, n, 23)
    full = oracle.reduce_scatter(xs, op="avg")
    L = oracle.shard_len(n, k)
    idx = np.array([0, 500, 501, 1999, 4000, 3500], np.int64)
    comp = [np.ascontiguousarray(x[idx]) for x in xs]
    got = oracle.fold_at(comp, idx // L, op="avg")
    assert np.array_equal(got, np.array([full[i // L][i % L] for i in idx], np.float32))


def test_fold_bf16_at_matches_full_and_ring():
    """The compact bf16 fold at sampled indices, shard boundaries included,
    equals the full bf16 ReduceScatter and the literal ring on the widened
    inputs followed by the library's rounding."""
    k, n = 8, 4001
    xb = _bf16_grads(k, n, 67, std=1.0)
    L = oracle.shard_len(n, k)
    idx = np.array([0, 1, L - 1, L, 2 * L - 1, 2 * L, 7 * L - 1, 7 * L, n - 1, 1234, 3001],
                   np.int64)
    comp = [np.ascontiguousarray(x[idx]) for x in xb]
    for op in ("sum", "avg"):
        full = oracle.reduce_scatter(xb, op=op)
        ring = ring_sim.rs_f32([_widen(x) for x in xb], op=op)
        got = oracle.fold_at(comp, idx // L, op=op)
        for s_, i in enumerate(idx):
            c, j = int(i // L), int(i % L)
            assert got[s_] == full[c][j], (op, i)
            assert got[s_] == _torch_bf16_bits(ring[c][j:j + 1])[0], (op, i)


def test_rs_f32_at_matches_full():
    k, n = 6, 9_001
    xs = _rand_f32(k, n, 68)
    L = oracle.shard_len(n, k)
    idx = np.array([0, L - 1, L, 3 * L + 5, n - 1, 4000], np.int64)
    for op in ("sum", "avg"):
        full = oracle.reduce_scatter(xs, op=op)
        ring = ring_sim.rs_f32(xs, op=op)
        got = oracle.rs_at(xs, idx, op=op)
        for s_, i in enumerate(idx):
            assert got[s_] == full[i // L][i % L] == ring[i // L][i % L]


# ------------------------------------------------------------------ shapes

def test_shard_shapes_from_the_pages():
    for g_rows, g_cols, dev, l_rows, l_cols in (map(int, r) for r in _read_golden("shard_shapes.txt")):
        assert oracle.shard_len(g_rows, dev) == l_rows
        assert oracle.shard_len(g_rows * g_cols, dev) == l_rows * l_cols
    assert oracle.shard_len(1_048_576, 4) == 262_144
    L = oracle.shard_len(10_000_019, 8)
    assert L == 1_250_003
    assert oracle.shard_valid(10_000_019, L, 7) == 1_249_998
    assert oracle.shard_len(0, 8) == 0
    assert [oracle.shard_valid(3, 1, c) for c in range(8)] == [1, 1, 1, 0, 0, 0, 0, 0]


# ------------------------------------------------------------------- GEMM

def test_gemm_f64_matches_numpy():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((37, 53)).astype(np.float32)
    b = rng.standard_normal((53, 29)).astype(np.float32)
    c, ab = oracle.gemm_f64(a, b)
    ref = a.astype(np.float64) @ b.astype(np.float64)
    assert np.allclose(c, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    assert np.allclose(ab, np.abs(a).astype(np.float64) @ np.abs(b).astype(np.float64))
    ct, _ = oracle.gemm_f64(np.ascontiguousarray(a.T), b, trans_a=True)
    assert np.array_equal(ct, c)


def test_gemm_bf16_at_matches_numpy():
    """Both B layouts against numpy's fp64 product of the exactly widened bf16
    values, with the |A||B| sums."""
    a = gen.bf16_normal(5, 30, 0, 40 * 96, 1.0).view(40, 96)
    b_kn = gen.bf16_normal(5, 31, 0, 96 * 24, 1.0).view(96, 24)
    b_nk = b_kn.t().contiguous()
    ab = a.view(torch.int16).numpy().view(np.uint16)
    rows = np.array([0, 3, 39, 17], np.int64)
    cols = np.array([0, 23, 5, 11], np.int64)
    ref = a.double().numpy() @ b_kn.double().numpy()
    refa = np.abs(a.double().numpy()) @ np.abs(b_kn.double().numpy())
    for layout, b in (("kn", b_kn), ("nk", b_nk)):
        vals, absv = oracle.gemm_bf16_at(ab, b.view(torch.int16).numpy().view(np.uint16), rows,
                                         cols, b_layout=layout)
        assert np.allclose(vals, ref[rows, cols], rtol=0, atol=1e-12), layout
        assert np.allclose(absv, refa[rows, cols], rtol=1e-15), layout
    # the [n,kk] array read as if it were [kk,n] (a layout mix-up) is caught
    nk_bits = b_nk.view(torch.int16).numpy().view(np.uint16)
    bad, _ = oracle.gemm_bf16_at(ab, nk_bits.reshape(96, 24), rows, cols, b_layout="kn")
    assert not np.allclose(bad, ref[rows, cols], atol=1e-6)


def test_fsdp_global_view_invariance():
    """Concatenating the ranks' y gives x @ w, and the dW shards concatenate to
    x^T dy (global-view invariance of sharded arrays)."""
    fx = gen.fsdp_fixture(k=8, m=64, d=32, f=24)
    k, x, w, dy = 8, fx["x"].numpy(), fx["w"].numpy(), fx["dy"].numpy()
    ml, R = 64 // k, oracle.shard_len(32, k)
    xl = [np.ascontiguousarray(x[r * ml:(r + 1) * ml]) for r in range(k)]
    dyl = [np.ascontiguousarray(dy[r * ml:(r + 1) * ml]) for r in range(k)]
    ws = [np.ascontiguousarray(w[c * R:(c + 1) * R]) for c in range(k)]
    out = oracle.fsdp_layer(xl, ws, dyl)
    for r in range(k):
        assert np.array_equal(out["w_full"][r], w)
    y = np.concatenate(out["y"])
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.allclose(y, ref, rtol=0, atol=1e-12)
    dw = np.concatenate(out["dw_shard"])
    refd = x.astype(np.float64).T @ dy.astype(np.float64)
    assert np.allclose(dw, refd, rtol=0, atol=1e-11)


def test_fsdp_non_divisible_rows_pad():
    k, ml, d, f = 3, 4, 7, 5
    rng = np.random.default_rng(3)
    w = rng.integers(-4, 5, (d, f)).astype(np.float32)
    xl = [rng.integers(-4, 5, (ml, d)).astype(np.float32) for _ in range(k)]
    dyl = [rng.integers(-4, 5, (ml, f)).astype(np.float32) for _ in range(k)]
    R = oracle.shard_len(d, k)
    ws = []
    for c in range(k):
        s = np.zeros((R, f), np.float32)
        rows = w[c * R:(c + 1) * R]
        s[:len(rows)] = rows
        ws.append(s)
    out = oracle.fsdp_layer(xl, ws, dyl)
    assert np.array_equal(out["w_full"][0], w)
    dw = sum(x.T.astype(np.float64) @ dy.astype(np.float64) for x, dy in zip(xl, dyl))
    for c in range(k):
        rows = dw[c * R:(c + 1) * R]
        assert np.array_equal(out["dw_shard"][c][:len(rows)], rows)
        assert not out["dw_shard"][c][len(rows):].any()


# ------------------------------------------------------ planted mistakes
# Each mutant below is a plausible bug in the oracle; the pins above must
# reject it. Mistakes are planted in oracle outputs on the CPU only.

def _ring_pin(rs_fn, k=5, n=1003):
    xs = _rand_f32(k, n, 31)
    ring = ring_sim.rs_f32(xs)
    got = rs_fn(xs)
    L = oracle.shard_len(n, k)
    return all(got[c][:oracle.shard_valid(n, L, c)].tobytes() == ring[c].tobytes()
               for c in range(k))


def test_mutant_rank_order_is_caught():
    assert _ring_pin(lambda xs: oracle.reduce_scatter(xs))
    assert not _ring_pin(lambda xs: oracle.reduce_scatter(xs, order="rank"))


def test_mutant_dropped_term_is_caught():
    assert not _ring_pin(lambda xs: oracle.reduce_scatter(xs[:-1] + [np.zeros_like(xs[-1])]))


def test_mutant_shard_swap_is_caught():
    def swapped(xs):
        s = oracle.reduce_scatter(xs)
        return [s[1], s[0]] + s[2:]
    assert not _ring_pin(swapped)


def test_mutant_transposed_operand_is_caught():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((16, 16)).astype(np.float32)
    b = rng.standard_normal((16, 16)).astype(np.float32)
    ref = a.astype(np.float64) @ b.astype(np.float64)
    bad, _ = oracle.gemm_f64(np.ascontiguousarray(a.T), b)   # A transposed by mistake
    assert not np.allclose(bad, ref, atol=1e-9)


def test_mutant_divide_by_wrong_count_is_caught():
    k = 4
    xs = _rand_f32(k, 999, 32)
    s = oracle.reduce_scatter(xs, op="sum")
    wrong = [x / np.float32(k - 1) for x in s]
    assert any(w.tobytes() != (x * np.float32(1 / k)).tobytes() for w, x in zip(wrong, s))


# --------------------------------------- scatter-accumulate and one settle

def _microbatches(k, counts, n, seed, integer=False):
    """g[r][m]: rank r's m-th microbatch gradient, fp32."""
    out = []
    for r in range(k):
        gs = []
        for m in range(counts[r]):
            x = gen.uniform_pm1(seed, 40 + m, r, n)
            gs.append((gen.int_copy(x).to(torch.float32) if integer else x).numpy())
        out.append(gs)
    return out


def test_scatter_accumulate_settle_is_the_exact_sum_on_integers():
    """Pushes of uneven microbatch counts in any order, then one settle, give
    sum over ranks and microbatches (exact for integer values)."""
    k, n, counts = 4, 1001, [1, 3, 0, 2]
    g = _microbatches(k, counts, n, 50, integer=True)
    exact = sum(gm.astype(np.int64) for gr in g for gm in gr)
    L = oracle.shard_len(n, k)
    rng = np.random.default_rng(0)
    pushes = [(r, m) for r in range(k) for m in range(counts[r])]
    for order in (pushes, list(reversed(pushes)), [pushes[i] for i in rng.permutation(len(pushes))]):
        acc = [np.zeros(L, np.float32) for _ in range(k)]
        for r, m in order:
            oracle.scatter_accumulate(g[r][m], acc, k)
        out = oracle.settle(acc, n, k)
        full = np.concatenate([out[c][:oracle.shard_valid(n, L, c)] for c in range(k)])
        assert np.array_equal(full.astype(np.int64), exact)


def test_padded_reduce_scatter_steps_match_on_integers():
    """The collective baseline pads every rank to the largest microbatch count
    with empty (zero) gradients and reduce-scatters step by step; on integer
    values it reaches the same sums as the pushes."""
    k, n, counts = 4, 777, [2, 1, 3, 1]
    g = _microbatches(k, counts, n, 51, integer=True)
    L = oracle.shard_len(n, k)
    acc_push = [np.zeros(L, np.float32) for _ in range(k)]
    for r in range(k):
        for gm in g[r]:
            oracle.scatter_accumulate(gm, acc_push, k)
    acc_pad = [np.zeros(L, np.float32) for _ in range(k)]
    zero = np.zeros(n, np.float32)
    for m in range(max(counts)):
        step = [g[r][m] if m < counts[r] else zero for r in range(k)]
        shards = oracle.reduce_scatter(step, op="sum")
        oracle.scatter_accumulate(np.concatenate(shards), acc_pad, k, L=L)
    for c in range(k):
        assert np.array_equal(acc_push[c], acc_pad[c])


def test_scatter_accumulate_within_summation_bound():
    k, n, counts = 8, 2003, [3, 1, 1, 4, 2, 1, 1, 2]
    g = _microbatches(k, counts, n, 52)
    L = oracle.shard_len(n, k)
    acc = [np.zeros(L, np.float32) for _ in range(k)]
    for r in range(k):
        for gm in g[r]:
            oracle.scatter_accumulate(gm, acc, k)
    got = np.concatenate([acc[c][:oracle.shard_valid(n, L, c)] for c in range(k)])
    ex = sum(gm.astype(np.float64) for gr in g for gm in gr)
    ab = sum(np.abs(gm.astype(np.float64)) for gr in g for gm in gr)
    assert np.all(np.abs(got - ex) <= _gamma(sum(counts)) * ab)


def test_settle_scaling_and_rounding():
    k, n = 3, 100
    acc = [gen.uniform_pm1(53, 0, c, 34).numpy() * np.float32(64) for c in range(k)]
    out = oracle.settle(acc, n, k, divisor=4.0)
    for c in range(k):
        nc = oracle.shard_valid(n, 34, c)
        assert out[c][:nc].tobytes() == (acc[c][:nc] * np.float32(0.25)).tobytes()
        assert not out[c][nc:].any()
    ob = oracle.settle(acc, n, k, dtype=np.uint16, divisor=4.0)
    want = torch.from_numpy(np.concatenate([(acc[c] * np.float32(0.25))[:oracle.shard_valid(n, 34, c)]
                                            for c in range(k)])).to(torch.bfloat16)
    got = np.concatenate([ob[c][:oracle.shard_valid(n, 34, c)] for c in range(k)])
    assert np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16))


def test_mutant_lost_push_is_caught():
    """Dropping one push (a gradient that never lands before the settle) is
    caught by the exact-sum pin."""
    k, n, counts = 4, 301, [1, 2, 1, 1]
    g = _microbatches(k, counts, n, 54, integer=True)
    exact = sum(gm.astype(np.int64) for gr in g for gm in gr)
    L = oracle.shard_len(n, k)
    acc = [np.zeros(L, np.float32) for _ in range(k)]
    for r in range(k):
        for gm in g[r][:1]:                      # rank r's later microbatches are lost
            oracle.scatter_accumulate(gm, acc, k)
    full = np.concatenate([acc[c][:oracle.shard_valid(n, L, c)] for c in range(k)])
    assert not np.array_equal(full.astype(np.int64), exact)
