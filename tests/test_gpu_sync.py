"""GPU parity of the sync kernels against the oracle, through the C ABI.

Every comparison is bit-exact: with the ring fold order fixed on both sides,
ReduceScatter, AllGather, AllReduce and the token-weighted reduction have one
correct result for f32, bf16 and int32.
"""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
import oracle
from gradient_sync_amd.buckets import BucketedSync, rank_buffers
from gradient_sync_amd.concurrency import CuMaskedStream
from tests.helpers import bits_equal, from_np, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
CANARY = 0x5A
GUARD = 64          # guard elements on each side of an output


class Guarded:
    """A device buffer of `n` elements at element offset `off` inside a larger
    allocation whose surroundings hold a canary pattern."""

    def __init__(self, n, dtype, off=0):
        self.full = torch.empty(n + off + 2 * GUARD, dtype=dtype, device=DEV)
        self.full.view(torch.uint8).fill_(CANARY)
        self.lo = GUARD + off
        self.t = self.full[self.lo:self.lo + n]

    def intact(self):
        raw = self.full.view(torch.uint8).cpu().numpy()
        es = self.full.element_size()
        return bool(np.all(raw[:self.lo * es] == CANARY) and
                    np.all(raw[(self.lo + self.t.numel()) * es:] == CANARY))


def make_inputs(dtype, k, n, seed, off=0):
    """K device input buffers (at element offset off) and their host copies."""
    xs = []
    for r in range(k):
        u = gen.uniform_pm1(seed, 0, r, n)
        if dtype == torch.int32:
            # full-range values so that the sums wrap
            v = gen.raw_u64(seed, 1, r, 0, n).to(torch.int32)
        elif dtype == torch.bfloat16:
            v = u.to(torch.bfloat16)
        else:
            v = u
        g = Guarded(n, dtype, off)
        g.t.copy_(v.to(DEV))
        xs.append(g)
    return xs, [to_np(g.t) for g in xs]


def _magnitude(a):
    """Bit pattern without the sign bit."""
    if a.dtype == np.uint16:
        return a & 0x7FFF
    return a.view(np.uint32) & 0x7FFFFFFF


# ------------------------------------------------------------ ReduceScatter

CASES_K = [1, 2, 3, 4, 5, 7, 8, 16, 64]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_rs_bruteforce_small(dtype):
    for k in CASES_K:
        small = range(0, 3 * k + 3) if k <= 8 else [0, 1, k - 1, k, k + 1, 2 * k + 3, 3 * k + 2]
        ns = sorted(set(list(small) + [97, 1000, 4099]))
        for n in ns:
            xs, hx = make_inputs(dtype, k, n, seed=1000 + k * 7 + n)
            L = dps.dp_shard_len(n, k)
            for op in (["sum"] if dtype == torch.int32 else ["sum", "avg"]):
                for s in (1, 3):
                    say(f"rs k={k} n={n} {dtype} {op} S={s}")
                    outs = [Guarded(max(L, 0), dtype) for _ in range(k)]
                    dps.dp_reduce_scatter([g.t for g in xs], [o.t for o in outs], op=op,
                                          s_chunks=s, n=n)
                    torch.cuda.synchronize()
                    want = oracle.reduce_scatter(hx, op=op)
                    for c in range(k):
                        assert bits_equal(to_np(outs[c].t), want[c]), (k, n, op, s, c)
                        assert outs[c].intact()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_rs_every_alignment(dtype):
    """Input offsets shift the address phase of every shard; output offsets
    make input and output phases differ (element-wise path)."""
    k, n = 8, 3 * 4096 + 37
    L = dps.dp_shard_len(n, k)
    for in_off in (0, 1, 2, 3, 5, 7):
        xs, hx = make_inputs(dtype, k, n, seed=77 + in_off, off=in_off)
        want = oracle.reduce_scatter(hx, op="sum")
        for out_off in (0, 1, 3, in_off):
            say(f"rs-align {dtype} in_off={in_off} out_off={out_off}")
            outs = [Guarded(L, dtype, out_off) for _ in range(k)]
            dps.dp_reduce_scatter([g.t for g in xs], [o.t for o in outs], op="sum")
            torch.cuda.synchronize()
            for c in range(k):
                assert bits_equal(to_np(outs[c].t), want[c]), (in_off, out_off, c)
                assert outs[c].intact()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("k,n", [(2, 2 * 3 * 4096 + 5), (4, (1 << 20) + 3), (6, 123_457),
                                 (8, 8 * 2048 * 5 - 1), (3, 1 << 16)])
def test_rs_multi_tile_ragged(dtype, k, n):
    xs, hx = make_inputs(dtype, k, n, seed=5)
    L = dps.dp_shard_len(n, k)
    for op in ("sum", "avg"):
        say(f"rs-tiles k={k} n={n} {dtype} {op}")
        outs = [Guarded(L, dtype) for _ in range(k)]
        dps.dp_reduce_scatter([g.t for g in xs], [o.t for o in outs], op=op)
        torch.cuda.synchronize()
        want = oracle.reduce_scatter(hx, op=op, nthreads=8)
        for c in range(k):
            assert bits_equal(to_np(outs[c].t), want[c])
            assert outs[c].intact()


# --------------------------------------------------------------- AllGather

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_ag_bruteforce_and_alignment(dtype):
    for k in (1, 2, 3, 8, 16):
        for n in (0, 1, k - 1 if k > 1 else 1, k + 1, 3 * k + 2, 1000, 3 * 4096 + 37):
            L = dps.dp_shard_len(n, k)
            for sh_off, out_off in ((0, 0), (1, 0), (0, 3), (5, 5)):
                say(f"ag k={k} n={n} {dtype} sh_off={sh_off} out_off={out_off}")
                shards = []
                for c in range(k):
                    g = Guarded(L, dtype, sh_off)
                    v = gen.raw_u64(9, 2, c, 0, L).to(torch.int32)
                    g.t.copy_((v if dtype == torch.int32 else
                               (v.to(torch.float32) * 2.0 ** -31).to(dtype)).to(DEV))
                    shards.append(g)
                outs = [Guarded(n, dtype, out_off) for _ in range(k)]
                dps.dp_all_gather([g.t for g in shards], [o.t for o in outs], n=n)
                torch.cuda.synchronize()
                want = oracle.all_gather([to_np(g.t) for g in shards], n)
                for r in range(k):
                    assert bits_equal(to_np(outs[r].t), want[r]), (k, n, r)
                    assert outs[r].intact()


# --------------------------------------------------------------- AllReduce

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
@pytest.mark.parametrize("k,n", [(4, 10_001), (8, 8 * 4096 * 3 + 11), (5, 777), (1, 100),
                                 (16, 50_000)])
def test_ar_is_rs_then_ag(dtype, k, n):
    xs, hx = make_inputs(dtype, k, n, seed=k + n)
    op = "sum" if dtype == torch.int32 else "avg"
    say(f"ar k={k} n={n} {dtype} {op}")
    outs = [Guarded(n, dtype) for _ in range(k)]
    dps.dp_all_reduce([g.t for g in xs], [o.t for o in outs], op=op, s_chunks=2)
    torch.cuda.synchronize()
    want = oracle.all_reduce(hx, op=op)
    # the same through the two separate calls on the GPU
    L = dps.dp_shard_len(n, k)
    sh = [torch.empty(L, dtype=dtype, device=DEV) for _ in range(k)]
    outs2 = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
    dps.dp_reduce_scatter([g.t for g in xs], sh, op=op)
    dps.dp_all_gather(sh, outs2, n=n)
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(outs[r].t), want[r])
        assert bits_equal(to_np(outs2[r]), want[r])
        assert outs[r].intact()
    # in place: recv == send
    dps.dp_all_reduce([g.t for g in xs], [g.t for g in xs], op=op)
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(xs[r].t), want[r])
        assert xs[r].intact()


def test_rs_and_ag_in_place_forms():
    k, n = 8, 8 * 5000
    dtype = torch.float32
    xs, hx = make_inputs(dtype, k, n, seed=3)
    L = n // k
    want = oracle.reduce_scatter(hx, op="avg")
    # ReduceScatter with recv[c] = send[c] + c*L
    dps.dp_reduce_scatter([g.t for g in xs], [g.t[c * L:(c + 1) * L] for c, g in enumerate(xs)],
                          op="avg")
    torch.cuda.synchronize()
    for c in range(k):
        assert bits_equal(to_np(xs[c].t[c * L:(c + 1) * L]), want[c])
    # AllGather with send[c] = recv[c] + c*L
    dps.dp_all_gather([g.t[c * L:(c + 1) * L] for c, g in enumerate(xs)], [g.t for g in xs], n=n)
    torch.cuda.synchronize()
    full = oracle.all_gather(want, n)
    for r in range(k):
        assert bits_equal(to_np(xs[r].t), full[r])


def test_invariant_to_s_and_repeatable():
    k, n = 8, 1_000_003
    for dtype in (torch.float32, torch.bfloat16):
        xs, hx = make_inputs(dtype, k, n, seed=11)
        want = oracle.all_reduce(hx, op="avg", nthreads=8)
        for s in (1, 2, 7, 64):
            say(f"S-invariance {dtype} S={s}")
            for rep in range(2):
                outs = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
                dps.dp_all_reduce([g.t for g in xs], outs, op="avg", s_chunks=s)
                torch.cuda.synchronize()
                for r in (0, k - 1):
                    assert bits_equal(to_np(outs[r]), want[r]), (dtype, s, rep)


def test_side_stream():
    k, n = 4, 300_000
    xs, hx = make_inputs(torch.float32, k, n, seed=12)
    st = torch.cuda.Stream()
    outs = [torch.empty(n, device=DEV) for _ in range(k)]
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        dps.dp_all_reduce([g.t for g in xs], outs, op="sum")
    st.synchronize()
    want = oracle.all_reduce(hx, op="sum")
    assert bits_equal(to_np(outs[2]), want[2])


def test_cu_masked_stream():
    """On a stream confined to 64 of the CUs (hipExtStreamCreateWithCUMask, the
    resource partitioning the concurrency measurement uses) the pipelined
    bucket step and the one-pass AllReduce give the oracle's bits."""
    with CuMaskedStream(0, 64) as ms:
        st = ms.stream
        k, total, cap = 8, 2_500_003, 1_000_003
        grads = [x.to(torch.bfloat16) for x in gen.ring_uniform_inputs(77, k, total, device=DEV)]
        out = [torch.full((total,), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(k)]
        sync = BucketedSync(grads, out, cap, op="avg")
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            sync.step_pipelined()
        st.synchronize()
        host = [to_np(g) for g in grads]
        for off, n in sync.plan:
            want = oracle.all_reduce([np.ascontiguousarray(h[off:off + n]) for h in host], op="avg")
            assert bits_equal(to_np(out[5][off:off + n]), want[5])
        for o in out:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            dps.dp_all_reduce(grads, out, op="sum")
        st.synchronize()
        assert bits_equal(to_np(out[0]), oracle.all_reduce(host, op="sum")[0])


# ------------------------------------------------------------ weighted

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_weighted_special_cases(dtype):
    k, n = 8, 77_777
    xs, hx = make_inputs(dtype, k, n, seed=13)
    outs = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
    ref = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
    say(f"weighted t=1 {dtype}")
    dps.dp_weighted_reduce([g.t for g in xs], outs, [1] * k)
    dps.dp_all_reduce([g.t for g in xs], ref, op="avg")
    torch.cuda.synchronize()
    assert bits_equal(to_np(outs[0]), to_np(ref[0]))
    for j in (0, 5):
        t = [0] * k
        t[j] = 64
        dps.dp_weighted_reduce([g.t for g in xs], outs, t)
        torch.cuda.synchronize()
        # one-hot power-of-two weight returns rank j's values (up to the sign of zero)
        assert np.array_equal(_magnitude(to_np(outs[3])), _magnitude(hx[j]))
    for toks in ([3, 1, 4, 1, 5, 9, 2, 6], [1000, 0, 0, 7, 123456, 1, 1, 2]):
        say(f"weighted {toks} {dtype}")
        dps.dp_weighted_reduce([g.t for g in xs], outs, toks, s_chunks=3)
        torch.cuda.synchronize()
        want = oracle.weighted_all_reduce(hx, toks)
        for r in range(k):
            assert bits_equal(to_np(outs[r]), want[r])


# ------------------------------------------------------- workloads, full size

def test_ring_allreduce_k4_1m_fp32_and_int32():
    """K=4 ranks, 1,048,576 fp32 gradients uniform in [-1,1), S=4, averaged;
    and the int32 copy round(1000 x), summed. Bit-exact, through RS+AG and AR."""
    k, n, s = 4, 1_048_576, 4
    xf = gen.ring_uniform_inputs(1, k, n, device=DEV)
    xi = [gen.int_copy(x) for x in xf]
    for xs, op in ((xf, "avg"), (xi, "sum"), ([x.to(torch.float32) for x in xi], "sum")):
        say(f"k4-1m {xs[0].dtype} {op}")
        hx = [to_np(x) for x in xs]
        L = dps.dp_shard_len(n, k)
        sh = [torch.empty(L, dtype=xs[0].dtype, device=DEV) for _ in range(k)]
        out = [torch.empty(n, dtype=xs[0].dtype, device=DEV) for _ in range(k)]
        dps.dp_reduce_scatter(xs, sh, op=op, s_chunks=s)
        dps.dp_all_gather(sh, out, s_chunks=s)
        out2 = [torch.empty(n, dtype=xs[0].dtype, device=DEV) for _ in range(k)]
        dps.dp_all_reduce(xs, out2, op=op, s_chunks=s)
        torch.cuda.synchronize()
        want_sh = oracle.reduce_scatter(hx, op=op)
        want = oracle.all_gather(want_sh, n)
        for c in range(k):
            assert bits_equal(to_np(sh[c]), want_sh[c])
            assert bits_equal(to_np(out[c]), want[c])
            assert bits_equal(to_np(out2[c]), want[c])
    # integer-valued fp32 sums are exact, so they equal the int32 sums
    a = [torch.empty(n, device=DEV) for _ in range(k)]
    b = [torch.empty(n, dtype=torch.int32, device=DEV) for _ in range(k)]
    dps.dp_all_reduce([x.to(torch.float32) for x in xi], a, op="sum")
    dps.dp_all_reduce(xi, b, op="sum")
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1].to(torch.float32))


def test_layer_buckets_k8_bf16_full_size():
    """K=8 ranks, one GQA+SwiGLU layer of bf16 gradients (218,103,808 per rank,
    N(0, 1e-3)), 9 buckets of at most 25,000,000, averaged ReduceScatter then
    AllGather, in the bucketed launch configuration and the rank layout the
    benchmark times (the pipelined step; ranks in one allocation, a fixed gap
    apart). Compared bit-exactly with the oracle for every element; the plain
    step must give the same bits."""
    k, total = 8, gen.LAYER_PARAMS
    say("layer-buckets: generating inputs")
    grads = rank_buffers(k, total, torch.bfloat16, device=DEV)
    for g, src in zip(grads, gen.layer_grads_bf16(3, k, device=DEV)):
        g.copy_(src)
    out = rank_buffers(k, total, torch.bfloat16, device=DEV)
    sync = BucketedSync(grads, out, gen.BUCKET_ELEMS, op="avg")
    say("layer-buckets: pipelined step")
    sync.step_pipelined()
    torch.cuda.synchronize()
    host = [to_np(g) for g in grads]
    say("layer-buckets: oracle")
    for b, (off, n) in enumerate(sync.plan):
        xs = [np.ascontiguousarray(h[off:off + n]) for h in host]
        want = oracle.reduce_scatter(xs, op="avg", nthreads=16)
        for c in range(k):
            assert bits_equal(to_np(sync.shard_view(b, c)), want[c]), (b, c)
        full = oracle.all_gather(want, n)
        for r in (0, 3, 7):
            assert bits_equal(to_np(out[r][off:off + n]), full[r]), (b, r)
    for r in range(1, k):
        assert torch.equal(out[0], out[r])
    say("layer-buckets: plain step")
    piped = out[0].clone()
    for o in out:
        o.fill_(float("nan"))
    sync.step()
    for r in range(k):
        assert torch.equal(out[r].view(torch.int16), piped.view(torch.int16)), r


def test_one_pass_layer_buckets_k8_bf16_full_size():
    """The same layer buckets as one one-pass AllReduce per bucket
    (BucketedSync.step_all_reduce, the launch configuration the one-pass
    benchmark times, ranks in its gapped layout): every element of every
    rank's output equals the oracle's AllGather of its ReduceScatter, bit for
    bit."""
    k, total = 8, gen.LAYER_PARAMS
    say("one-pass layer: generating inputs")
    grads = rank_buffers(k, total, torch.bfloat16, device=DEV)
    for g, src in zip(grads, gen.layer_grads_bf16(3, k, device=DEV)):
        g.copy_(src)
    out = rank_buffers(k, total, torch.bfloat16, device=DEV)
    for o in out:
        o.fill_(float("nan"))
    sync = BucketedSync(grads, out, gen.BUCKET_ELEMS, op="avg")
    say("one-pass layer: step")
    sync.step_all_reduce()
    torch.cuda.synchronize()
    for r in range(1, k):
        assert torch.equal(out[0], out[r]), r
    host = [to_np(g) for g in grads]
    got = to_np(out[0])
    say("one-pass layer: oracle")
    for b, (off, n) in enumerate(sync.plan):
        xs = [np.ascontiguousarray(h[off:off + n]) for h in host]
        want = oracle.all_reduce(xs, op="avg", nthreads=16)
        assert bits_equal(got[off:off + n], want[0]), b


def test_uneven_token_weighted_k8_10m():
    """K=8 ranks, N=10,000,019 fp32 (not divisible by 8: shards of 1,250,003,
    5 pads), token counts from sums of log-normal(7,1) document lengths,
    out = sum_r t_r g_r / sum_r t_r. Bit-exact for every element."""
    k, n = 8, 10_000_019
    xs = gen.ring_uniform_inputs(4, k, n, device=DEV)
    toks = gen.token_counts(4, k)
    say(f"weighted-10m tokens={toks}")
    out = [torch.empty(n, device=DEV) for _ in range(k)]
    dps.dp_weighted_reduce(xs, out, toks)
    torch.cuda.synchronize()
    hx = [to_np(x) for x in xs]
    want = oracle.weighted_all_reduce(hx, toks, nthreads=16)
    for r in range(k):
        assert bits_equal(to_np(out[r]), want[r])
    # the separate calls at this size take the shard-phase-mismatch path
    L = dps.dp_shard_len(n, k)
    sh = [torch.empty(L, device=DEV) for _ in range(k)]
    dps.dp_reduce_scatter(xs, sh, op="avg")
    dps.dp_all_gather(sh, out)
    torch.cuda.synchronize()
    want_sh = oracle.reduce_scatter(hx, op="avg", nthreads=16)
    for c in range(k):
        assert bits_equal(to_np(sh[c]), want_sh[c])
    want_full = oracle.all_gather(want_sh, n, nthreads=16)
    for r in (0, 7):
        assert bits_equal(to_np(out[r]), want_full[r])


def test_one_gib_per_rank_k8_fp32_sampled():
    """K=8 ranks of 268,435,456 fp32 (1 GiB each): ReduceScatter + AllGather.
    Checked at sampled positions (every shard boundary, the ends, and random
    indices) against the oracle's fold of the same input values, plus the
    property that all K outputs are equal."""
    k, n = 8, 268_435_456
    say("1gib: generating inputs")
    xs = gen.ring_uniform_inputs(5, k, n, device=DEV)
    L = dps.dp_shard_len(n, k)
    sh = [torch.empty(L, device=DEV) for _ in range(k)]
    out = [torch.empty(n, device=DEV) for _ in range(k)]
    say("1gib: rs+ag")
    dps.dp_reduce_scatter(xs, sh, op="sum")
    dps.dp_all_gather(sh, out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    idx = np.unique(np.concatenate([
        rng.integers(0, n, 200_000), np.arange(k) * L, np.arange(1, k + 1) * L - 1,
        np.arange(16), n - 1 - np.arange(16)]).astype(np.int64))
    ti = torch.from_numpy(idx).to(DEV)
    comp = [to_np(x[ti]) for x in xs]
    want = oracle.fold_at(comp, idx // L, op="sum")
    # shards at the sampled positions
    shard_vals = np.empty(idx.size, np.float32)
    for c in range(k):
        m = (idx // L) == c
        shard_vals[m] = to_np(sh[c][torch.from_numpy(idx[m] - c * L).to(DEV)])
    assert bits_equal(shard_vals, want)
    for r in range(k):
        assert bits_equal(to_np(out[r][ti]), want)
    for r in range(1, k):
        assert torch.equal(out[0], out[r])


def _uniform_chunked(seed, r, n, dtype, chunk=1 << 27):
    """gen.uniform_pm1 of n elements written chunk by chunk into one buffer."""
    t = torch.empty(n, dtype=dtype, device=DEV)
    for s0 in range(0, n, chunk):
        c = min(chunk, n - s0)
        t[s0:s0 + c] = gen.uniform_pm1(seed, 0, r, c, start=s0, device=DEV).to(dtype)
    return t


@pytest.mark.parametrize("dtype,n", [(torch.bfloat16, (1 << 31) + 7), (torch.float32, (1 << 30) + 5)])
def test_beyond_2g_elements_and_4gib_per_rank_sampled(dtype, n):
    """K=2 ranks with more than 2^31 elements (bf16) or more than 4 GiB
    (fp32) per buffer: ReduceScatter + AllGather, the one-pass AllReduce and
    the fused ReduceScatter+AllGather launch,
    checked at every shard boundary, around the 2^31-element and 4 GiB marks,
    at the ends and at random positions against the oracle's fold of the same
    values (the shard starts and the marks exercise 64-bit addressing)."""
    k = 2
    say(f"beyond-4g {dtype} n={n}: generating inputs")
    xs = [_uniform_chunked(9, r, n, dtype) for r in range(k)]
    L = dps.dp_shard_len(n, k)
    sh = [torch.empty(L, dtype=dtype, device=DEV) for _ in range(k)]
    out = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
    rng = np.random.default_rng(1)
    es = xs[0].element_size()
    marks = [(1 << 31) // es, (1 << 32) // es, 1 << 31, L, n]
    idx = np.concatenate([rng.integers(0, n, 100_000), np.arange(k) * L, np.arange(1, k + 1) * L - 1,
                          np.arange(16), n - 1 - np.arange(16)] +
                         [np.arange(m - 16, m + 16) for m in marks])
    idx = np.unique(idx[(idx >= 0) & (idx < n)].astype(np.int64))
    ti = torch.from_numpy(idx).to(DEV)
    comp = [to_np(x[ti]) for x in xs]
    want = oracle.fold_at(comp, idx // L, op="avg")
    say(f"beyond-4g {dtype}: rs+ag")
    dps.dp_reduce_scatter(xs, sh, op="avg")
    dps.dp_all_gather(sh, out)
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(out[r][ti]), want), r
    assert torch.equal(out[0], out[1])
    say(f"beyond-4g {dtype}: one-pass all-reduce")
    for o in out:
        o.fill_(float("nan"))
    dps.dp_all_reduce(xs, out, op="avg")
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(out[r][ti]), want), r
    assert torch.equal(out[0], out[1])
    say(f"beyond-4g {dtype}: fused launch (AllGather of the shards above beside a new ReduceScatter)")
    sh2 = [torch.empty(L, dtype=dtype, device=DEV) for _ in range(k)]
    for o in out:
        o.fill_(float("nan"))
    dps.dp_reduce_scatter_all_gather(xs, sh2, sh, out, op="avg")
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(out[r][ti]), want), r
    for c in range(k):
        assert torch.equal(sh2[c], sh[c]), c


def test_fp32_1gib_pipelined_buckets_full_size_sampled():
    """The pipelined bucket step in fp32 at 1 GiB per rank: K=8 ranks of
    268,435,456 fp32 (ranks in the gapped layout), 8 buckets of 33,554,432
    with the ReduceScatter of bucket b+1 fused with the AllGather of bucket b,
    summed. Each bucket is its own AllReduce, so the
    ring order of an element follows its shard within its bucket; checked
    against the oracle's fold at bucket and shard boundaries, the ends and
    random positions, and every rank's output equal."""
    k, n = 8, 268_435_456
    cap = n // 8
    say("fp32 1 GiB pipelined buckets: generating inputs")
    xs = rank_buffers(k, n, torch.float32, device=DEV)
    for x, src in zip(xs, gen.ring_uniform_inputs(5, k, n, device=DEV)):
        x.copy_(src)
    out = rank_buffers(k, n, torch.float32, device=DEV)
    for o in out:
        o.fill_(float("nan"))
    sync = BucketedSync(xs, out, cap, op="sum")
    sync.step_pipelined()
    torch.cuda.synchronize()
    Lb = dps.dp_shard_len(cap, k)
    rng = np.random.default_rng(3)
    edges = np.concatenate([b * cap + c * Lb + np.array([-1, 0, 1]) for b in range(8) for c in range(k)])
    idx = np.concatenate([rng.integers(0, n, 200_000), edges, np.arange(8), n - 1 - np.arange(8)])
    idx = np.unique(idx[(idx >= 0) & (idx < n)].astype(np.int64))
    ti = torch.from_numpy(idx).to(DEV)
    owner = (idx % cap) // Lb
    want = oracle.fold_at([to_np(x[ti]) for x in xs], owner, op="sum")
    for r in range(k):
        assert bits_equal(to_np(out[r][ti]), want), r
        assert torch.equal(out[r].view(torch.int32), out[0].view(torch.int32)), r


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_capped_grid_is_bit_identical(dtype):
    """With a cap on resident workgroups the kernels walk their tiles
    persistently; the results must not change."""
    for k, n, off in ((8, 8 * 4096 * 5 + 37, 0), (3, 100_003, 1), (8, 10_000_019 // 16, 3)):
        xs, hx = make_inputs(dtype, k, n, seed=40 + k, off=off)
        op = "sum" if dtype == torch.int32 else "avg"
        want_sh = oracle.reduce_scatter(hx, op=op)
        want = oracle.all_gather(want_sh, n)
        L = dps.dp_shard_len(n, k)
        for cap in (1, 3, 64, 256):
            say(f"capped k={k} n={n} {dtype} cap={cap}")
            sh = [Guarded(L, dtype) for _ in range(k)]
            out = [Guarded(n, dtype, 1) for _ in range(k)]
            out2 = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
            dps.dp_reduce_scatter_ex([g.t for g in xs], [s.t for s in sh], op=op, s_chunks=2,
                                     max_workgroups=cap)
            dps.dp_all_gather_ex([s.t for s in sh], [o.t for o in out], n=n, max_workgroups=cap)
            dps.dp_all_reduce_ex([g.t for g in xs], out2, op=op, max_workgroups=cap)
            torch.cuda.synchronize()
            for c in range(k):
                assert bits_equal(to_np(sh[c].t), want_sh[c]), (cap, c)
                assert sh[c].intact() and out[c].intact()
            for r in (0, k - 1):
                assert bits_equal(to_np(out[r].t), want[r]), (cap, r)
                assert bits_equal(to_np(out2[r]), want[r]), (cap, r)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
@pytest.mark.parametrize("k,n,in_off,out_off", [(8, 8 * 4096 * 3 + 11, 0, 0), (8, 100_003, 1, 3),
                                                (5, 7777, 0, 2), (1, 64, 0, 0), (16, 50_001, 2, 2),
                                                (8, 3, 0, 0)])
def test_one_pass_all_reduce_equals_two_phase(dtype, k, n, in_off, out_off):
    """The one-pass AllReduce (default) and the ReduceScatter + AllGather pair
    give the oracle's bits, out of place (any alignment) and in place."""
    xs, hx = make_inputs(dtype, k, n, seed=60 + n % 97, off=in_off)
    op = "sum" if dtype == torch.int32 else "avg"
    want = oracle.all_reduce(hx, op=op)
    for two_phase in (False, True):
        for cap in (0, 5):
            say(f"ar k={k} n={n} {dtype} two_phase={two_phase} cap={cap}")
            outs = [Guarded(n, dtype, out_off) for _ in range(k)]
            dps.dp_all_reduce_ex([g.t for g in xs], [o.t for o in outs], op=op, s_chunks=3,
                                 max_workgroups=cap, two_phase=two_phase)
            torch.cuda.synchronize()
            for r in range(k):
                assert bits_equal(to_np(outs[r].t), want[r]), (two_phase, cap, r)
                assert outs[r].intact()
    # in place, one pass
    dps.dp_all_reduce([g.t for g in xs], [g.t for g in xs], op=op)
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(xs[r].t), want[r])
        assert xs[r].intact()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_weighted_one_pass_equals_two_phase(dtype):
    k, n = 8, 1_000_003
    xs, hx = make_inputs(dtype, k, n, seed=61)
    toks = gen.token_counts(7, k)
    want = oracle.weighted_all_reduce(hx, toks, nthreads=8)
    for two_phase in (False, True):
        out = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
        dps.dp_weighted_reduce_ex([g.t for g in xs], out, toks, two_phase=two_phase)
        torch.cuda.synchronize()
        for r in (0, 3, k - 1):
            assert bits_equal(to_np(out[r]), want[r]), two_phase


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_lean_variant_is_bit_identical(dtype):
    """The 64-VGPR kernel variant (one vector per lane per rank) against the
    oracle: ReduceScatter, one-pass and two-phase AllReduce, weighted, with and
    without a grid cap, over aligned, misaligned, multi-tile and ragged sizes."""
    for k, n, off in ((8, 8 * 2048 * 5 + 37, 0), (3, 100_003, 1), (8, 1_250_003, 3), (5, 17, 0),
                      (16, 4096 * 16 + 5, 2)):
        xs, hx = make_inputs(dtype, k, n, seed=70 + k, off=off)
        op = "sum" if dtype == torch.int32 else "avg"
        want_sh = oracle.reduce_scatter(hx, op=op)
        want = oracle.all_gather(want_sh, n)
        L = dps.dp_shard_len(n, k)
        for cap in (0, 7, 256):
            say(f"lean k={k} n={n} {dtype} cap={cap}")
            sh = [Guarded(L, dtype) for _ in range(k)]
            out = [Guarded(n, dtype, 1) for _ in range(k)]
            out2 = [Guarded(n, dtype) for _ in range(k)]
            dps.dp_reduce_scatter_ex([g.t for g in xs], [s.t for s in sh], op=op, s_chunks=2,
                                     max_workgroups=cap, lean=True)
            dps.dp_all_reduce_ex([g.t for g in xs], [o.t for o in out], op=op,
                                 max_workgroups=cap, lean=True)
            dps.dp_all_reduce_ex([g.t for g in xs], [o.t for o in out2], op=op,
                                 max_workgroups=cap, lean=True, two_phase=True)
            torch.cuda.synchronize()
            for c in range(k):
                assert bits_equal(to_np(sh[c].t), want_sh[c]), (cap, c)
                assert sh[c].intact()
            for r in range(k):
                assert bits_equal(to_np(out[r].t), want[r]), (cap, r)
                assert bits_equal(to_np(out2[r].t), want[r]), (cap, r)
                assert out[r].intact() and out2[r].intact()
            if dtype != torch.int32:
                toks = gen.token_counts(70 + k, k)
                wo = [torch.empty(n, dtype=dtype, device=DEV) for _ in range(k)]
                dps.dp_weighted_reduce_ex([g.t for g in xs], wo, toks, max_workgroups=cap,
                                          lean=True)
                torch.cuda.synchronize()
                ww = oracle.weighted_all_reduce(hx, toks)
                for r in (0, k - 1):
                    assert bits_equal(to_np(wo[r]), ww[r]), (cap, r)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_fused_rs_ag_equals_separate(dtype):
    """One launch doing a ReduceScatter of one set and an AllGather of another:
    both results bit-exact against the oracle, for equal and unequal sizes
    (so one kind of tile runs out first), misaligned buffers, in-place forms and
    an empty side."""
    op = "sum" if dtype == torch.int32 else "avg"
    for k, n_rs, n_ag, off, in_place in ((8, 25_000 * 8 + 3, 25_000 * 8 + 3, 0, False),
                                         (8, 8 * 2048 * 3 + 5, 8 * 2048 * 9 + 1, 1, False),
                                         (3, 100_003, 7, 2, False), (5, 17, 40_000, 0, False),
                                         (8, 8 * 4096 * 4, 8 * 4096 * 4, 0, True),
                                         (4, 0, 9_999, 0, False), (4, 9_999, 0, 3, False)):
        say(f"fused rs+ag k={k} n_rs={n_rs} n_ag={n_ag} off={off} in_place={in_place} {dtype}")
        xs, hx = make_inputs(dtype, k, n_rs, seed=300 + k, off=off)
        L_rs, L_ag = dps.dp_shard_len(n_rs, k), dps.dp_shard_len(n_ag, k)
        gs, hg = make_inputs(dtype, k, n_ag, seed=400 + k)      # gather sources: values per rank
        shards = [Guarded(max(L_ag, 1), dtype, off) for _ in range(k)]
        want_ag_sh = [h[c * L_ag:(c + 1) * L_ag] for c, h in enumerate(hg)] if n_ag else []
        for c in range(k):
            if n_ag:
                v = np.zeros(L_ag, dtype=hg[0].dtype)
                v[:len(want_ag_sh[c])] = want_ag_sh[c]
                shards[c].t[:L_ag].copy_(from_np(v)[:L_ag])
        ag_out = [Guarded(max(n_ag, 1), dtype) for _ in range(k)]
        if in_place:
            rs_out = [xs[c].t[c * L_rs:(c + 1) * L_rs] for c in range(k)]
            ag_out = [Guarded(n_ag, dtype) for _ in range(k)]
            for c in range(k):
                ag_out[c].t[c * L_ag:(c + 1) * L_ag].copy_(shards[c].t[:L_ag])
            ag_src = [ag_out[c].t[c * L_ag:(c + 1) * L_ag] for c in range(k)]
        else:
            rs_out = [Guarded(max(L_rs, 1), dtype).t[:L_rs] for _ in range(k)]
            ag_src = [s.t[:L_ag] for s in shards]
        want_rs = oracle.reduce_scatter(hx, op=op) if n_rs else []
        want_ag = oracle.all_gather([np.ascontiguousarray(to_np(s)) for s in ag_src], n_ag) if n_ag else []
        dps.dp_reduce_scatter_all_gather([g.t for g in xs], rs_out, ag_src,
                                         [o.t[:n_ag] for o in ag_out], op=op, rs_n=n_rs, ag_n=n_ag)
        torch.cuda.synchronize()
        for c in range(k):
            if n_rs:
                assert bits_equal(to_np(rs_out[c]), want_rs[c]), (k, n_rs, c)
            if n_ag:
                assert bits_equal(to_np(ag_out[c].t[:n_ag]), want_ag[c]), (k, n_ag, c)
            assert ag_out[c].intact()
            if not in_place:
                assert xs[c].intact()


def test_pipelined_layer_step_k8_bf16_full_size():
    """The bucket pipeline (ReduceScatter of bucket b+1 fused with the
    AllGather of bucket b) over the full layer equals the oracle bucket by
    bucket, every element, and equals the plain step."""
    k = 8
    say("pipelined layer step k=8 bf16")
    grads = gen.layer_grads_bf16(3, k, device=DEV)
    out = [torch.full((gen.LAYER_PARAMS,), float("nan"), dtype=torch.bfloat16, device=DEV)
           for _ in range(k)]
    sync = BucketedSync(grads, out, gen.BUCKET_ELEMS, op="avg")
    sync.step_pipelined()
    torch.cuda.synchronize()
    got = [to_np(o) for o in out]
    hg = [to_np(g) for g in grads]
    for b, (off, n) in enumerate(sync.plan):
        want_sh = oracle.reduce_scatter([h[off:off + n] for h in hg], op="avg", nthreads=16)
        for c in range(k):
            assert bits_equal(to_np(sync.shard_view(b, c)), want_sh[c]), (b, c)
        want = oracle.all_gather(want_sh, n, nthreads=16)
        for r in (0, 3, k - 1):
            assert bits_equal(got[r][off:off + n], want[r]), (b, r)
    out2 = [torch.empty_like(o) for o in out]
    sync2 = BucketedSync(grads, out2, gen.BUCKET_ELEMS, op="avg")
    sync2.step()
    torch.cuda.synchronize()
    for r in range(k):
        assert bits_equal(to_np(out2[r]), got[r])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.int32])
def test_ag_misaligned_shards_multi_tile(dtype):
    """Shards whose 16-byte phase differs from the outputs' (the shifted-load
    path: dword loads, for 2-byte elements joined with a 2-byte shift), over
    several tiles per shard, a ragged last shard, shards starting at the
    buffer's first element and ending at its last valid one; and outputs whose
    phases differ from each other (element-wise path)."""
    for k, n in ((8, 8 * 4096 * 3 + 5), (3, 100_003), (8, 10_000_019 // 64)):
        L = dps.dp_shard_len(n, k)
        for sh_off, out_offs in ((1, [0] * k), (3, [0] * k), (2, [0] * k), (0, [1] * k),
                                 (5, [3] * k), (1, [r % 3 for r in range(k)])):
            say(f"ag-misaligned k={k} n={n} {dtype} sh_off={sh_off} out_offs={out_offs[:3]}")
            shards = []
            for c in range(k):
                nc = max(0, min(L, n - c * L))
                g = Guarded(nc, dtype, sh_off)          # exactly the valid elements
                v = gen.raw_u64(12, 2, c, 0, nc).to(torch.int32)
                g.t.copy_((v if dtype == torch.int32 else
                           (v.to(torch.float32) * 2.0 ** -31).to(dtype)).to(DEV))
                shards.append(g)
            outs = [Guarded(n, dtype, out_offs[r]) for r in range(k)]
            want = oracle.all_gather([to_np(g.t) for g in shards], n, L=L)
            dps.dp_all_gather([g.t for g in shards], [o.t for o in outs], n=n)
            torch.cuda.synchronize()
            for r in range(k):
                assert bits_equal(to_np(outs[r].t), want[r]), (k, n, sh_off, r)
                assert outs[r].intact()
