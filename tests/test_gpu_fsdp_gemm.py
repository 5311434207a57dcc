"""GPU parity of the FSDP layer step and of the bf16 GEMM, through the C ABI.

The gathered weights are exact copies and must match bit for bit. The GEMMs
run on MFMA with an accumulation order of their own, so each entry is checked
against the oracle's fp64 value within the recursive-summation bound
gamma_n * sum |a||b| (Higham, Accuracy and Stability of Numerical Algorithms,
eq. 3.5); with small-integer inputs every step is exact and the comparison is
bit-exact.
"""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
import oracle
from tests.helpers import bits_equal, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
U32 = 2.0 ** -24
U_BF16 = 2.0 ** -8


def gamma(n, u=U32):
    return n * u / (1 - n * u)


def shard_rows(w, k):
    d, f = w.shape
    R = -(-d // k)
    out = []
    for c in range(k):
        s = torch.zeros(R, f, dtype=w.dtype)
        rows = w[c * R:(c + 1) * R]
        s[:rows.shape[0]] = rows
        out.append(s)
    return out


def run_fsdp(x, w, dy, k, backward=True, with_dx=False):
    m, d = x.shape
    f = w.shape[1]
    ml = m // k
    R = -(-d // k)
    xl = [x[r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    dyl = [dy[r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    ws = [s.to(DEV) for s in shard_rows(w, k)]
    wf = [torch.full((d, f), float("nan"), device=DEV) for _ in range(k)]
    y = [torch.full((ml, f), float("nan"), device=DEV) for _ in range(k)]
    dwf = [torch.full((d, f), float("nan"), device=DEV) for _ in range(k)]
    dws = [torch.full((R, f), float("nan"), device=DEV) for _ in range(k)]
    dx = [torch.full((ml, d), float("nan"), device=DEV) for _ in range(k)] if with_dx else None
    dps.dp_fsdp_layer(xl, ws, dyl if backward else None, wf, y,
                      dwf if backward else None, dws if backward else None, dx_local=dx)
    torch.cuda.synchronize()
    host = dict(xl=[to_np(t) for t in xl], ws=[to_np(t) for t in ws],
                dyl=[to_np(t) for t in dyl])
    return dict(wf=[to_np(t) for t in wf], y=[to_np(t) for t in y], dwf=[to_np(t) for t in dwf],
                dws=[to_np(t) for t in dws], dx=[to_np(t) for t in dx] if with_dx else None), host


def check_fsdp(x, w, dy, k, exact=False, with_dx=False):
    m, d = x.shape
    f = w.shape[1]
    ml = m // k
    R = -(-d // k)
    got, host = run_fsdp(x, w, dy, k, with_dx=with_dx)
    want = oracle.fsdp_layer(host["xl"], host["ws"], host["dyl"], d=d, nthreads=8)
    wn, xn, dyn = w.numpy(), x.numpy(), dy.numpy()
    for r in range(k):
        assert bits_equal(got["wf"][r], want["w_full"][r])
        yr = want["y"][r]
        if exact:
            assert bits_equal(got["y"][r], yr.astype(np.float32))
        else:
            _, ab = oracle.gemm_f64(host["xl"][r], wn)
            err = np.abs(got["y"][r].astype(np.float64) - yr)
            assert np.all(err <= gamma(d + 2) * ab), float((err / (ab + 1e-300)).max())
    _, ab_dw = oracle.gemm_f64(xn, dyn, trans_a=True)      # sum over all ranks' rows
    for c in range(k):
        rows = min(R, max(0, d - c * R))
        ws_ = want["dw_shard"][c]
        g = got["dws"][c]
        assert not g[rows:].any(), "pad rows must be zero"
        if exact:
            assert bits_equal(g[:rows], ws_[:rows].astype(np.float32))
        else:
            ab = ab_dw[c * R:c * R + rows]
            err = np.abs(g[:rows].astype(np.float64) - ws_[:rows])
            assert np.all(err <= gamma(ml + k + 2) * ab)
    # dw_full: each rank's x_r^T dy_r within the summation bound, and dw_shard is
    # exactly the ring-order ReduceScatter of the dw_full the GPU wrote (the
    # fused backward kernel folds its blocks from LDS; the other path runs the
    # ReduceScatter kernel on dw_full)
    for r in range(k):
        ref, ab = oracle.gemm_f64(host["xl"][r], host["dyl"][r], trans_a=True)
        if exact:
            assert bits_equal(got["dwf"][r], ref.astype(np.float32))
        else:
            err = np.abs(got["dwf"][r].astype(np.float64) - ref)
            assert np.all(err <= gamma(ml + 2) * ab)
    rs = oracle.reduce_scatter([g.ravel() for g in got["dwf"]], op="sum", L=R * f)
    for c in range(k):
        assert bits_equal(got["dws"][c].ravel(), rs[c])
    # dx_r = dy_r W^T (the gathered W, from the oracle), within the summation bound
    if with_dx:
        wt = np.ascontiguousarray(want["w_full"][0].T)
        for r in range(k):
            ref, ab = oracle.gemm_f64(host["dyl"][r], wt)
            if exact:
                assert bits_equal(got["dx"][r], ref.astype(np.float32))
            else:
                err = np.abs(got["dx"][r].astype(np.float64) - ref)
                assert np.all(err <= gamma(f + 2) * ab), float((err / (ab + 1e-300)).max())
    # global view: concatenated y is x @ w (normwise)
    ycat = np.concatenate(got["y"]).astype(np.float64)
    ref = xn.astype(np.float64) @ wn.astype(np.float64)
    rel = np.linalg.norm(ycat - ref) / np.linalg.norm(ref)
    assert rel < 1e-6, rel
    return rel


def test_fsdp_fixture_k8():
    """x[1024,512] ~ N(0,1), w[512,512] ~ N(0,0.02^2) row-sharded over 8 ranks to
    x_local[128,512] and w[64,512]; dy[1024,512] ~ N(0,1)."""
    say("fsdp fixture k=8")
    fx = gen.fsdp_fixture(seed=2, k=8)
    check_fsdp(fx["x"], fx["w"], fx["dy"], 8)
    say("fsdp fixture k=8 with dx")
    check_fsdp(fx["x"], fx["w"], fx["dy"], 8, with_dx=True)


def test_fsdp_integer_values_exact():
    say("fsdp integer fixture")
    g = torch.Generator().manual_seed(0)
    x = torch.randint(-4, 5, (1024, 512), generator=g).float()
    w = torch.randint(-4, 5, (512, 512), generator=g).float()
    dy = torch.randint(-4, 5, (1024, 512), generator=g).float()
    check_fsdp(x, w, dy, 8, exact=True)
    check_fsdp(x, w, dy, 8, exact=True, with_dx=True)


@pytest.mark.parametrize("k,m,d,f", [(3, 111, 45, 29), (8, 64, 100, 70), (1, 5, 3, 2),
                                     (5, 5 * 33, 64, 130), (2, 256, 96, 64),
                                     (4, 4 * 64, 256, 96), (7, 7 * 32, 7 * 32, 64),
                                     (8, 8 * 32, 512, 32), (2, 256, 128, 128),
                                     (4, 4 * 64, 256, 64), (8, 8 * 64, 256, 128),
                                     (1, 64, 256, 64), (2, 64, 512, 96), (4, 128, 256, 32)])
def test_fsdp_ragged_shapes(k, m, d, f):
    """The shapes span every path of the call: the first five take the
    separate launches (AllGather, GEMM, GEMM, ReduceScatter); the others the
    fused backward kernel (whole 32x32 blocks, shards of a multiple of 32 rows,
    m_local a multiple of 32) with K = 4, 7 and 8, the fused forward (whole 64x64
    tiles: the AllGather folded into the GEMM's operand loads), and the whole
    step in one launch: with dx where m_local is a multiple of 64, without dx
    as the one-wave step where f is a multiple of 64 and d of 128 (at most
    512), else with 32x32 forward blocks."""
    say(f"fsdp ragged k={k} m={m} d={d} f={f}")
    g = torch.Generator().manual_seed(k * m + d)
    x = torch.randn(m, d, generator=g)
    w = torch.randn(d, f, generator=g) * 0.02
    dy = torch.randn(m, f, generator=g)
    check_fsdp(x, w, dy, k)
    check_fsdp(x, w, dy, k, with_dx=True)
    xi = torch.randint(-3, 4, (m, d), generator=g).float()
    wi = torch.randint(-3, 4, (d, f), generator=g).float()
    dyi = torch.randint(-3, 4, (m, f), generator=g).float()
    check_fsdp(xi, wi, dyi, k, exact=True, with_dx=True)


@pytest.mark.parametrize("k,m,d,f", [(1, 32, 128, 64), (2, 2 * 96, 384, 192), (4, 4 * 32, 512, 128),
                                     (8, 8 * 64, 256, 320), (6, 6 * 32, 384, 64),
                                     (8, 1024, 512, 512)])
def test_fsdp_one_wave_step(k, m, d, f):
    """The step without dx as one wave of workgroups (each wave a forward and a
    backward chain): forward tile and backward position counts equal (with the
    XCD-major tile order: (8, 512, 256, 320) and the fixture's shape) or not
    (the other workgroups then run one part only)."""
    say(f"fsdp one-wave step k={k} m={m} d={d} f={f}")
    g = torch.Generator().manual_seed(k * m + d + f)
    x = torch.randn(m, d, generator=g)
    w = torch.randn(d, f, generator=g) * 0.02
    dy = torch.randn(m, f, generator=g)
    check_fsdp(x, w, dy, k)
    xi = torch.randint(-3, 4, (m, d), generator=g).float()
    wi = torch.randint(-3, 4, (d, f), generator=g).float()
    dyi = torch.randint(-3, 4, (m, f), generator=g).float()
    check_fsdp(xi, wi, dyi, k, exact=True)


def _fsdp_outputs_at(off, k, ml, d, f, R):
    """Output tensors whose first element is off floats past a 256-byte boundary."""
    def mk(*shape):
        n = int(np.prod(shape))
        return torch.full((n + off,), float("nan"), device=DEV)[off:].view(*shape)
    return dict(wf=[mk(d, f) for _ in range(k)], y=[mk(ml, f) for _ in range(k)],
                dwf=[mk(d, f) for _ in range(k)], dws=[mk(R, f) for _ in range(k)])


def test_fsdp_step_outputs_not_16_byte_aligned():
    """The fixture's step (K = 8, 128 tokens, d = f = 512) runs the kernel with
    every size fixed at compile time (16-byte output stores) when the W shards
    and all outputs are 16-byte aligned, else the runtime-shaped step kernel:
    the same bits either way, and both within the bounds."""
    say("fsdp step, outputs aligned and 4 bytes off")
    k, m, d, f = 8, 1024, 512, 512
    fx = gen.fsdp_fixture(seed=5, k=k)
    ml, R = m // k, d // k
    xl = [fx["x"][r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    dyl = [fx["dy"][r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    ws = [s.to(DEV) for s in shard_rows(fx["w"], k)]
    outs = []
    for off in (0, 1):
        o = _fsdp_outputs_at(off, k, ml, d, f, R)
        dps.dp_fsdp_layer(xl, ws, dyl, o["wf"], o["y"], o["dwf"], o["dws"])
        torch.cuda.synchronize()
        outs.append({n: [to_np(t) for t in ts] for n, ts in o.items()})
    for n in ("wf", "y", "dwf", "dws"):
        for r in range(k):
            assert bits_equal(outs[0][n][r], outs[1][n][r]), (n, r)
    check_fsdp(fx["x"], fx["w"], fx["dy"], k)


def test_fsdp_step_with_dx_outputs_not_16_byte_aligned():
    """With dx at the fixture's sizes: all outputs 16-byte aligned run the
    compile-time-sized kernel with a dx chain per wave, dx 4 bytes off runs the
    runtime-shaped step kernel. W copies, dW and its shards have the same bits
    either way (the same backward chains); y and dx (other k orders) are each
    within the fp32 summation bound of the fp64 oracle."""
    say("fsdp step with dx, dx aligned and 4 bytes off")
    k, m, d, f = 8, 1024, 512, 512
    fx = gen.fsdp_fixture(seed=6, k=k)
    ml, R = m // k, d // k
    xl = [fx["x"][r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    dyl = [fx["dy"][r * ml:(r + 1) * ml].contiguous().to(DEV) for r in range(k)]
    ws = [s.to(DEV) for s in shard_rows(fx["w"], k)]
    outs = []
    for off in (0, 1):
        o = _fsdp_outputs_at(0, k, ml, d, f, R)
        dx = [torch.full((ml * d + off,), float("nan"), device=DEV)[off:].view(ml, d) for _ in range(k)]
        dps.dp_fsdp_layer(xl, ws, dyl, o["wf"], o["y"], o["dwf"], o["dws"], dx_local=dx)
        torch.cuda.synchronize()
        o["dx"] = dx
        outs.append({n: [to_np(t) for t in ts] for n, ts in o.items()})
    for n in ("wf", "dwf", "dws"):
        for r in range(k):
            assert bits_equal(outs[0][n][r], outs[1][n][r]), (n, r)
    host_xl = [to_np(t) for t in xl]
    host_dy = [to_np(t) for t in dyl]
    wn = fx["w"].numpy()
    wt = np.ascontiguousarray(wn.T)
    for got in outs:
        for r in range(k):
            ref, ab = oracle.gemm_f64(host_xl[r], wn)
            assert np.all(np.abs(got["y"][r].astype(np.float64) - ref) <= gamma(d + 2) * ab)
            ref, ab = oracle.gemm_f64(host_dy[r], wt)
            assert np.all(np.abs(got["dx"][r].astype(np.float64) - ref) <= gamma(f + 2) * ab)


def test_fsdp_forward_only():
    fx = gen.fsdp_fixture(seed=7, k=8, m=256, d=128, f=64)
    got, host = run_fsdp(fx["x"], fx["w"], fx["dy"], 8, backward=False)
    want = oracle.fsdp_layer(host["xl"], host["ws"], None, d=128)
    for r in range(8):
        assert bits_equal(got["wf"][r], want["w_full"][r])
        assert np.all(np.isnan(got["dws"][r]))      # untouched


# ------------------------------------------------------------------ bf16 GEMM

def _bits(t):
    return to_np(t)


def run_gemm(a, b, layout="kn", **opts):
    m = a.shape[0]
    n = b.shape[1] if layout == "kn" else b.shape[0]
    c = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    dps.dp_gemm_bf16_ex(a, b, c, b_layout=layout, **opts)
    torch.cuda.synchronize()
    return c


def check_gemm(a, b, layout="kn", rows=None, cols=None, exact=False, c=None):
    """The product against the oracle's fp64 value of the same bf16 operands,
    read in the same layout (no transposition on either side)."""
    m, kk = a.shape
    n = b.shape[1] if layout == "kn" else b.shape[0]
    if c is None:
        c = run_gemm(a, b, layout)
    if rows is None:
        rows, cols = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
        rows, cols = rows.ravel(), cols.ravel()
    ref, absr = oracle.gemm_bf16_at(_bits(a), _bits(b), rows, cols, nthreads=16, b_layout=layout)
    got = oracle.bf16_to_f32(_bits(c)[rows, cols]).astype(np.float64)
    if exact:
        assert np.array_equal(got, ref)
        return c
    g = gamma(kk + 1)
    bound = U_BF16 * (np.abs(ref) + g * absr) + g * absr
    err = np.abs(got - ref)
    assert np.all(err <= bound), float((err - bound).max())
    return c


def _small_int_inputs(m, n, kk, layout, seed, lo=-1, hi=2):
    g = torch.Generator().manual_seed(seed)
    ai = torch.randint(lo, hi, (m, kk), generator=g).to(torch.bfloat16).to(DEV)
    shape = (kk, n) if layout == "kn" else (n, kk)
    bi = torch.randint(lo, hi, shape, generator=g).to(torch.bfloat16).to(DEV)
    return ai, bi


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("m,n,kk", [(128, 128, 32), (256, 384, 64), (200, 136, 40), (1, 1, 8),
                                    (129, 255, 1000), (512, 512, 4096)])
def test_gemm_bf16_small(m, n, kk, layout):
    say(f"gemm bf16 {layout} {m}x{n}x{kk}")
    a, b = gen.gemm_bf16_inputs(8, m, n, kk, device=DEV, b_layout=layout)
    check_gemm(a, b, layout)
    if kk <= 256:
        check_gemm(*_small_int_inputs(m, n, kk, layout, m + n), layout, exact=True)


def test_gemm_bf16_8192_sampled():
    """C = A B with A, B bf16 [8192,8192] ~ N(0,1) (B stored [k,n]: the
    direct-to-LDS kernel with transposing LDS reads): sampled entries; then B
    stored [n,k] (the other direct-to-LDS kernel) gives the same bits."""
    m = n = kk = 8192
    say("gemm bf16 8192^3")
    a, b = gen.gemm_bf16_inputs(5, m, n, kk, device=DEV)
    rng = np.random.default_rng(1)
    rows = np.concatenate([rng.integers(0, m, 3000), [0, 0, m - 1, m - 1, 127, 128]])
    cols = np.concatenate([rng.integers(0, n, 3000), [0, n - 1, 0, n - 1, 128, 127]])
    c = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    dps.dp_gemm_bf16(a, b, c)
    torch.cuda.synchronize()
    check_gemm(a, b, "kn", rows.astype(np.int64), cols.astype(np.int64), c=c)
    b_nk = b.t().contiguous()
    del b
    c_nk = run_gemm(a, b_nk, "nk")
    assert torch.equal(c.view(torch.int16), c_nk.view(torch.int16))


@pytest.mark.parametrize("m,n,kk", [(256, 256, 2048), (512, 768, 2112), (1024, 256, 4096),
                                    (512, 512, 1024), (256, 768, 1472),
                                    (768, 512, 320), (2048, 2048, 64), (256, 256, 960),
                                    (264, 280, 1032), (512, 768, 256), (768, 256, 640),
                                    (256, 512, 128), (256, 512, 8192)])
def test_gemm_bf16_variants_and_layouts_bit_identical(m, n, kk):
    """Whole 256x256 tiles with an even number of depth-64 k stages and kk >=
    256 (B stored [kk,n]) or >= 384 (B stored [n,kk]) run the direct-to-LDS
    4-wave kernels (16x16x32 MFMAs for both, B's fragments assembled with
    transposing LDS reads for B stored [kk,n]); with an odd number and kk >=
    1024 the register-staged 4-wave kernel;
    the 8-wave variants (DP_LAUNCH_LEAN: depth-64 stages,
    DP_LAUNCH_SHARE_CU: depth-32) add the same k steps in the same order, for
    B stored [kk,n] (transposing LDS reads) and [n,kk] alike, so all six agree
    bit for bit (shorter or odd k ranges and edge tiles take the 8-wave kernel
    on every path). The default result is also checked against the oracle
    (exactly on small-integer inputs, within the fp32 summation bound on N(0,1)
    inputs); kk = 8192 (C in nontemporal stores), an odd number of k stages
    (2112 = 33 x 64) and grids that are not a
    multiple of 8 tiles are among the cases."""
    say(f"gemm bf16 variants {m}x{n}x{kk}")
    a, b_kn = gen.gemm_bf16_inputs(11, m, n, kk, device=DEV, b_layout="kn")
    b_nk = b_kn.t().contiguous()
    outs = []
    for layout, b in (("kn", b_kn), ("nk", b_nk)):
        for opts in ({}, {"lean": True}, {"share_cu": True}):
            outs.append(_bits(run_gemm(a, b, layout, **opts)))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)
    rng = np.random.default_rng(kk)
    rows = np.concatenate([rng.integers(0, m, 1500), [0, m - 1, 255, 256 % m]]).astype(np.int64)
    cols = np.concatenate([rng.integers(0, n, 1500), [n - 1, 0, 256 % n, 255]]).astype(np.int64)
    check_gemm(a, b_kn, "kn", rows, cols)
    # small integers: every fp32 partial sum is exact (|sum| <= 4 kk < 2^24), so
    # the result is the exact sum rounded once to bf16
    ai, bi = _small_int_inputs(m, n, kk, "kn", m + kk, -2, 3)
    c = run_gemm(ai, bi, "kn")
    ref, _ = oracle.gemm_bf16_at(_bits(ai), _bits(bi), rows, cols, nthreads=16)
    assert np.array_equal(_bits(c)[rows, cols], oracle.bf16_from_f32(ref.astype(np.float32)))


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("m,n,kk", [(256, 256, 32), (200, 136, 40), (512, 768, 1024),
                                    (8192, 8192, 8192)])
def test_gemm_bf16_share_cu_variant(m, n, kk, layout):
    """The depth-32 variant (DP_LAUNCH_SHARE_CU) against the oracle, including
    shapes with edge tiles."""
    say(f"gemm bf16 share-cu {layout} {m}x{n}x{kk}")
    a, b = gen.gemm_bf16_inputs(9, m, n, kk, device=DEV, b_layout=layout)
    c = run_gemm(a, b, layout, share_cu=True)
    rng = np.random.default_rng(m + kk)
    rows = np.concatenate([rng.integers(0, m, 2000), [0, m - 1]]).astype(np.int64)
    cols = np.concatenate([rng.integers(0, n, 2000), [n - 1, 0]]).astype(np.int64)
    check_gemm(a, b, layout, rows, cols, c=c)


def _offset_copy(t, off):
    """t's values in a fresh buffer starting `off` elements into its allocation."""
    full = torch.empty(t.numel() + off, dtype=t.dtype, device=DEV)
    v = full[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("off", [1, 3, 4, 8])
@pytest.mark.parametrize("opts", [{}, {"lean": True}, {"share_cu": True}], ids=["w4", "lean", "share_cu"])
def test_gemm_bf16_output_at_any_element_offset(layout, off, opts):
    """The 4-wave direct-to-LDS kernels (both layouts, an even number of k
    stages) and the 8-wave variants with aligned operands and C at an element
    offset that is not 16-byte aligned (2-byte stores; 4 elements: 8-byte
    aligned) or is (8 elements: 16-byte stores): the same bits as C at the
    start of its allocation, and the elements around C untouched."""
    m = n = 512
    kk = 1024
    say(f"gemm bf16 output offset {layout} off={off} {opts}")
    a, b = gen.gemm_bf16_inputs(13, m, n, kk, device=DEV, b_layout=layout)
    want = run_gemm(a, b, layout)
    c_full = torch.empty((m * n + off + 8,), dtype=torch.bfloat16, device=DEV)
    c_full.view(torch.int16).fill_(0x5A5A)
    c = c_full[off:off + m * n].view(m, n)
    dps.dp_gemm_bf16_ex(a, b, c, b_layout=layout, **opts)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(c), _bits(want))
    guard = np.concatenate([to_np(c_full[:off]), to_np(c_full[off + m * n:])])
    assert np.all(guard == 0x5A5A)


@pytest.mark.parametrize("layout", ["kn", "nk"])
@pytest.mark.parametrize("m,n,kk,off", [(64, 64, 13, 0), (97, 45, 1003, 0), (256, 256, 1024, 1),
                                        (33, 300, 77, 3), (1, 5, 1, 1), (130, 7, 200, 0)])
def test_gemm_bf16_any_shape_and_alignment(m, n, kk, off, layout):
    """Rows that are not 16-byte aligned (kk or n not a multiple of 8, or
    operands at an odd element offset) take the element-gathering kernel: it
    matches the oracle (exactly on small integers), and where the same values
    also fit the staged kernels (copied to aligned buffers, kk padded with
    zeros to a multiple of 8) both give the same bits."""
    say(f"gemm bf16 any {layout} {m}x{n}x{kk} off={off}")
    a, b = gen.gemm_bf16_inputs(12, m, n, kk, device=DEV, b_layout=layout)
    a_o, b_o = _offset_copy(a, off), _offset_copy(b, off)
    c_full = torch.empty((m * n + off + 8,), dtype=torch.bfloat16, device=DEV)
    c_full.view(torch.int16).fill_(0x5A5A)                 # canary around the output
    c = c_full[off:off + m * n].view(m, n)
    dps.dp_gemm_bf16_ex(a_o, b_o, c, b_layout=layout)
    torch.cuda.synchronize()
    check_gemm(a, b, layout, c=c)
    guard = np.concatenate([to_np(c_full[:off]), to_np(c_full[off + m * n:])])
    assert np.all(guard == 0x5A5A)
    # the staged kernels on zero-padded, aligned copies of the same values
    k8 = -(-kk // 8) * 8
    n8 = -(-n // 8) * 8 if layout == "kn" else n
    ap = torch.zeros(m, k8, dtype=torch.bfloat16, device=DEV)
    ap[:, :kk] = a
    if layout == "kn":
        bp = torch.zeros(k8, n8, dtype=torch.bfloat16, device=DEV)
        bp[:kk, :n] = b
    else:
        bp = torch.zeros(n, k8, dtype=torch.bfloat16, device=DEV)
        bp[:, :kk] = b
    cp = run_gemm(ap, bp, layout)
    assert np.array_equal(_bits(cp)[:, :n], _bits(c))
    if kk <= 256:
        ai, bi = _small_int_inputs(m, n, kk, layout, 7 * m + kk)
        ci = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
        dps.dp_gemm_bf16_ex(_offset_copy(ai, off), _offset_copy(bi, off), ci, b_layout=layout)
        torch.cuda.synchronize()
        check_gemm(ai, bi, layout, exact=True, c=ci)
