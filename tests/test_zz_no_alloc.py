"""dp_fsdp_layer_static (no caller workspaces, nothing allocated) against
dp_fsdp_layer_ex with caller workspaces: the same kernels run, so y, dx and the
dW shards must be bit-identical. Two calls in a row, the second with a smaller
problem, so that the static buffer's leftovers from the first call cannot leak
into the second; plus the forward-only form and the size limit."""
import numpy as np
import pytest
import torch

import gen
import gradient_sync_amd as dps
from tests.helpers import say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(k, m, d, f, seed):
    fx = gen.fsdp_fixture(seed=seed, k=k, m=m, d=d, f=f, device=DEV)
    ml, R = m // k, dps.dp_shard_len(d, k)
    xl = [fx["x"][r * ml:(r + 1) * ml].contiguous() for r in range(k)]
    dyl = [fx["dy"][r * ml:(r + 1) * ml].contiguous() for r in range(k)]
    ws = []
    for c in range(k):
        s = torch.zeros(R, f, device=DEV)
        rows = fx["w"][c * R:(c + 1) * R]
        s[:rows.shape[0]] = rows
        ws.append(s)
    return xl, ws, dyl, ml, R


def _run_both(k, m, d, f, seed, with_dx, backward=True):
    xl, ws, dyl, ml, R = _case(k, m, d, f, seed)
    nan = lambda *shape: torch.full(shape, float("nan"), device=DEV)
    # reference: caller workspaces
    wf = [nan(d, f) for _ in range(k)]
    dwf = [nan(d, f) for _ in range(k)]
    y_ref = [nan(ml, f) for _ in range(k)]
    dws_ref = [nan(R, f) for _ in range(k)]
    dx_ref = [nan(ml, d) for _ in range(k)] if with_dx else None
    dps.dp_fsdp_layer(xl, ws, dyl if backward else None, wf, y_ref, dwf if backward else None,
                      dws_ref if backward else None, dx_local=dx_ref)
    # allocation-free form
    y = [nan(ml, f) for _ in range(k)]
    dws = [nan(R, f) for _ in range(k)]
    dx = [nan(ml, d) for _ in range(k)] if with_dx else None
    torch.cuda.synchronize()
    dps.dp_fsdp_layer_static(xl, ws, dyl if backward else None, y,
                             dw_shard=dws if backward else None, dx_local=dx)
    torch.cuda.synchronize()
    for r in range(k):
        assert to_np(y[r]).tobytes() == to_np(y_ref[r]).tobytes(), r
        if backward:
            assert to_np(dws[r]).tobytes() == to_np(dws_ref[r]).tobytes(), r
        else:
            assert np.all(np.isnan(to_np(dws[r])))         # untouched
        if with_dx:
            assert to_np(dx[r]).tobytes() == to_np(dx_ref[r]).tobytes(), r


def test_static_fsdp_two_calls_second_smaller():
    say("static fsdp: K=8, x[1024,512], w[512,512], with dx")
    _run_both(8, 1024, 512, 512, seed=2, with_dx=True)
    say("static fsdp: K=4, x[256,256], w[256,128], no dx")
    _run_both(4, 256, 256, 128, seed=3, with_dx=False)


def test_static_fsdp_other_shapes_and_forward_only():
    say("static fsdp: K=3, non-divisible rows, separate launches")
    _run_both(3, 96, 70, 40, seed=4, with_dx=True)
    say("static fsdp: K=8 forward only")
    _run_both(8, 512, 256, 256, seed=5, with_dx=False, backward=False)
    say("static fsdp: K=8 again after the smaller calls")
    _run_both(8, 1024, 512, 512, seed=6, with_dx=False)


def test_static_fsdp_rejects_beyond_the_limit():
    # 2 * K * d * f * 4 bytes: K = 8, d = f = 1024 needs 64 MiB > 32 MiB
    k, m, d, f = 8, 64, 1024, 1024
    xl, ws, dyl, ml, R = _case(k, m, d, f, 7)
    y = [torch.empty(ml, f, device=DEV) for _ in range(k)]
    dws = [torch.empty(R, f, device=DEV) for _ in range(k)]
    with pytest.raises(dps.DpsyncError) as e:
        dps.dp_fsdp_layer_static(xl, ws, dyl, y, dw_shard=dws)
    assert e.value.code == dps.DP_ERR_SCRATCH
