"""The collective cost model against the values and closed forms the pages
print (CPU only)."""
import math
import os

import pytest

from gradient_sync_amd import costmodel as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cost_model_printed_values.txt")
UNIT = {"MB": 1e6, "ms": 1e-3, "B": 1.0}


def printed():
    rows = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        table, param, value, unit = line.split()
        rows[(table, param)] = (float(value) * UNIT[unit], len(value.split(".")[-1]) if "." in value else 0, unit)
    return rows


def close_to_printed(x, printed_value, decimals, unit):
    """x rounds to the printed value at the printed number of decimals."""
    return round(x / UNIT[unit], decimals) == pytest.approx(printed_value / UNIT[unit], abs=1e-12)


def test_fsdp_gather_table():
    p = printed()
    shard = p[("shard_bytes", "all")][0]
    assert shard == 1_610_612_736 / 8
    for f in (1, 2, 4, 8):
        want, dec, unit = p[("fsdp_ag_bytes", str(f))]
        # the gathered buffer of an f-way FSDP group is f local shards
        got = cm.ring_bytes_sent_per_rank(f * shard, f)
        assert close_to_printed(got, want, dec, unit), (f, got)
    for f in (2, 4, 8):
        want, dec, unit = p[("fsdp_ag_time", str(f))]
        got = cm.t_all_gather_ring(f * shard, f, cm.XGMI_LINK_BPS)
        assert close_to_printed(got, want, dec, unit), (f, got)
        # the matching ReduceScatter has the same ideal ring term
        assert cm.t_reduce_scatter_ring(f * shard, f, cm.XGMI_LINK_BPS) == got


def test_expert_dispatch_table():
    p = printed()
    payload = p[("a2a_payload", "all")][0]
    assert payload == 32_768 * 2 * 6_144 * 2
    for e in (8, 4, 2, 1):
        want, dec, unit = p[("a2a_remote_bytes", str(e))]
        assert close_to_printed(cm.all_to_all_remote_bytes(payload, e), want, dec, unit), e
    for e in (8, 2):
        want, dec, unit = p[("a2a_direct_time", str(e))]
        assert close_to_printed(cm.t_all_to_all_direct_links(payload, e), want, dec, unit), e


def test_ring_broadcast_closed_forms():
    n, b = 1e9, 50e9
    for k in range(2, 10):
        # sent whole: K-1 hops of N/B
        assert cm.ring_broadcast_time(n, k, b) == pytest.approx((k - 1) * n / b)
        # S = 1 is the whole message
        assert cm.ring_broadcast_time(n, k, b, 1) == cm.ring_broadcast_time(n, k, b)
        # chopping never hurts, and tends to N/B as S grows
        ts = [cm.ring_broadcast_time(n, k, b, s) for s in (1, 2, 4, 16, 1 << 20)]
        assert all(x >= y for x, y in zip(ts, ts[1:]))
        assert ts[-1] == pytest.approx(n / b, rel=1e-5)
        assert min(ts) >= n / b
    # two GPUs: one hop whatever S
    for s in (1, 3, 64):
        assert cm.ring_broadcast_time(n, 2, b, s) == pytest.approx(n / b)
    assert cm.ring_broadcast_time(n, 1, b, 4) == 0.0


def test_ring_bounds_relations():
    buf, w = 50e6, cm.XGMI_LINK_BPS
    for x in (1, 2, 4, 8):
        ag = cm.t_all_gather_ring(buf, x, w)
        assert ag == pytest.approx(buf * (x - 1) / (x * w))
        assert cm.t_all_reduce_ring(buf, x, w) == pytest.approx(2 * ag)
    # all seven links at once against one ring hop: 7x faster for K = 8
    assert cm.t_direct_pull(buf, 8) * 7 == pytest.approx(cm.t_all_gather_ring(buf, 8, cm.XGMI_LINK_BPS))
    assert math.isclose(cm.XGMI_PEERS * cm.XGMI_LINK_BPS, 537.6e9)
    with pytest.raises(ValueError):
        cm.ring_bytes_sent_per_rank(1.0, 0)


def test_mutant_off_by_one_hop_is_caught():
    # a model with X hops instead of X-1 misses the printed FSDP rows
    p = printed()
    shard = p[("shard_bytes", "all")][0]
    want, dec, unit = p[("fsdp_ag_bytes", "4")]
    wrong = 4 * shard * 4 / 4
    assert not close_to_printed(wrong, want, dec, unit)
