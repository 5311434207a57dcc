"""Transport-time and byte models of the collectives, for predicting what the
synchronisation would cost when the K ranks are K GPUs linked by xGMI.

Sources:
- "CMU 11-868 L14-L15: Distributed Training and Data Parallelism, and Where
  Gradient Sync Costs Come From", section "Why a ring: chop the data so
  transfers pipeline": time of a one-way ring broadcast of N bytes over K GPUs at
  link bandwidth B, sent whole or cut into S messages.
- "Sharding and Parallelism", section "The cost of the inserted collectives":
  lower bounds of the ring AllGather, ReduceScatter and AllReduce of a B-byte
  buffer over X devices at per-hop bandwidth W, and of AllToAll at aggregate
  egress W_X; section "Communication predictions": the FSDP-gather and
  expert-dispatch byte tables and their times on xGMI; section "Extending the
  mesh across nodes": the directional link ceilings.

All sizes are bytes and all bandwidths bytes per second; times are seconds.
These are best-case bounds (no launch, synchronisation or protocol cost).
"""
from __future__ import annotations

# Directional line-rate ceilings inside an eight-GPU MI355X board ("Sharding and
# Parallelism", section "Extending the mesh across nodes").
XGMI_LINK_BPS = 76.8e9          # one direct peer link, one direction
XGMI_PEERS = 7                  # direct peers of one GPU on the board


def ring_broadcast_time(n_bytes: float, k: int, link_bps: float, s_messages: int = 1) -> float:
    """One-way ring broadcast of n_bytes over k GPUs: whole, (k-1) hops of
    n/B each; cut into S messages that pipeline hop to hop,
    (k - 2 + S) * n / (S * B). S = 1 gives the whole-message time."""
    if k < 1 or s_messages < 1:
        raise ValueError("k and s_messages must be >= 1")
    if k == 1:
        return 0.0
    return (k - 2 + s_messages) * n_bytes / (s_messages * link_bps)


def ring_bytes_sent_per_rank(buffer_bytes: float, x: int) -> float:
    """Bytes each rank sends in a ring AllGather (or ReduceScatter) of a
    buffer_bytes buffer over x devices: its 1/x chunk once per round, x-1
    rounds."""
    if x < 1:
        raise ValueError("x must be >= 1")
    return buffer_bytes * (x - 1) / x


def t_all_gather_ring(buffer_bytes: float, x: int, w_bps: float) -> float:
    """Lower bound B(X-1)/(XW) of a ring AllGather that completes a B-byte buffer."""
    return ring_bytes_sent_per_rank(buffer_bytes, x) / w_bps


def t_reduce_scatter_ring(buffer_bytes: float, x: int, w_bps: float) -> float:
    """Lower bound B(X-1)/(XW) of a ring ReduceScatter of a B-byte buffer."""
    return ring_bytes_sent_per_rank(buffer_bytes, x) / w_bps


def t_all_reduce_ring(buffer_bytes: float, x: int, w_bps: float) -> float:
    """Lower bound 2B(X-1)/(XW): ReduceScatter then AllGather."""
    return 2.0 * ring_bytes_sent_per_rank(buffer_bytes, x) / w_bps


def all_to_all_remote_bytes(local_bytes: float, x: int) -> float:
    """Bytes each rank sends off-rank in an AllToAll of local_bytes split into
    x destination blocks (one block stays local)."""
    if x < 1:
        raise ValueError("x must be >= 1")
    return local_bytes * (x - 1) / x


def t_all_to_all(local_bytes: float, x: int, egress_bps: float) -> float:
    """Lower bound L(X-1)/(X W_X) at aggregate egress bandwidth W_X."""
    return all_to_all_remote_bytes(local_bytes, x) / egress_bps


def t_all_to_all_direct_links(local_bytes: float, x: int,
                              link_bps: float = XGMI_LINK_BPS) -> float:
    """AllToAll with all x-1 direct peer links busy at once: W_X = (x-1) * link,
    so the bound becomes L / (x * link)."""
    if x <= 1:
        return 0.0
    return t_all_to_all(local_bytes, x, (x - 1) * link_bps)


def t_direct_pull(buffer_bytes: float, x: int, link_bps: float = XGMI_LINK_BPS) -> float:
    """ReduceScatter or AllGather done as one direct exchange: every GPU moves
    its x-1 remote chunks of B/x bytes over x-1 peer links at once, so the bound
    is B/(x * link) (the AllToAll bound with the same per-destination blocks)."""
    return t_all_to_all_direct_links(buffer_bytes, x, link_bps)
