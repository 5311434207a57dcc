"""Gradient buckets: a flat per-rank gradient cut into fixed-size buckets, each
synchronised as one ReduceScatter followed by one AllGather.

DDP groups gradients into buckets whose size is capped, with a parameter ->
bucket mapping fixed up front and the same bucket order on every rank; each
ready bucket gets one collective (CMU 11-868 L14-L15 notes, section "When to
sync: gradient bucketing", and "What the paper adds beyond the slides": 25 MB
default cap, buckets issued strictly in order). Here the K ranks' flattened
gradients are K contiguous device buffers and a bucket is an (offset, length)
view of all of them, so bucketing copies nothing.

All argument marshalling (pointer arrays, shard buffers) is done once at
construction, so a step only enqueues 2 launches per bucket.
"""
from __future__ import annotations

import torch

from . import (DP_AVG, DP_SUM, _DTYPES, _check, _stream, dp_shard_len, lib, ptr_array)


def bucket_plan(total: int, cap: int) -> list[tuple[int, int]]:
    """(offset, length) of consecutive buckets of at most `cap` elements, in order."""
    if cap < 1:
        raise ValueError("bucket cap must be >= 1")
    return [(o, min(cap, total - o)) for o in range(0, total, cap)]


# Extra bytes between consecutive emulated ranks' buffers in one allocation,
# and between consecutive shards of a bucket. Every sync kernel touches the K
# ranks at the same offset at the same time. Measured on MI355X (same bits in
# every layout; medians of 10 shuffled rounds, three allocations):
#   K = 8 bf16 layer step, 218,103,808 values per rank in 25,000,000-value
#   buckets: 75.4-75.5% of HBM peak with separately allocated buffers or one
#   allocation with no gaps; 75.9-76.6% with rank gaps of 64-128 KiB;
#   8 x 1 GiB fp32 ReduceScatter + AllGather: 72.1% separately allocated,
#   76.5-76.8% with gaps of 96-160 KiB (64 KiB: 76.1% in one allocation,
#   71.6% in another).
RANK_STAGGER_BYTES = 128 * 1024
SHARD_STAGGER_BYTES = 64 * 1024


def rank_buffers(k: int, n: int, dtype=torch.bfloat16, device="cuda",
                 stagger: int = RANK_STAGGER_BYTES) -> list[torch.Tensor]:
    """K contiguous length-n tensors, one per emulated rank, carved from one
    allocation: rank r starts at r * (n * element_size rounded up to 256 bytes
    + stagger) bytes. `stagger` must be a multiple of 256."""
    if k < 1 or n < 0 or stagger < 0 or stagger % 256:
        raise ValueError("rank_buffers: need k >= 1, n >= 0 and a stagger that is a multiple of 256")
    es = torch.empty(0, dtype=dtype).element_size()
    stride = (-(-n * es // 256) * 256 + stagger) // es
    slab = torch.empty(max(1, (k - 1) * stride + n), dtype=dtype, device=device)
    return [slab[r * stride:r * stride + n] for r in range(k)]


class BucketedSync:
    """Averaged (or summed) AllReduce of K flat gradients, bucket by bucket,
    as ReduceScatter into per-bucket shard buffers and AllGather into `out`.

    grads, out : K contiguous device tensors of the same dtype and length.
    cap        : bucket size in elements.
    The shards of bucket b for rank c live in one preallocated buffer; each
    shard starts on a 256-byte boundary, `shard_stagger` bytes after the end
    of the previous one (the gap of `rank_buffers`).
    """

    def __init__(self, grads, out, cap: int, op: str = "avg", s_chunks: int = 1,
                 shard_stagger: int = SHARD_STAGGER_BYTES):
        self.k = k = len(grads)
        if len(out) != k:
            raise ValueError("grads and out need one tensor per rank")
        dt = grads[0].dtype
        total = grads[0].numel()
        for t in list(grads) + list(out):
            if t.dtype != dt or t.numel() != total or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError("grads/out must be contiguous GPU tensors of one dtype and length")
        self.dtype = _DTYPES[dt]
        self.es = grads[0].element_size()
        self.op = {"sum": DP_SUM, "avg": DP_AVG}[op]
        self.s_chunks = s_chunks
        self.plan = bucket_plan(total, cap)
        if shard_stagger < 0 or shard_stagger % 256:
            raise ValueError("shard_stagger must be a non-negative multiple of 256")
        align = max(1, 256 // self.es)
        self.shard_len = [dp_shard_len(n, k) for _, n in self.plan]
        self.slot = [-(-L // align) * align + shard_stagger // self.es for L in self.shard_len]
        self.shards = torch.empty(k * sum(self.slot), dtype=dt, device=grads[0].device)
        base = self.shards.data_ptr()
        self.calls = []
        pos = 0
        for (off, n), slot in zip(self.plan, self.slot):
            send = ptr_array([g.data_ptr() + off * self.es for g in grads])
            sh = ptr_array([base + (pos + c * slot) * self.es for c in range(k)])
            dst = ptr_array([o.data_ptr() + off * self.es for o in out])
            self.calls.append((send, sh, dst, n))
            pos += k * slot
        self.grads, self.out = grads, out   # keep the tensors alive

    def shard_view(self, b: int, c: int) -> torch.Tensor:
        """Shard c of bucket b (L_b elements, pads included)."""
        pos = sum(self.k * s for s in self.slot[:b]) + c * self.slot[b]
        return self.shards[pos:pos + self.shard_len[b]]

    def reduce_scatter(self, b: int, stream=None):
        send, sh, _, n = self.calls[b]
        _check(lib().dp_reduce_scatter(send, sh, n, self.k, self.dtype, self.op, self.s_chunks,
                                       _stream(stream)), "dp_reduce_scatter")

    def all_gather(self, b: int, stream=None):
        _, sh, dst, n = self.calls[b]
        _check(lib().dp_all_gather(sh, dst, n, self.k, self.dtype, self.s_chunks,
                                   _stream(stream)), "dp_all_gather")

    def step(self, stream=None, events=None):
        """One pass over every bucket in order. With `events` (a list), a pair of
        torch.cuda.Event is recorded around each launch and appended as
        (kind, bucket, start, end)."""
        st = _stream(stream)
        L = lib()
        torch_stream = stream if isinstance(stream, torch.cuda.Stream) else None
        for b, (send, sh, dst, n) in enumerate(self.calls):
            for kind in ("rs", "ag"):
                if events is not None:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(torch_stream)
                if kind == "rs":
                    rc = L.dp_reduce_scatter(send, sh, n, self.k, self.dtype, self.op,
                                             self.s_chunks, st)
                else:
                    rc = L.dp_all_gather(sh, dst, n, self.k, self.dtype, self.s_chunks, st)
                if rc:
                    _check(rc, f"bucket {b} {kind}")
                if events is not None:
                    e1.record(torch_stream)
                    events.append((kind, b, e0, e1))

    def step_all_reduce(self, stream=None):
        """Each bucket as one AllReduce call (the one-pass kernel: every shard
        folded once and written to all K outputs; no shard buffer)."""
        st = _stream(stream)
        L = lib()
        for b, (send, _, dst, n) in enumerate(self.calls):
            rc = L.dp_all_reduce(send, dst, n, self.k, self.dtype, self.op, self.s_chunks, st)
            if rc:
                _check(rc, f"bucket {b} all_reduce")

    def all_reduce_bytes(self) -> int:
        """Bytes one one-pass AllReduce step must move: K*n read, K*n written."""
        return sum(2 * self.k * n * self.es for _, n in self.plan)

    def algorithmic_bytes(self) -> int:
        """Bytes one step must move: per bucket, ReduceScatter reads K*n and
        writes n elements, AllGather reads n and writes K*n."""
        return sum(2 * (self.k + 1) * n * self.es for _, n in self.plan)

    def step_pipelined(self, stream=None, events=None):
        """The same step with consecutive buckets overlapped: ReduceScatter of
        bucket 0, then for b = 1.. one launch that reduces bucket b while
        gathering bucket b-1, then the AllGather of the last bucket. Same bits as
        step(). `events` as in step(), kinds "rs", "rsag", "ag"."""
        st = _stream(stream)
        L = lib()
        torch_stream = stream if isinstance(stream, torch.cuda.Stream) else None
        nb = len(self.calls)

        def launch(kind, b, fn):
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(torch_stream)
            rc = fn()
            if rc:
                _check(rc, f"bucket {b} {kind}")
            if events is not None:
                e1.record(torch_stream)
                events.append((kind, b, e0, e1))
        # bucket 0 alone through the standalone call, nontemporal shard stores:
        # its shards are then read from HBM by the next launch, and still the
        # step is faster than with the pipeline call's cached shard stores
        # (1.2370 against 1.2407 ms per step, interleaved, same bits)
        send, sh, dst, n = self.calls[0]
        launch("rs", 0, lambda: L.dp_reduce_scatter(send, sh, n, self.k, self.dtype, self.op,
                                                     self.s_chunks, st))
        for b in range(1, nb):
            send, sh, _, n = self.calls[b]
            _, psh, pdst, pn = self.calls[b - 1]
            launch("rsag", b, lambda: L.dp_reduce_scatter_all_gather(
                send, sh, n, psh, pdst, pn, self.k, self.dtype, self.op, self.s_chunks, st))
        _, sh, dst, n = self.calls[nb - 1]
        launch("ag", nb - 1, lambda: L.dp_all_gather(sh, dst, n, self.k, self.dtype,
                                                     self.s_chunks, st))
