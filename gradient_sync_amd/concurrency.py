"""Concurrent computation and communication on one GPU (C3 schedules).

A collective (ReduceScatter then AllGather, fp32 sum) on one stream and a bf16
GEMM on another, with no data dependence between them ("Optimizing ML
Concurrent Computation and Communication with GPU DMA Engines", section "Problem
Formulation": T_serial is the sum of the two kernels' isolated times,
T_concurrent the time of the pair run together, S = T_serial / T_concurrent).
The schedules are that page's levers (section Q2, schedule prioritisation and
resource partitioning) in the form one GPU offers:

  base              default grids, the GEMM enqueued first
  base_comm_first   default grids, the collective enqueued first
  sp_capN           schedule prioritisation: the collective enqueued first, its
                    resident workgroups capped at N so the GEMM still gets CUs
  share_cu*         one persistent sync workgroup per CU beside one workgroup of
                    the GEMM variant with the smaller register footprint
  rp_commN          resource partitioning: the collective on a stream confined
                    to N CUs, the GEMM on a stream holding the other CUs

Everything here is stream and launch plumbing around the library's calls; the
arithmetic runs in libdpsync's kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import dp_all_gather_ex, dp_gemm_bf16_ex, dp_reduce_scatter_ex


@dataclass(frozen=True)
class Schedule:
    name: str
    comm_max_workgroups: int = 0     # 0: one workgroup per tile
    gemm_share_cu: bool = False
    first: str = "gemm"              # which kernel is enqueued first
    comm_cus: int = 0                # > 0: RP with the collective on CUs [0, comm_cus)


SCHEDULES = {s.name: s for s in (
    Schedule("base"),
    Schedule("base_comm_first", first="comm"),
    Schedule("sp_cap256", comm_max_workgroups=256, first="comm"),
    Schedule("sp_cap128", comm_max_workgroups=128, first="comm"),
    Schedule("share_cu", comm_max_workgroups=256, gemm_share_cu=True, first="comm"),
    Schedule("share_cu_gemm_first", comm_max_workgroups=256, gemm_share_cu=True),
    *(Schedule(f"rp_comm{n}", comm_cus=n) for n in (128, 144, 160, 176, 192)),
)}

_hip = None


def _hip_runtime():
    """The HIP runtime torch already loaded (stream calls torch does not wrap)."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipExtStreamCreateWithCUMask.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                   ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
        h.hipExtStreamCreateWithCUMask.restype = ctypes.c_int
        h.hipStreamDestroy.argtypes = [ctypes.c_void_p]
        h.hipStreamDestroy.restype = ctypes.c_int
        h.hipGetErrorString.argtypes = [ctypes.c_int]
        h.hipGetErrorString.restype = ctypes.c_char_p
        _hip = h
    return _hip


class CuMaskedStream:
    """A stream of default priority whose kernels run only on CU mask bits
    [first_cu, last_cu). Mask bits go round-robin over the XCDs, so a
    contiguous range gives every XCD the same number of CUs, which the driver
    requires of a mask. `.stream` is a torch stream view of it; close() (or
    the context manager) synchronises the device and destroys it."""

    def __init__(self, first_cu: int, last_cu: int):
        hip = _hip_runtime()
        n_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        if not 0 <= first_cu < last_cu <= n_cus:
            raise ValueError(f"CU range [{first_cu}, {last_cu}) outside [0, {n_cus})")
        words = (n_cus + 31) // 32
        mask = (ctypes.c_uint32 * words)()
        for b in range(first_cu, last_cu):
            mask[b // 32] |= 1 << (b % 32)
        raw = ctypes.c_void_p()
        rc = hip.hipExtStreamCreateWithCUMask(ctypes.byref(raw), words, mask)
        if rc != 0:
            raise RuntimeError("hipExtStreamCreateWithCUMask: "
                               + hip.hipGetErrorString(rc).decode())
        self._raw = raw
        self.stream = torch.cuda.ExternalStream(raw.value)

    def close(self):
        if self._raw is not None:
            torch.cuda.synchronize()
            _hip_runtime().hipStreamDestroy(self._raw)
            self._raw = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


class C3Pair:
    """The (collective, GEMM) pair: ReduceScatter (sum) of xs into shards then
    AllGather of the shards into out, and c = dp_gemm_bf16(a, b)."""

    def __init__(self, xs, shards, out, a, b, c):
        self.xs, self.shards, self.out = xs, shards, out
        self.a, self.b, self.c = a, b, c

    def comm(self, stream=None, max_workgroups: int = 0):
        dp_reduce_scatter_ex(self.xs, self.shards, op="sum", max_workgroups=max_workgroups,
                             stream=stream)
        dp_all_gather_ex(self.shards, self.out, max_workgroups=max_workgroups, stream=stream)

    def gemm(self, stream=None, share_cu: bool = False):
        dp_gemm_bf16_ex(self.a, self.b, self.c, share_cu=share_cu, stream=stream)

    def streams(self, sched: Schedule):
        """(comm stream, gemm stream, closers) for a schedule."""
        if sched.comm_cus:
            n_cus = torch.cuda.get_device_properties(
                torch.cuda.current_device()).multi_processor_count
            sc = CuMaskedStream(0, sched.comm_cus)
            try:
                sg = CuMaskedStream(sched.comm_cus, n_cus)
            except Exception:
                sc.close()
                raise
            return sc.stream, sg.stream, [sc, sg]
        return torch.cuda.Stream(), torch.cuda.Stream(), []

    def launch(self, sched: Schedule, comm_stream, gemm_stream):
        """Enqueue the pair after a start event on the current stream; returns
        (start, comm_done, gemm_done) timing events. The caller synchronises."""
        start = torch.cuda.Event(enable_timing=True)
        done_c = torch.cuda.Event(enable_timing=True)
        done_g = torch.cuda.Event(enable_timing=True)
        start.record(torch.cuda.current_stream())
        comm_stream.wait_event(start)
        gemm_stream.wait_event(start)
        jobs = [(lambda: self.comm(comm_stream, sched.comm_max_workgroups), comm_stream, done_c),
                (lambda: self.gemm(gemm_stream, sched.gemm_share_cu), gemm_stream, done_g)]
        if sched.first == "gemm":
            jobs.reverse()
        for fn, st, ev in jobs:
            fn()
            ev.record(st)
        return start, done_c, done_g
