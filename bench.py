#!/usr/bin/env python3
"""Throughput of data-parallel gradient synchronisation on one MI355X.

Default workload (one JSON line): K=8 data-parallel ranks emulated as 8 HBM
buffers, each holding the bf16 gradients of one transformer layer (GQA q/o
4096x4096, k/v 4096x1024, SwiGLU 3 x 4096x14336: 218,103,808 values,
N(0, 1e-3)), cut into 9 buckets of at most 25,000,000 elements. A step is, for
every bucket in order, an averaged ReduceScatter (fp32 accumulation in ring
order) into per-rank shards followed by an AllGather back to every rank, with
consecutive buckets pipelined: the ReduceScatter of bucket b+1 and the
AllGather of bucket b run in one launch. `value` is algorithmic HBM bytes per
step (ReduceScatter reads K*n and writes n, AllGather reads n and writes K*n,
per bucket of n elements) times steps, over the wall time of the timed steps,
in GB/s. The same step without the pipelining is reported beside it.

Other measurements (each prints its own JSON line):
  --config ring1m    K=4, 1,048,576 fp32 and int32, S=4, AllReduce
  --config fsdp      FSDP layer step, K=8, x[1024,512], w[512,512]
  --config weighted  token-weighted AllReduce, K=8, 10,000,019 fp32
  --config c3        RS+AG of 1 GiB/rank fp32 (K=8) concurrent with a bf16
                     8192^3 GEMM on another stream
  --config fused_ar  the layer buckets as one-pass AllReduce, against RS+AG
  --config odc       one minibatch with uneven microbatch counts: ODC pushes
                     and one settle vs padded per-microbatch ReduceScatter
  --config odc_push  the ODC push (8 gradients per launch) and settle kernels
                     alone, for profiling
  --config overlap   backward weight GEMMs of one layer (K=8) with the bucketed
                     AllReduce overlapped on a second stream, vs one stream
  --config gemm      the bf16 8192^3 GEMM alone (and the library GEMM for context)
  --config copy      plain 1 GiB elementwise copy (HBM ceiling, counter scale)
  --config all       the default line, then all of the above
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F32_TFLOPS = 157.3        # dense fp32 matrix
MFMA_BF16_TFLOPS = 2500.0      # dense bf16 matrix


# HBM bytes per full-size launch from two rocprofv3 PMC passes (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0, factors from a plain 1 GiB copy) recorded in
# profiles/sync_kernels_layer_k8_bf16.md, valid only for the kernel sources they
# were taken on (sha256 of sync_kernels.hip + sync_internal.h; the gfx950 code of
# these sources is the same as that of the tree the counters were taken on).
MEASURED_TRAFFIC = {
    "sources_sha256": "3a3ca48c3af27a5b60f65de0d68051dea2c9c4b12ca009b940fbd130c74c80c7"
                      "f16581e6b16ca798c1f240711e1e80c1a3d4fdf4628ca177e96c534422299b95",
    "rs_kernel<bf16, avg, K=8>": (2 * 195384.2 + 49415.8) * 1024,
    "ag_kernel<2-byte, K=8>": (2 * 25142.5 + 390736.1) * 1024,
    "rsag_kernel<bf16, avg, K=8>": (2 * 220517.3 + 439723.3) * 1024,
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_sha256() -> str:
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    out = ""
    for f in ("sync_kernels.hip", "sync_internal.h"):
        with open(os.path.join(here, "gradient_sync_amd", "csrc", f), "rb") as fh:
            out += hashlib.sha256(fh.read()).hexdigest()
    return out


# The oracle baselines use at most this many threads: a one-GPU machine is
# allotted 16 host cores, whatever the affinity mask of the process shows.
HOST_CORE_CAP = 16


def host_cores() -> int:
    return min(len(os.sched_getaffinity(0)), HOST_CORE_CAP)


def cores_note() -> str:
    return (f"oracle threads = min(affinity {len(os.sched_getaffinity(0))}, "
            f"cap {HOST_CORE_CAP}: the host cores a one-GPU box is allotted)")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bf16_bits(t):
    import numpy as np
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------- headline

def _in_rank_layout(ts):
    """The generated per-rank tensors copied into one allocation with the ranks
    a fixed gap apart (buckets.rank_buffers), the layout the sync steps are
    measured in; the separately allocated originals are freed by the caller."""
    from gradient_sync_amd.buckets import rank_buffers
    out = rank_buffers(len(ts), ts[0].numel(), ts[0].dtype, device=ts[0].device)
    for o, t in zip(out, ts):
        o.copy_(t)
    return out


def _rank_layout_note():
    from gradient_sync_amd.buckets import RANK_STAGGER_BYTES, SHARD_STAGGER_BYTES
    return (f"each of grads/shards/out in one allocation, ranks {RANK_STAGGER_BYTES // 1024} KiB "
            f"apart (bucket shards {SHARD_STAGGER_BYTES // 1024} KiB apart)")


def bench_layer(args):
    import torch

    import gen
    from gradient_sync_amd.buckets import BucketedSync

    k = 8
    total = gen.LAYER_PARAMS
    log(f"[bench] generating {k} x {total} bf16 gradients on the GPU")
    grads = _in_rank_layout(gen.layer_grads_bf16(3, k, device="cuda"))
    out = _in_rank_layout([torch.empty(total, dtype=torch.bfloat16, device="cuda") for _ in range(k)])
    sync = BucketedSync(grads, out, gen.BUCKET_ELEMS, op="avg")
    step_bytes = sync.algorithmic_bytes()
    # shard bytes: written by each bucket's ReduceScatter, read by its AllGather
    shard_bytes = sum(2 * n * 2 for _, n in sync.plan)

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record()
        for _ in range(args.steps):
            step()
        ev1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, ev0.elapsed_time(ev1)

    log(f"[bench] warmup {args.warmup}; timing {args.steps} pipelined steps, then plain steps")
    wall, gpu_ms = timed(sync.step_pipelined)
    value = step_bytes * args.steps / wall / 1e9
    wall_plain, _ = timed(sync.step)
    value_plain = step_bytes * args.steps / wall_plain / 1e9
    # Per-kernel durations: the same steps again, with a pair of HIP events
    # recorded on the launch stream around every launch. Kept out of the
    # throughput loops above because an event pair per launch costs ~0.1 ms.
    events = []
    torch.cuda.synchronize()
    for _ in range(args.steps):
        sync.step_pipelined(events=events)
    torch.cuda.synchronize()

    # per-launch durations of launches on full-size buckets only, per kernel
    full = gen.BUCKET_ELEMS
    per = {"rs": [], "rsag": [], "ag": []}
    tot = {"rs": 0.0, "rsag": 0.0, "ag": 0.0}
    for kind, b, e0, e1 in events:
        ms = e0.elapsed_time(e1)
        tot[kind] += ms
        sizes = [sync.plan[b][1]] + ([sync.plan[b - 1][1]] if kind == "rsag" else [])
        if all(n == full for n in sizes):
            per[kind].append(ms)
    bytes_of = {"rs": (k + 1) * full * 2, "ag": (k + 1) * full * 2, "rsag": 2 * (k + 1) * full * 2}
    kern = {kind: {"avg_us": 1e3 * statistics.mean(v), "median_us": 1e3 * statistics.median(v),
                   "gbs": bytes_of[kind] / (statistics.mean(v) * 1e-3) / 1e9, "launches": len(v)}
            for kind, v in per.items() if v}
    dom = max(tot, key=tot.get)
    achieved = kern[dom]["gbs"]
    launch_bytes = bytes_of[dom]
    names = {"rs": "rs_kernel<bf16, avg, K=8>", "ag": "ag_kernel<2-byte, K=8>",
             "rsag": "rsag_kernel<bf16, avg, K=8>"}
    traffic = (round(MEASURED_TRAFFIC[names[dom]])
               if kernel_sources_sha256() == MEASURED_TRAFFIC["sources_sha256"]
               and names[dom] in MEASURED_TRAFFIC else None)
    line = {
        "metric": "reduce-scatter+all-gather HBM GB/s (% of peak), K=8 bf16 25M-elem buckets",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "K=8 emulated ranks, one GQA+SwiGLU layer (hidden 4096) of bf16 "
                               "grads = 218,103,808 per rank, 9 buckets of <=25,000,000, "
                               "averaged ReduceScatter then AllGather per bucket, the "
                               "ReduceScatter of bucket b+1 fused with the AllGather of b",
                   "ranks": k, "params_per_rank": total, "bucket_elems": gen.BUCKET_ELEMS,
                   "buckets": len(sync.plan), "op": "avg", "accumulate": "fp32, ring order",
                   "rank_layout": _rank_layout_note()},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "bytes": "algorithmic: per bucket of n elements and phase, (K+1)*n*2 (each input "
                 "element read once, each output element written once). In the pipelined "
                 "step the shards (2*n*2 of the 2*(K+1)*n*2 bytes of a bucket) go through the "
                 "256 MB Infinity Cache between the two phases, so not all counted bytes "
                 "cross the HBM interface; plain_step below has no such reuse",
        "plain_step": {"value": round(value_plain, 2),
                       "pct_of_peak": round(100 * value_plain / HBM_PEAK_GBS, 2),
                       "ms_per_step": round(1e3 * wall_plain / args.steps, 4),
                       "schedule": "ReduceScatter then AllGather, one launch each, bucket by "
                                   "bucket (dp_reduce_scatter, dp_all_gather): shards stored "
                                   "with the nontemporal hint and read back from HBM, no cache "
                                   "reuse between the phases, every byte from or to HBM (the "
                                   "figure the 70%-of-HBM-peak target is judged on)"},
        "pipelined_excluding_shard_bytes": {
            "value": round((step_bytes - shard_bytes) * args.steps / wall / 1e9, 2),
            "pct_of_peak": round(100 * (step_bytes - shard_bytes) * args.steps / wall / 1e9
                                 / HBM_PEAK_GBS, 2),
            "what": "the pipelined step with the shard round trip left out of the bytes: a "
                    "lower bound on its HBM-only rate"},
        "kernel_timing": "HIP events around every launch in a second pass of the same steps",
        "bytes_per_step": step_bytes,
        "kernels": {names[k_]: {kk: (round(v, 2) if isinstance(v, float) else v)
                                for kk, v in d.items()} for k_, d in kern.items()},
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "traffic_source": "not measured in this run: the per-launch counters of "
                                       "profiles/sync_kernels_layer_k8_bf16.md, used only "
                                       "while the sync kernel sources hash to the value they "
                                       "were taken on (else null). FETCH_SIZE and WRITE_SIZE "
                                       "count L2-to-fabric bytes, so they include bytes the "
                                       "Infinity Cache serves and cannot separate them from "
                                       "HBM bytes",
                     "bytes_per_launch": launch_bytes,
                     "unit_bytes": "(K+1)*n*2 per bucket of n bf16 elements and phase; the "
                                   "fused launch carries one ReduceScatter and one AllGather"},
    }
    line["sharded_model"] = sharded_model(sync.plan, k, 2)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_layer(grads, k, args.cpu_seconds)
    return line


def sharded_model(plan, k, s):
    """Best-case transport time of the same step on K GPUs of one board, from
    the ring and direct-link bounds (no launch or protocol cost)."""
    from gradient_sync_amd import costmodel as cm
    ring = sum(cm.t_reduce_scatter_ring(n * s, k, cm.XGMI_LINK_BPS) +
               cm.t_all_gather_ring(n * s, k, cm.XGMI_LINK_BPS) for _, n in plan)
    direct = sum(2 * cm.t_direct_pull(n * s, k) for _, n in plan)
    return {"ring_xgmi_ms_per_step": round(1e3 * ring, 4),
            "direct_7link_ms_per_step": round(1e3 * direct, 4),
            "model": "ReduceScatter + AllGather per bucket over K GPUs, xGMI 76.8 GB/s per "
                     "directional link: one ring B(K-1)/(K W) per phase, or all K-1 peer "
                     "links at once B/(K W)"}


def cpu_baseline_layer(grads, k, seconds):
    """The oracle's ReduceScatter + AllGather of one 25,000,000-element bf16
    bucket (the first bucket of the same inputs), repeated for ~`seconds`."""
    import numpy as np

    import gen
    import oracle

    n = gen.BUCKET_ELEMS
    xs = [np.ascontiguousarray(bf16_bits(g[:n])) for g in grads]
    cores = host_cores()
    reps, t = 0, 0.0
    while reps == 0 or t < seconds:
        t0 = time.perf_counter()
        sh = oracle.reduce_scatter(xs, op="avg", nthreads=cores)
        out = oracle.all_gather(sh, n, nthreads=cores)
        t += time.perf_counter() - t0
        reps += 1
    b = 2 * (k + 1) * n * 2
    # once more on one thread: the per-element order does not depend on the
    # thread count, so the bits must be the same
    t0 = time.perf_counter()
    sh1 = oracle.reduce_scatter(xs, op="avg", nthreads=1)
    out1 = oracle.all_gather(sh1, n, nthreads=1)
    t1 = time.perf_counter() - t0
    same = all(a.tobytes() == c.tobytes() for a, c in zip(out, out1))
    if not same:
        raise RuntimeError("oracle results differ between 1 and many threads")
    return {"value": round(reps * b / t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x (ReduceScatter avg + AllGather) of bucket 0 "
                      f"(K=8 x 25,000,000 bf16), {t:.1f} s",
            "single_thread_value": round(b / t1 / 1e9, 3),
            "single_thread_bits_equal": same,
            "cpu_model": cpu_model(), "cores_note": cores_note()}


def _timed_reps(fn, seconds):
    """Run fn until ~seconds of CPU time have passed (at least once); returns
    (reps, seconds taken)."""
    reps, t = 0, 0.0
    while reps == 0 or t < seconds:
        t0 = time.perf_counter()
        fn()
        t += time.perf_counter() - t0
        reps += 1
    return reps, t


def cpu_baseline_rs_ag(xs, op, nbytes, seconds, sample, tokens=None):
    """The oracle's ReduceScatter + AllGather (token-weighted when tokens are
    given) of the host arrays xs, repeated for ~seconds; GB/s on nbytes per
    repetition."""
    import oracle
    cores = host_cores()
    n = int(xs[0].size)

    def once():
        if tokens is None:
            sh = oracle.reduce_scatter(xs, op=op, nthreads=cores)
        else:
            sh = oracle.weighted_reduce_scatter(xs, tokens, nthreads=cores)
        oracle.all_gather(sh, n, nthreads=cores)
    reps, t = _timed_reps(once, seconds)
    return {"value": round(reps * nbytes / t / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "sample": f"{reps} x {sample}, {t:.1f} s",
            "cores_note": cores_note(), "cpu_model": cpu_model()}


# ------------------------------------------------------------ other configs

def _time_ms(fn, warm=6, reps=9, stream=None):
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def _time_batch_ms(fn, batch=10, warm=1, reps=7):
    """Per-call ms of `batch` back-to-back calls between two events, so that
    the host-side argument marshalling of a call overlaps the previous launch
    instead of being timed with it."""
    def many():
        for _ in range(batch):
            fn()
    return [t / batch for t in _time_ms(many, warm=warm, reps=reps)]


def bench_ring1m(args):
    import torch

    import gen
    import gradient_sync_amd as dps
    k, n, s = 4, 1_048_576, 4
    xf = gen.ring_uniform_inputs(1, k, n, device="cuda")
    xi = [gen.int_copy(x) for x in xf]
    res = {}
    lib = dps.lib()
    for name, xs, op in (("f32_avg", xf, "avg"), ("i32_sum", xi, "sum")):
        out = [torch.empty_like(x) for x in xs]
        call = lambda: dps.dp_all_reduce(xs, out, op=op, s_chunks=s)
        ms = _time_ms(call)
        med = statistics.median(ms)
        back = statistics.median(_time_batch_ms(call, batch=20))
        # the same calls with the pointer arrays built once (no per-call
        # marshalling), and recorded once into a HIP graph and replayed
        dt = dps.DP_F32 if xs[0].dtype == torch.float32 else dps.DP_I32
        opc = dps.DP_AVG if op == "avg" else dps.DP_SUM
        sp, rp = dps.ptr_array([t.data_ptr() for t in xs]), dps.ptr_array([t.data_ptr() for t in out])

        def abi():
            rc = lib.dp_all_reduce(sp, rp, n, k, dt, opc, s, dps._stream(None))
            if rc:
                raise dps.DpsyncError(rc, "dp_all_reduce")
        back_abi = statistics.median(_time_batch_ms(abi, batch=20))
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            abi()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            for _ in range(20):
                abi()
        torch.cuda.synchronize()
        back_graph = statistics.median(_time_ms(graph.replay)) / 20
        b = 2 * (k + 1) * n * 4
        res[name] = {"median_us": round(1e3 * med, 2), "min_us": round(1e3 * min(ms), 2),
                     "back_to_back_us": round(1e3 * back, 2),
                     "back_to_back_abi_us": round(1e3 * back_abi, 2),
                     "graph_replay_us": round(1e3 * back_graph, 2),
                     "gbs_rs_ag_bytes": round(b / (back_graph * 1e-3) / 1e9, 1)}
    b = 2 * (k + 1) * n * 4
    line = {"metric": "ring AllReduce K=4 N=1,048,576 S=4 (cache-resident, launch-bound)",
            "unit": "us", "results": res,
            "roofline": {"bound": "hbm", "kernel": "rs_kernel<f32, avg, K=4, AllReduce> (one "
                                                   "pass), per call of a graph replay",
                         "achieved": res["f32_avg"]["gbs_rs_ag_bytes"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s",
                         "frac": round(res["f32_avg"]["gbs_rs_ag_bytes"] / HBM_PEAK_GBS, 4),
                         "traffic": None,
                         "note": "41.9 MB per call: inputs and outputs stay in the 256 MB "
                                 "Infinity Cache and a call lasts a few microseconds, so this "
                                 "measures launch latency, not HBM; GB/s on 2(K+1)N*4 bytes"},
            "timing": "median_us: one call between two events (host latency included); "
                      "back_to_back_us: per call of 20 back-to-back calls through the Python "
                      "binding; back_to_back_abi_us: the same through the C ABI with the "
                      "pointer arrays built once; graph_replay_us: 20 calls recorded in a "
                      "HIP graph, per call of a replay; GB/s (on the graph time) on the "
                      "ReduceScatter + AllGather bytes 2(K+1)Ns",
            "config": {"workload": "K=4, 1,048,576 fp32/int32, S=4"}}
    if not args.no_cpu_baseline:
        hx = [x.cpu().numpy() for x in xf]
        line["cpu_baseline"] = cpu_baseline_rs_ag(
            hx, "avg", b, args.cpu_seconds,
            "ReduceScatter (avg) + AllGather of the same K=4 x 1,048,576 fp32; GB/s on "
            "2(K+1)N*4 bytes")
    return line


def bench_fsdp(args):
    import torch

    import gen
    import gradient_sync_amd as dps
    k, m, d, f = 8, 1024, 512, 512
    fx = gen.fsdp_fixture(seed=2, k=k, device="cuda")
    ml, R = m // k, d // k
    xl = [fx["x"][r * ml:(r + 1) * ml].contiguous() for r in range(k)]
    dyl = [fx["dy"][r * ml:(r + 1) * ml].contiguous() for r in range(k)]
    ws = [fx["w"][c * R:(c + 1) * R].contiguous() for c in range(k)]
    wf = [torch.empty(d, f, device="cuda") for _ in range(k)]
    y = [torch.empty(ml, f, device="cuda") for _ in range(k)]
    dwf = [torch.empty(d, f, device="cuda") for _ in range(k)]
    dws = [torch.empty(R, f, device="cuda") for _ in range(k)]
    dx = [torch.empty(ml, d, device="cuda") for _ in range(k)]
    dps.dp_fsdp_layer(xl, ws, dyl, wf, y, dwf, dws, dx_local=dx)     # checks shapes once
    P = lambda ts: dps.ptr_array([t.data_ptr() for t in ts])
    args_c = (k, ml, d, f, P(xl), P(ws), P(dyl), P(wf), P(y), P(dwf), P(dws))
    args_x = (k, ml, d, f, P(xl), P(ws), P(dyl), P(wf), P(y), P(dx), P(dwf), P(dws))
    lib = dps.lib()
    batch = 20
    res = {}
    for name, fn, args_ in (("step", lib.dp_fsdp_layer, args_c),
                            ("step_with_dx", lib.dp_fsdp_layer_ex, args_x)):
        def steps():
            st = dps._stream(None)
            for _ in range(batch):
                rc = fn(*args_, st)
                if rc:
                    raise dps.DpsyncError(rc, name)
        ms = [t / batch for t in _time_ms(steps, warm=2, reps=9)]
        med = statistics.median(ms)
        gemms = 2 if name == "step" else 3
        flops = gemms * (2 * k * ml * d * f)
        res[name] = {"median_us": round(1e3 * med, 2), "min_us": round(1e3 * min(ms), 2),
                     "gemm_flops": flops,
                     "effective_tflops": round(flops / (med * 1e-3) / 1e12, 2)}
    line = {"metric": "FSDP layer step (AG w, y=xW, dW=x^T dy, RS dW), K=8",
            "timing": f"{batch} back-to-back calls between two HIP events, per call",
            "unit": "us", "median_us": res["step"]["median_us"], "min_us": res["step"]["min_us"],
            "gemm_flops": res["step"]["gemm_flops"],
            "effective_tflops": res["step"]["effective_tflops"],
            "with_dx": dict(res["step_with_dx"], what="the same plus the input gradient "
                                                       "dx = dy W^T (dp_fsdp_layer_ex)"),
            "mfma_peak_tflops": MFMA_F32_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "fsdp_step_k8_kernel (the one-launch step with every size fixed at compile time: one workgroup per CU, each wave a backward then a forward MFMA chain)",
                         "achieved": res["step"]["effective_tflops"], "peak": MFMA_F32_TFLOPS,
                         "unit": "TFLOP/s",
                         "frac": round(res["step"]["effective_tflops"] / MFMA_F32_TFLOPS, 4),
                         "traffic": None,
                         "unit_flops": "2 GEMMs of 2*m_local*d*f per rank (y = x W, dW = x^T dy), "
                                       "K=8: 1,073,741,824 per step; the AllGather and "
                                       "ReduceScatter bytes are folded into the operand loads"},
            "roofline_with_dx": {"bound": "mfma", "kernel": "fsdp_step_k8_kernel with dx (each wave a backward, a forward and a dx = dy W^T MFMA chain)",
                                 "achieved": res["step_with_dx"]["effective_tflops"], "peak": MFMA_F32_TFLOPS,
                                 "unit": "TFLOP/s",
                                 "frac": round(res["step_with_dx"]["effective_tflops"] / MFMA_F32_TFLOPS, 4),
                                 "traffic": None,
                                 "unit_flops": "3 GEMMs of 2*m_local*d*f per rank, K=8: 1,610,612,736 per step"},
            "config": {"workload": "K=8, x[1024,512] N(0,1), w[512,512] N(0,0.02^2), "
                                   "dy[1024,512] N(0,1), fp32"}}
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        hxl = [t.cpu().numpy() for t in xl]
        hws = [t.cpu().numpy() for t in ws]
        hdy = [t.cpu().numpy() for t in dyl]
        reps, t = _timed_reps(lambda: oracle.fsdp_layer(hxl, hws, hdy, nthreads=cores),
                              args.cpu_seconds)
        line["cpu_baseline"] = {
            "value": round(reps * res["step"]["gemm_flops"] / t / 1e9, 3), "unit": "GFLOP/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{reps} x the oracle's FSDP layer step (AllGather, fp64 y and dW, "
                      f"fp64 ReduceScatter) on the same K=8 fixture, {t:.1f} s; GFLOP/s on the "
                      f"same 2-GEMM flop count",
            "cores_note": cores_note(), "cpu_model": cpu_model()}
    return line


def bench_weighted(args):
    import torch

    import gen
    import gradient_sync_amd as dps
    k, n = 8, 10_000_019
    xs = gen.ring_uniform_inputs(4, k, n, device="cuda")
    toks = gen.token_counts(4, k)
    out = [torch.empty(n, device="cuda") for _ in range(k)]
    # rotate between two input sets so the working set exceeds the cache
    xs2 = gen.ring_uniform_inputs(6, k, n, device="cuda")
    out2 = [torch.empty(n, device="cuda") for _ in range(k)]
    flip = [0]
    res = {}
    for name, two_phase, b in (("one_pass", False, 2 * k * n * 4),
                               ("two_phase", True, 2 * (k + 1) * n * 4)):
        def go():
            a, o = (xs, out) if flip[0] == 0 else (xs2, out2)
            flip[0] ^= 1
            dps.dp_weighted_reduce_ex(a, o, toks, two_phase=two_phase)
        med = statistics.median(_time_batch_ms(go))
        single = statistics.median(_time_ms(go))
        res[name] = {"median_us": round(1e3 * med, 2), "bytes": b,
                     "gbs": round(b / (med * 1e-3) / 1e9, 1),
                     "pct_of_peak": round(100 * b / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                     "single_call_us": round(1e3 * single, 2)}
    line = {"metric": "token-weighted AllReduce K=8 N=10,000,019 fp32", "unit": "GB/s",
            "value": res["one_pass"]["gbs"], "results": res, "tokens": toks,
            "roofline": {"bound": "hbm", "kernel": "rs_kernel<f32, weighted, K=8, AllReduce> "
                                                   "(one pass)",
                         "achieved": res["one_pass"]["gbs"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(res["one_pass"]["gbs"] / HBM_PEAK_GBS, 4),
                         "traffic": None,
                         "unit_bytes": "2*K*n*4 per call (each input read once, each output "
                                       "written once), n = 10,000,019"},
            "timing": "median per call of 10 back-to-back calls between two events; "
                      "single_call_us: one call between two events (host latency included)",
            "config": {"workload": "K=8, 10,000,019 fp32 uniform[-1,1), log-normal(7,1) "
                                   "token counts, 2 docs/rank"}}
    if not args.no_cpu_baseline:
        hx = [x.cpu().numpy() for x in xs]
        line["cpu_baseline"] = cpu_baseline_rs_ag(
            hx, None, 2 * k * n * 4, args.cpu_seconds,
            "token-weighted ReduceScatter + AllGather of the same K=8 x 10,000,019 fp32; GB/s "
            "on the one-pass bytes 2*K*n*4", tokens=toks)
    return line


def bench_fused_ar(args):
    """The layer buckets as one one-pass AllReduce per bucket, against the
    ReduceScatter + AllGather step over the same buckets."""
    import torch

    import gen
    from gradient_sync_amd.buckets import BucketedSync
    k = 8
    grads = _in_rank_layout(gen.layer_grads_bf16(3, k, device="cuda"))
    out = _in_rank_layout([torch.empty(gen.LAYER_PARAMS, dtype=torch.bfloat16, device="cuda")
                           for _ in range(k)])
    sync = BucketedSync(grads, out, gen.BUCKET_ELEMS, op="avg")
    res = {}
    for name, fn, b in (("one_pass_all_reduce", sync.step_all_reduce, sync.all_reduce_bytes()),
                        ("reduce_scatter_all_gather", sync.step, sync.algorithmic_bytes())):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / args.steps
        res[name] = {"ms_per_step": round(1e3 * t, 4), "bytes_per_step": b,
                     "gbs": round(b / t / 1e9, 1), "pct_of_peak": round(100 * b / t / 1e9 / HBM_PEAK_GBS, 2)}
    res["speedup"] = round(res["reduce_scatter_all_gather"]["ms_per_step"] /
                           res["one_pass_all_reduce"]["ms_per_step"], 4)
    return {"metric": "averaged AllReduce of the K=8 bf16 layer buckets: one pass vs RS+AG",
            "unit": "ms", "results": res,
            "config": {"workload": "K=8, 218,103,808 bf16 per rank, 9 buckets of <=25,000,000",
                       "rank_layout": _rank_layout_note()}}


def bench_c3(args):
    import torch

    import gen
    import gradient_sync_amd as dps
    from gradient_sync_amd.buckets import rank_buffers
    from gradient_sync_amd.concurrency import SCHEDULES, C3Pair
    k, n = 8, 268_435_456
    log("[c3] generating 8 x 1 GiB fp32 and 2 x 8192^2 bf16")
    xs = rank_buffers(k, n, torch.float32)
    for r in range(k):
        xs[r].copy_(gen.uniform_pm1(5, 0, r, n, device="cuda"))
    L = dps.dp_shard_len(n, k)
    sh = rank_buffers(k, L, torch.float32)
    out = rank_buffers(k, n, torch.float32)
    a, b = gen.gemm_bf16_inputs(5, 8192, 8192, 8192, device="cuda")
    c = torch.empty(8192, 8192, dtype=torch.bfloat16, device="cuda")
    pair = C3Pair(xs, sh, out, a, b, c)
    comm_bytes = 2 * (k + 1) * n * 4
    flops = 2 * 8192 ** 3

    # T_comm and T_gemm: each kernel alone on the streams the schedule uses
    # (the CU-masked ones for RP); T_concurrent: start event to the later of
    # the two completion events. 6 warm-up + 9 measured runs, median.
    iso = {}
    res = {}
    wanted = args.schedules.split(",") if args.schedules else list(SCHEDULES)
    for name in wanted:
        if name not in SCHEDULES:
            raise SystemExit(f"bench.py: unknown C3 schedule {name!r}; known: {', '.join(SCHEDULES)}")
    for name in ["base"] + [w for w in wanted if w != "base"]:
        sched = SCHEDULES[name]
        try:
            sc, sg, closers = pair.streams(sched)
        except RuntimeError as e:
            res[name] = {"error": str(e)}
            continue
        try:
            key_c = ("comm", sched.comm_max_workgroups, sched.comm_cus)
            key_g = ("gemm", sched.gemm_share_cu, sched.comm_cus)
            if key_c not in iso:
                iso[key_c] = statistics.median(_time_ms(
                    lambda: pair.comm(sc, sched.comm_max_workgroups), stream=sc))
            if key_g not in iso:
                iso[key_g] = statistics.median(_time_ms(
                    lambda: pair.gemm(sg, sched.gemm_share_cu), stream=sg))

            def conc():
                start, ec, eg = pair.launch(sched, sc, sg)
                torch.cuda.synchronize()
                return max(start.elapsed_time(ec), start.elapsed_time(eg))
            for _ in range(6):
                conc()
            tc = statistics.median([conc() for _ in range(9)])
        finally:
            for st in closers:
                st.close()
        t_comm, t_gemm = iso[key_c], iso[key_g]
        s_ = (t_comm + t_gemm) / tc
        s_ideal = (t_comm + t_gemm) / max(t_comm, t_gemm)
        log(f"[c3] {name}: T_comm {t_comm:.3f} T_gemm {t_gemm:.3f} T_conc {tc:.3f} S {s_:.3f}")
        r = {"first": sched.first, "t_comm_ms": round(t_comm, 4), "t_gemm_ms": round(t_gemm, 4),
             "t_concurrent_ms": round(tc, 4), "S": round(s_, 4), "S_ideal": round(s_ideal, 4),
             "S_over_S_ideal": round(s_ / s_ideal, 4),
             "pct_of_ideal_gain": round(100 * (s_ - 1) / (s_ideal - 1), 1) if s_ideal > 1 else None}
        if sched.comm_cus:
            r["comm_cus"] = sched.comm_cus
            r["gemm_cus"] = torch.cuda.get_device_properties(0).multi_processor_count - sched.comm_cus
        else:
            r["comm_max_workgroups"] = sched.comm_max_workgroups
            r["gemm_share_cu"] = sched.gemm_share_cu
        res[name] = r
    comm_iso = [v for key, v in iso.items() if key[0] == "comm" and key[2] == 0]
    gemm_iso = [v for key, v in iso.items() if key[0] == "gemm" and key[2] == 0]
    best_serial = min(comm_iso) + min(gemm_iso)
    for v in res.values():
        if "t_concurrent_ms" in v:
            v["S_vs_best_serial"] = round(best_serial / v["t_concurrent_ms"], 4)
    t_comm0, t_gemm0 = iso[("comm", 0, 0)], iso[("gemm", False, 0)]
    best_name = max((kk for kk, v in res.items() if "S" in v),
                    key=lambda kk: res[kk]["S_vs_best_serial"])
    best = res[best_name]
    line = {"metric": "C3: RS+AG (K=8, 1 GiB/rank fp32) concurrent with bf16 GEMM 8192^3",
            "unit": "x (S = T_serial / T_concurrent)", "value": res["base"]["S"],
            "higher_is_better": True,
            "t_comm_ms": round(t_comm0, 4), "t_gemm_ms": round(t_gemm0, 4),
            "comm_gbs": round(comm_bytes / (t_comm0 * 1e-3) / 1e9, 1),
            "gemm_tflops": round(flops / (t_gemm0 * 1e-3) / 1e12, 1),
            "best_serial_ms": round(best_serial, 4),
            "best_schedule": {"name": best_name, "t_concurrent_ms": best["t_concurrent_ms"],
                              "S_vs_best_serial": best["S_vs_best_serial"]},
            "S_definition": "S = (T_comm + T_gemm) / T_concurrent with T_comm, T_gemm of the "
                            "same kernels run alone on the same streams; S_ideal = "
                            "(T_comm + T_gemm) / max; pct_of_ideal_gain = (S-1)/(S_ideal-1); "
                            "S_vs_best_serial = (fastest T_comm + fastest T_gemm, default "
                            "streams) / T_concurrent",
            "results": res,
            "roofline": {"bound": "hbm", "kernel": "the collective alone: rs_kernel<f32, sum, "
                                                   "K=8> then ag_kernel<4-byte, K=8>",
                         "achieved": round(comm_bytes / (t_comm0 * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(comm_bytes / (t_comm0 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None,
                         "unit_bytes": "(K+1)*n*4 per phase, n = 268,435,456, two phases"},
            "roofline_gemm": {"bound": "mfma", "kernel": "dp_gemm_bf16 8192^3",
                              "achieved": round(flops / (t_gemm0 * 1e-3) / 1e12, 1),
                              "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(flops / (t_gemm0 * 1e-3) / 1e12 / MFMA_BF16_TFLOPS, 4)},
            "config": {"workload": "K=8 x 268,435,456 fp32 RS(sum)+AG on stream A, "
                                   "bf16 GEMM 8192^3 on stream B; 6 warm-up + 9 measured",
                       "rank_layout": _rank_layout_note()}}
    if not args.no_cpu_baseline:
        n_s = 1 << 24
        hx = [xs[r][:n_s].cpu().numpy() for r in range(k)]
        line["cpu_baseline"] = cpu_baseline_rs_ag(
            hx, "sum", 2 * (k + 1) * n_s * 4, args.cpu_seconds,
            "ReduceScatter (sum) + AllGather of the first 16,777,216 elements of each rank "
            "(K=8 fp32); GB/s on the same (K+1)*n*4 bytes per phase")
    return line


def _odc_kernel_rooflines(rounds8, singles, acc, out, n, div, with_np1):
    """Average launch time of the push kernel with np = 8 (rotating over
    rounds8, each a list of 8 gradients) and np = 1 (rotating over singles),
    and of the bf16 settle with reset, against HBM peak."""
    import gradient_sync_amd as dps
    k = len(acc)
    L = dps.dp_shard_len(n, k)
    flip = [0, 0]

    def push8():
        flip[0] = (flip[0] + 1) % len(rounds8)
        dps.dp_scatter_accumulate(rounds8[flip[0]], acc)

    def push1():
        flip[1] = (flip[1] + 1) % len(singles)
        dps.dp_scatter_accumulate(singles[flip[1]], acc)

    def settle():
        dps.dp_settle(acc, out, n, divisor=div, reset=True)
    cases = [("scatter_accumulate_np8", push8, 8 * n * 2 + 8 * n)]
    if with_np1:
        cases.append(("scatter_accumulate_np1", push1, n * 2 + 8 * n))
    cases.append(("settle_bf16_reset", settle, 8 * n + k * L * 2))
    kern = {}
    batch = 10

    def many(fn):
        return lambda: [fn() for _ in range(batch)]
    for name, fn, b in cases:
        # back-to-back launches between two events, so that host-side argument
        # marshalling overlaps the previous launch
        med = statistics.median(_time_ms(many(fn), warm=1, reps=5)) / batch
        kern[name] = {"median_us": round(1e3 * med, 2), "bytes": b,
                      "gbs": round(b / (med * 1e-3) / 1e9, 1),
                      "frac_of_peak": round(b / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return kern


def bench_odc_push(args):
    """The ODC kernels alone at layer size (for profiling): 60 pushes of 8
    gradients each, then 60 bf16 settles with reset."""
    import torch

    import gen
    import gradient_sync_amd as dps
    k, n = 8, gen.LAYER_PARAMS
    L = dps.dp_shard_len(n, k)
    grads = [gen.microbatch_grad(1, r, m, n, device="cuda") for m in range(2) for r in range(k)]
    acc = [torch.zeros(L, dtype=torch.float32, device="cuda") for _ in range(k)]
    out = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    kern = _odc_kernel_rooflines([grads[:k], grads[k:]], grads, acc, out, n, 16.0, with_np1=False)
    return {"metric": "ODC push (8 gradients per launch) and settle kernels, K=8, one layer",
            "unit": "us", "kernels": kern,
            "config": {"workload": "K=8, 218,103,808 bf16 N(0,1e-3^2) gradients, two sets of 8 "
                                   "alternating, fp32 accumulators, bf16 settle with reset"}}


def bench_odc(args):
    """One minibatch of gradient synchronisation with uneven microbatch counts:
    on-demand scatter-accumulate pushes with one settle, against the padded
    per-microbatch ReduceScatter baseline. A push carries one microbatch's
    gradients of a whole transformer layer; every microbatch slot, padded ones
    included, has its own gradient buffer, so the working set (about 23 GB) is
    far larger than the on-chip caches."""
    import torch

    import gen
    import gradient_sync_amd as dps
    k, n, s = 8, gen.LAYER_PARAMS, 2
    counts = gen.microbatch_counts(1, k)
    mmax, total = max(counts), sum(counts)
    L = dps.dp_shard_len(n, k)
    grads = [[gen.microbatch_grad(1, r, m, n, device="cuda") for m in range(counts[r])]
             for r in range(k)]
    # an empty (padding) bucket contributes a zero gradient of its own
    padded = [[grads[r][m] if counts[r] > m else torch.zeros(n, dtype=torch.bfloat16, device="cuda")
               for r in range(k)] for m in range(mmax)]
    rounds = [[padded[m][r] for r in range(k) if counts[r] > m] for m in range(mmax)]
    acc = [torch.zeros(L, dtype=torch.float32, device="cuda") for _ in range(k)]
    out = [torch.empty(L, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    shard_buf = torch.empty(k * L, dtype=torch.bfloat16, device="cuda")
    shard_views = [shard_buf[c * L:(c + 1) * L] for c in range(k)]
    div = float(total)

    def settle():
        dps.dp_settle(acc, out, n, divisor=div, reset=True)

    def odc_nopad_drain():
        for rnd in rounds:
            dps.dp_scatter_accumulate(rnd, acc)
        settle()

    def odc_nopad_per_push():
        for rnd in rounds:
            for g in rnd:
                dps.dp_scatter_accumulate(g, acc)
        settle()

    def odc_pad_drain():
        for rnd in padded:
            dps.dp_scatter_accumulate(rnd, acc)
        settle()

    def nccl_pad():
        for rnd in padded:
            dps.dp_reduce_scatter(rnd, shard_views, op="sum")
            dps.dp_scatter_accumulate(shard_buf, acc)
        settle()

    settle_b = 8 * n + k * L * s
    push_b = lambda p: p * n * s + 8 * n
    sched = {
        "odc_nopad_drain": (odc_nopad_drain, mmax * 8 * n + total * n * s + settle_b, mmax + 1),
        "odc_nopad_per_push": (odc_nopad_per_push, total * push_b(1) + settle_b, total + 1),
        "odc_pad_drain": (odc_pad_drain, mmax * push_b(k) + settle_b, mmax + 1),
        "nccl_pad": (nccl_pad, mmax * (k * n * s + k * L * s + k * L * s + 8 * k * L) + settle_b,
                     2 * mmax + 1),
    }
    res = {}
    for name, (fn, b, launches) in sched.items():
        log(f"[bench] odc schedule {name}")
        ms = _time_ms(fn, warm=2, reps=7)
        med = statistics.median(ms)
        res[name] = {"median_ms": round(med, 4), "min_ms": round(min(ms), 4), "launches": launches,
                     "bytes": b, "gbs": round(b / (med * 1e-3) / 1e9, 1),
                     "pct_of_peak": round(100 * b / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    for name in ("odc_nopad_drain", "odc_pad_drain", "odc_nopad_per_push"):
        res[name]["speedup_vs_nccl_pad"] = round(res["nccl_pad"]["median_ms"] /
                                                 res[name]["median_ms"], 4)
    # kernel rooflines: one push of all K ranks' gradients, one single push, the settle
    flat = [g for rnd in rounds for g in rnd]
    kern = _odc_kernel_rooflines(padded, flat, acc, out, n, div, with_np1=True)
    return {"metric": "one minibatch of ODC gradient sync vs padded ReduceScatter, K=8, "
                      "one layer (218,103,808 bf16) per microbatch gradient",
            "unit": "ms", "counts": counts, "results": res, "kernels": kern,
            "config": {"workload": "K=8, 218,103,808 bf16 N(0,1e-3^2) per microbatch, microbatch "
                                   "counts ceil(tokens/2048) from log-normal(7,1) token counts "
                                   "(2 docs/rank, seed 1), fp32 owner accumulators, bf16 settle"}}


def bench_overlap(args):
    """Backward weight-gradient GEMMs of one layer for K=8 ranks with the
    bucketed averaged AllReduce overlapped on a second stream (a bucket goes as
    soon as all its gradients exist), against the same work on one stream.
    Variants: default kernels; the lean AllReduce (64 VGPRs, fits beside a GEMM
    workgroup) capped at 256 workgroups; the GEMM variant that leaves room for a
    default AllReduce workgroup; and the two streams on disjoint CU-masked sets
    (32 or 64 CUs for the AllReduces)."""
    import torch

    import gen
    import gradient_sync_amd as dps
    from gradient_sync_amd.buckets import BucketedSync
    from gradient_sync_amd.concurrency import CuMaskedStream
    k, total, cap = 8, gen.LAYER_PARAMS, gen.BUCKET_ELEMS
    pieces = gen.layer_backward_pieces()
    grad = [torch.empty(total, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    out = [torch.empty(total, dtype=torch.bfloat16, device="cuda") for _ in range(k)]
    nb = -(-total // cap)
    ev = dps.HipEvents(nb)
    comm = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    sync = BucketedSync(grad, out, cap, op="avg")
    n_cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for t in (256, 1024):
        log(f"[bench] overlap t={t}")
        dy, x = gen.backward_operands(6, k, pieces, t, device="cuda")
        flops = 2 * total * t * k

        def gemms(share_cu=False, lean=False):
            for g, (off, m, n) in enumerate(pieces):
                for r in range(k):
                    dps.dp_gemm_bf16_ex(dy[g * k + r], x[g * k + r],
                                        grad[r][off:off + m * n].view(m, n), share_cu=share_cu,
                                        lean=lean, b_layout="nk")

        def serial(**o):
            dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, cap, op="avg", **o)

        def overlapped(**o):
            comm.wait_stream(cur)
            dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, cap, op="avg",
                                              compute_stream=cur, comm_stream=comm, events=ev, **o)
            cur.wait_stream(comm)
        med = lambda fn: statistics.median(_time_ms(fn, warm=3, reps=9))
        r = {"gemm_flops": flops}
        r["t_gemm_ms"] = med(gemms)
        r["t_gemm_lean_ms"] = med(lambda: gemms(lean=True))
        r["t_gemm_share_cu_ms"] = med(lambda: gemms(share_cu=True))
        r["t_comm_ms"] = med(sync.step_all_reduce)
        variants = (("overlap", {}), ("overlap_lean_cap256", {"lean": True, "max_workgroups": 256}),
                    ("overlap_share_cu_cap256", {"share_cu": True, "max_workgroups": 256}))
        # serial reference: the default (fastest) kernels on one stream
        r["t_serial_ms"] = med(lambda: serial())
        r["t_serial_lean_ms"] = med(lambda: serial(lean=True))
        for name, o in variants:
            r[f"t_{name}_ms"] = med(lambda: overlapped(**o))
        names = [name for name, _ in variants]
        # RP: the GEMMs on a CU-masked stream with CUs [n_comm, all), the
        # AllReduces on one with CUs [0, n_comm), default kernels
        for n_comm in (32, 64):
            name = f"overlap_rp_comm{n_comm}"
            raw = []
            try:
                raw.append(CuMaskedStream(n_comm, n_cus))
                raw.append(CuMaskedStream(0, n_comm))
            except RuntimeError as e:
                r[f"error_{name}"] = str(e)
                for st in raw:
                    st.close()
                continue
            sc, sm = (st.stream for st in raw)

            def rp():
                sc.wait_stream(cur)
                sm.wait_stream(cur)
                dps.dp_backward_allreduce_overlap(pieces, t, dy, x, grad, out, cap, op="avg",
                                                  compute_stream=sc, comm_stream=sm, events=ev)
                cur.wait_stream(sc)
                cur.wait_stream(sm)
            r[f"t_{name}_ms"] = med(rp)
            for st in raw:
                st.close()
            names.append(name)
        for name in names:
            r[f"hidden_comm_frac_{name}"] = round(
                (r["t_serial_ms"] - r[f"t_{name}_ms"]) / r["t_comm_ms"], 4)
            r[f"speedup_{name}"] = round(r["t_serial_ms"] / r[f"t_{name}_ms"], 4)
        r["gemm_tflops"] = round(flops / (r["t_gemm_ms"] * 1e-3) / 1e12, 1)
        res[f"t{t}"] = {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in r.items()}
        del dy, x
        torch.cuda.empty_cache()
    ev.close()
    return {"metric": "backward weight GEMMs with bucketed averaged AllReduce overlapped, K=8, "
                      "one layer", "unit": "ms", "results": res,
            "config": {"workload": "K=8 ranks, the layer's 7 weight gradients (218,103,808 per "
                                   "rank) as bf16 GEMMs dW = dY^T X over t tokens per rank "
                                   "(t = 256 and 1024), 25,000,000-element buckets, one-pass "
                                   "averaged AllReduce per bucket"}}


def bench_gemm(args):
    """The bf16 GEMM of the concurrency measurement alone (C = A B, 8192^3,
    B stored [k, n]): the default (4-wave) kernel, the same with B stored [n, k]
    (C = A B^T, the direct-to-LDS kernel), and the two 8-wave variants that
    leave room for a sync workgroup on each CU, against the MFMA roofline; the
    vendor library GEMM (torch.matmul, hipBLASLt) on the same operands in both
    layouts for context; then the same kernels on a short k range (4096 x
    14336 x 256, a weight-gradient GEMM over 256 tokens). The variants
    are timed in interleaved rounds of 8 back-to-back calls after ~1 s of
    warm-up, so that they see the same clock and power state."""
    import torch

    import gen
    import gradient_sync_amd as dps
    m = n = kk = 8192
    a, b = gen.gemm_bf16_inputs(5, m, n, kk, device="cuda")
    b_nk = b.t().contiguous()
    c = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    flops = 2 * m * n * kk
    fns = {"dp_gemm_bf16": lambda: dps.dp_gemm_bf16(a, b, c),
           "dp_gemm_bf16_b_nk": lambda: dps.dp_gemm_bf16_ex(a, b_nk, c, b_layout="nk"),
           "dp_gemm_bf16_lean": lambda: dps.dp_gemm_bf16_ex(a, b, c, lean=True),
           "dp_gemm_bf16_share_cu": lambda: dps.dp_gemm_bf16_ex(a, b, c, share_cu=True),
           "library_torch_matmul": lambda: torch.matmul(a, b, out=c),
           "library_torch_matmul_b_nk": lambda: torch.matmul(a, b_nk.t(), out=c)}
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
    times = {name: [] for name in fns}
    for _ in range(8):
        for name, fn in fns.items():
            times[name].extend(_time_batch_ms(fn, batch=8, warm=0, reps=1))
    res = {}
    for name, v in times.items():
        med = statistics.median(v)
        tf = flops / (med * 1e-3) / 1e12
        res[name] = {"median_ms": round(med, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / MFMA_BF16_TFLOPS, 4)}
    line = {"metric": "bf16 GEMM C = A B, 8192^3, fp32 accumulation", "unit": "TFLOP/s",
            "value": res["dp_gemm_bf16"]["tflops"], "results": res,
            "timing": "interleaved rounds of 8 back-to-back calls between two events, "
                      "after ~1 s of warm-up; median per call",
            "roofline": {"bound": "mfma", "kernel": "gemm_bf16_w4dn_kernel (B stored [k, n], operands loaded straight into LDS, transposing LDS reads, 16x16x32 MFMAs, C in 16-byte stores)",
                         "achieved": res["dp_gemm_bf16"]["tflops"],
                         "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": res["dp_gemm_bf16"]["frac_of_peak"], "traffic": None},
            "roofline_b_nk": {"bound": "mfma",
                              "kernel": "gemm_bf16_w4d_kernel (B stored [n, k], operands loaded "
                                        "straight into LDS, 16x16x32 MFMAs, C in 16-byte stores)",
                              "achieved": res["dp_gemm_bf16_b_nk"]["tflops"],
                              "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": res["dp_gemm_bf16_b_nk"]["frac_of_peak"], "traffic": None},
            "config": {"workload": "A [8192, 8192], B [8192, 8192] bf16 ~ N(0,1), row-major"}}
    # a short k range (a weight-gradient GEMM over 256 tokens: 4096 x 14336,
    # kk = 256), where writing C weighs most: the default (direct-to-LDS) kernel
    # against the 8-wave one (DP_LAUNCH_LEAN) and the library, both layouts
    del a, b, b_nk, c
    ms, ns, ks = 4096, 14336, 256
    a, b = gen.gemm_bf16_inputs(6, ms, ns, ks, device="cuda")
    b_nk = b.t().contiguous()
    c = torch.empty(ms, ns, dtype=torch.bfloat16, device="cuda")
    fns = {"dp_gemm_bf16": lambda: dps.dp_gemm_bf16(a, b, c),
           "dp_gemm_bf16_lean": lambda: dps.dp_gemm_bf16_ex(a, b, c, lean=True),
           "library_torch_matmul": lambda: torch.matmul(a, b, out=c),
           "dp_gemm_bf16_b_nk": lambda: dps.dp_gemm_bf16_ex(a, b_nk, c, b_layout="nk"),
           "dp_gemm_bf16_b_nk_lean": lambda: dps.dp_gemm_bf16_ex(a, b_nk, c, b_layout="nk", lean=True),
           "library_torch_matmul_b_nk": lambda: torch.matmul(a, b_nk.t(), out=c)}
    times = {name: [] for name in fns}
    for _ in range(8):
        for name, fn in fns.items():
            times[name].extend(_time_batch_ms(fn, batch=8, warm=2, reps=1))
    line["short_k"] = {"workload": f"A [{ms}, {ks}], B [{ks}, {ns}] (or [{ns}, {ks}]) bf16, C [{ms}, {ns}]",
                       "results": {name: {"median_us": round(statistics.median(v) * 1e3, 2),
                                          "tflops": round(2 * ms * ns * ks / (statistics.median(v) * 1e-3) / 1e12, 1)}
                                   for name, v in times.items()}}
    del a, b, b_nk, c
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle
        cores = host_cores()
        a, b = gen.gemm_bf16_inputs(5, m, n, kk, device="cuda")
        ab, bb = bf16_bits(a), bf16_bits(b)
        rng = np.random.default_rng(0)
        rows = rng.integers(0, m, 256).astype(np.int64)
        cols = rng.integers(0, n, 256).astype(np.int64)
        reps, t = _timed_reps(lambda: oracle.gemm_bf16_at(ab, bb, rows, cols, nthreads=cores),
                              args.cpu_seconds)
        line["cpu_baseline"] = {
            "value": round(reps * 256 * 2 * kk / t / 1e9, 3), "unit": "GFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} x 256 sampled entries of the same product in fp64 (the oracle "
                      f"never forms the whole 8192^3 product), {t:.1f} s",
            "cores_note": cores_note(), "cpu_model": cpu_model()}
    return line


def bench_copy(args):
    """A plain elementwise device copy of known size (1 GiB read + 1 GiB
    written): the practical HBM ceiling on this GPU, and the reference against
    which the HBM byte counters are scaled."""
    import torch
    n = 1 << 28
    xs = [torch.ones(n, device="cuda") for _ in range(2)]
    ys = [torch.empty(n, device="cuda") for _ in range(2)]
    flip = [0]

    def go():
        i = flip[0]
        flip[0] ^= 1
        torch.neg(xs[i], out=ys[i])
    ms = _time_batch_ms(go, batch=10, warm=1, reps=7)
    med = statistics.median(ms)
    b = 2 * n * 4
    return {"metric": "plain elementwise copy (torch.neg), 1 GiB fp32 in, 1 GiB out",
            "unit": "GB/s", "value": round(b / (med * 1e-3) / 1e9, 1),
            "median_us": round(1e3 * med, 2), "bytes_per_launch": b,
            "pct_of_peak": round(100 * b / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


CONFIGS = {"ring1m": bench_ring1m, "fsdp": bench_fsdp, "weighted": bench_weighted, "c3": bench_c3,
           "fused_ar": bench_fused_ar, "odc": bench_odc, "odc_push": bench_odc_push,
           "overlap": bench_overlap, "gemm": bench_gemm, "copy": bench_copy}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="layer", choices=["layer", "all", *CONFIGS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--schedules", default="",
                    help="--config c3: comma-separated schedule names (default: all; the "
                         "base schedule always runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU (K ranks are emulated as K buffers in "
              f"one MI355X's HBM); --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import gradient_sync_amd  # noqa: F401  (fails loudly if the library is not built)
    if args.config in ("layer", "all"):
        print(json.dumps(bench_layer(args)), flush=True)
    for name, fn in CONFIGS.items():
        if args.config in (name, "all"):
            log(f"[bench] config {name}")
            print(json.dumps(fn(args)), flush=True)
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
