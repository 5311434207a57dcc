"""Compile libdpsync.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

The library is built in-tree next to this file so it travels with the source
tree. It links libamdhip64 by soname, so inside a PyTorch process it binds to
the HIP runtime PyTorch has already loaded (one runtime, shared streams).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdpsync.so")
SOURCES = ["api.hip", "sync_kernels.hip", "gemm_f32.hip", "gemm_bf16.hip", "odc_kernels.hip",
           "fsdp_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # fp32 arithmetic exactly as written: no contraction into FMA, IEEE
    # division, denormals kept
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
    inc = ["-I", CSRC, "-I", os.path.join(ROOT, "include")]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(ROOT, "_build", src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
