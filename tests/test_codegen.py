"""Properties of the gfx950 code the library's kernels compile to (CPU only:
hipcc cross-compiles the device code; nothing runs).

- no kernel spills to scratch;
- the sync kernels move data with 16-byte vector loads and stores;
- the lean ReduceScatter/AllReduce variant stays within 64 VGPRs, and the GEMM
  variants within the budgets that let a sync workgroup share a CU with them;
- no packed-fp32 instructions (the build disables them) and no scalar-cache
  stores anywhere.
"""
import os
import re
import subprocess
import tempfile

import pytest

from gradient_sync_amd import _build as B

SOURCES = ["sync_kernels.hip", "odc_kernels.hip", "gemm_bf16.hip", "gemm_f32.hip", "fsdp_kernels.hip"]


@pytest.fixture(scope="module")
def kernels():
    """{kernel symbol: (descriptor text, body text)} over all sources."""
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in SOURCES:
            asm = os.path.join(tmp, src + ".s")
            cmd = [B.HIPCC, *B.FLAGS, "-I", B.CSRC, "-I", os.path.join(B.ROOT, "include"),
                   "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", asm]
            procs.append((asm, subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                                stderr=subprocess.DEVNULL)))
        for asm, p in procs:
            assert p.wait() == 0, f"hipcc failed for {asm}"
            text = open(asm).read()
            for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
                name = m.group(1)
                start = re.search(r"^" + re.escape(name) + r":", text, re.M).start()
                end = text.index(".Lfunc_end", start)
                out[name] = (m.group(2), text[start:end])
    assert len(out) > 50
    return out


def field(desc, key):
    return int(re.search(r"\." + key + r" (\d+)", desc).group(1))


def pick(kernels, *parts):
    found = {n: v for n, v in kernels.items() if all(p in n for p in parts)}
    assert found, parts
    return found


def test_no_scratch(kernels):
    for name, (desc, _) in kernels.items():
        assert field(desc, "amdhsa_private_segment_fixed_size") == 0, name


def test_sync_kernels_use_16_byte_accesses(kernels):
    for parts in (("rs_kernelILi1ELi1ELi8ELi1ELb0",), ("rs_kernelILi1ELi1ELi8ELi1ELb1",),
                  ("ag_kernelILi2ELi8ELi1",), ("rsag_kernelILi1ELi1ELi8",),
                  ("scatter_accumulate_kernelILi1",)):
        for name, (_, body) in pick(kernels, *parts).items():
            assert "global_load_dwordx4" in body, name
            assert "global_store_dwordx4" in body, name


def test_register_budgets(kernels):
    for name, (desc, _) in pick(kernels, "rs_kernel_lean").items():
        assert field(desc, "amdhsa_next_free_vgpr") <= 64, name
    # two waves per SIMD of the default GEMM leave 512 - 2*224 = 64 registers:
    # room for one lean sync wave
    for name, (desc, _) in pick(kernels, "gemm_bf16_kernelILb0ELi64").items():
        assert field(desc, "amdhsa_next_free_vgpr") <= 224, name
    # the 4-wave GEMM: 256 accumulators in the accumulation registers, the
    # rest within the 256 architectural VGPRs (one wave per SIMD)
    for name, (desc, _) in list(pick(kernels, "gemm_bf16_w4_kernel").items()) + \
            list(pick(kernels, "gemm_bf16_w4d_kernel").items()) + \
            list(pick(kernels, "gemm_bf16_w4dn_kernel").items()):
        acc0, nfree = field(desc, "amdhsa_accum_offset"), field(desc, "amdhsa_next_free_vgpr")
        assert acc0 <= 256 and nfree - acc0 >= 256 and nfree <= 512, name
    # the FSDP step kernels: 8 waves per workgroup, two per SIMD (<= 256 each)
    for name, (desc, _) in list(pick(kernels, "fsdp_step_k8_kernel").items()) + \
            list(pick(kernels, "fsdp_step2_kernel").items()):
        assert field(desc, "amdhsa_next_free_vgpr") <= 256, name
    # the CU-sharing GEMM leaves room for one default sync wave (<= 96)
    sync = max(field(d, "amdhsa_next_free_vgpr")
               for d, _ in pick(kernels, "rs_kernelILi1ELi1ELi8ELi1").values())
    for name, (desc, _) in pick(kernels, "gemm_bf16_kernelILb0ELi32").items():
        assert 2 * field(desc, "amdhsa_next_free_vgpr") + sync <= 512, name


def test_no_packed_fp32_and_no_scalar_stores(kernels):
    banned = re.compile(r"\b(v_pk_(add|mul|fma)_f32|s_store_|s_buffer_store|s_atomic_|"
                        r"s_buffer_atomic|s_dcache_wb|s_dcache_discard)")
    for name, (_, body) in kernels.items():
        m = banned.search(body)
        assert m is None, (name, m.group(0) if m else None)


def _stores(body):
    return re.findall(r"^\s*global_store_dwordx4 [^\n]*", body, re.M)


def _loads(body):
    return re.findall(r"^\s*global_load_dwordx4 [^\n]*", body, re.M)


def test_cache_hints_reach_the_code(kernels):
    """The nontemporal hints the sync kernels choose are in the compiled code:
    a standalone ReduceScatter streams its inputs and stores its shards
    nontemporally, the variant for shards an AllGather reads next stores them
    with ordinary stores, the AllGather stores its outputs nontemporally. (A
    store kind chosen by a run-time flag inside the kernel was once merged by
    the compiler into one ordinary store; the kinds are template parameters.)"""
    nt = re.compile(r"\bnt\b")
    # bf16, avg by x1/8, K = 8, one vector per lane, not AllReduce
    for name, (_, body) in pick(kernels, "rs_kernelILi1ELi1ELi8ELi1ELb0ELb0E").items():
        assert _stores(body) and all(nt.search(s) for s in _stores(body)), name
        assert _loads(body) and all(nt.search(s) for s in _loads(body)), name
    for name, (_, body) in pick(kernels, "rs_kernelILi1ELi1ELi8ELi1ELb0ELb1E").items():
        assert _stores(body) and not any(nt.search(s) for s in _stores(body)), name
        assert _loads(body) and all(nt.search(s) for s in _loads(body)), name
    for name, (_, body) in pick(kernels, "ag_kernelILi2ELi8ELi1E").items():
        assert _stores(body) and all(nt.search(s) for s in _stores(body)), name
    # the fused launch: ordinary shard stores (ReduceScatter half) beside
    # nontemporal output stores (AllGather half)
    for name, (_, body) in pick(kernels, "rsag_kernelILi1ELi1ELi8E").items():
        st = _stores(body)
        assert any(nt.search(s) for s in st) and not all(nt.search(s) for s in st), name
    # the FSDP step of the compile-time sizes: every output store is a
    # nontemporal 16-byte store (y, the W copies, dw_full, dw_shard)
    for name, (_, body) in pick(kernels, "fsdp_step_k8_kernel").items():
        st = _stores(body)
        assert len(st) >= 4 and all(nt.search(x) for x in st), name
        assert not re.search(r"^\s*(global|buffer)_store_dword\b", body, re.M), name


def _loop_body(body):
    """The instructions of the innermost loop (the block the compiler marks as
    the loop header, up to the next label)."""
    lines = body.splitlines()
    start = next(i for i, ln in enumerate(lines) if "Inner Loop Header" in ln)
    end = next(i for i in range(start + 1, len(lines)) if re.match(r"^\.LBB\d+_\d+:", lines[i]))
    return "\n".join(lines[start:end])


def test_direct_to_lds_gemm_loops(kernels):
    """The main loops of both direct-to-LDS GEMM kernels keep every
    accumulator in place (no accumulation-register moves inside the loop);
    the kernel for B stored [k, n] assembles B's fragments with transposing LDS
    reads, runs 16x16x32 MFMAs, waits for its LDS reads only where its own
    waits stand (15 per stage) and for the loads in flight only at its
    barriers, and reads no accumulator after the loop before the fence that
    waits out the last MFMAs (the compiler sees neither, they are inline asm)."""
    for parts in (("gemm_bf16_w4d_kernel",), ("gemm_bf16_w4dn_kernel",)):
        for name, (_, body) in pick(kernels, *parts).items():
            loop = _loop_body(body)
            assert re.search(r"\bv_mfma_", loop), name
            assert not re.search(r"\bv_accvgpr_(mov|write|read)", loop), name
    for name, (_, body) in pick(kernels, "gemm_bf16_w4dn_kernel").items():
        loop = _loop_body(body)
        assert len(re.findall(r"\bds_read_b64_tr_b16\b", loop)) == 64, name
        assert len(re.findall(r"\bv_mfma_f32_16x16x32_bf16\b", loop)) == 256, name
        assert len(re.findall(r"s_waitcnt vmcnt\(0\)", loop)) == 2, name
        assert len(re.findall(r"s_waitcnt lgkmcnt\(\d+\)", loop)) == 30, name
        # the inline LDS reads' results go straight into the MFMA operand
        # registers: no vector instruction in the loop but the MFMAs (a copy
        # of a read's result would read it before it lands, and free its
        # register while the read is still in flight)
        valu = [m for m in re.findall(r"^\s*(v_\w+)", loop, re.M) if not m.startswith("v_mfma_")]
        assert not valu, (name, sorted(set(valu)))
        tail = body[body.index(loop) + len(loop):]
        first_read = re.search(r"\bv_accvgpr_read_b32\b", tail).start()
        assert tail.rfind("s_nop 7", 0, first_read) > tail.rfind("v_mfma", 0, first_read), name
