"""Properties of the generated gfx950 code, checked on the CPU (hipcc
cross-compiles): every translation unit of the library is compiled to device
assembly with the library's own flags, and the assembly must hold

* no packed fp32 instructions (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32...):
  the build turns the feature off, and hand-written code must not use them;
* no scalar-cache stores or atomics: device code writes through vector
  stores only;
* no scratch (private segment) use in any kernel: every instance stays in
  registers;
* the chained instances hold as many workgroups per compute unit as the
  split calls' plan assumes (split_rules.residency, up to 2).
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from reverse_linear_recurrence_amd import build as B
from split_rules import residency

HIPCC = B.hipcc()
pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")

SCALAR_WRITES = re.compile(r"^\s*(s_store_|s_buffer_store|s_scratch_store|s_atomic|s_buffer_atomic|"
                           r"s_dcache_wb|s_dcache_discard)", re.M)
PACKED_FP32 = re.compile(r"^\s*v_pk_\w+_f32\b", re.M)


def device_asm(src, out):
    cmd = B.compile_command(src, out)
    cmd = [c for c in cmd if c not in ("-c", "-fPIC")]
    cmd[cmd.index("-o"):cmd.index("-o")] = ["-S", "--cuda-device-only"]
    rc, msg = B._run(cmd)
    assert rc == 0, msg
    return open(out).read()


@pytest.fixture(scope="module")
def assembly():
    tmp = tempfile.mkdtemp(prefix="rlca_asm_")
    try:
        outs = [os.path.join(tmp, os.path.basename(s) + ".s") for s in B.SOURCES]
        with ThreadPoolExecutor(len(B.SOURCES)) as ex:
            texts = list(ex.map(device_asm, B.SOURCES, outs))
        yield dict(zip((os.path.basename(s) for s in B.SOURCES), texts))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_no_packed_fp32_instructions(assembly):
    for name, text in assembly.items():
        assert not PACKED_FP32.search(text), name


def test_no_scalar_cache_writes(assembly):
    for name, text in assembly.items():
        hit = SCALAR_WRITES.search(text)
        assert hit is None, (name, hit and hit.group(0))


def test_no_kernel_uses_scratch(assembly):
    kernels = 0
    for name, text in assembly.items():
        for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
            kernels += 1
            size = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2)).group(1))
            assert size == 0, (name, m.group(1), size)
    assert kernels >= 400  # the scan, window and policy-table instances


# scan_kernel<A, InT, K, LPR, WPR, kUniform, kChunk, kTiles, kAligned, kChain>,
# mangled: InT is t (uint16_t, bf16 bits) or f (float).
SCAN_KERNEL = re.compile(r"_ZN4rlca11scan_kernelILi(\d+)E([tf])Li(\d+)ELi(\d+)ELi(\d+)ELb([01])E"
                         r"Lb([01])ELi(\d+)ELb([01])ELb([01])EE")
ALGO_NAMES = ["returns", "gae", "td_lambda", "vtrace", "retrace", "eligibility", "cumsum",
              "affine", "affine"]


def test_chained_residency_matches_the_compiled_code(assembly):
    # Workgroups of W wavefronts resident on one CU: VGPRs are allocated in
    # granules of 8 out of 512 per SIMD lane, at most 8 wavefronts per SIMD,
    # the workgroup's wavefronts spread over the CU's 4 SIMDs; LDS: 160 KiB.
    checked = 0
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel",
                         assembly["kernels_chain.hip"], re.S):
        k = SCAN_KERNEL.match(m.group(1))
        if k is None or k.group(10) != "1":
            continue
        algo, bf16 = ALGO_NAMES[int(k.group(1))], k.group(2) == "t"
        K, waves, tiles = int(k.group(3)), int(k.group(5)), int(k.group(8))
        vgprs = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", m.group(2)).group(1))
        lds = int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", m.group(2)).group(1))
        per_simd = min(8, 512 // (-(-vgprs // 8) * 8))
        held = min(per_simd // (waves // 4), (160 << 10) // max(lds, 1))
        assert held >= 1, (m.group(1), vgprs, lds)
        assert min(2, held) == residency(algo, K, waves, tiles, bf16), (
            algo, "bf16" if bf16 else "f32", K, waves, tiles, vgprs, lds)
        checked += 1
    assert checked >= 150  # every chained instance
