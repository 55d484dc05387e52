"""Properties of the generated gfx950 code, checked on the CPU (hipcc
cross-compiles): every translation unit of the library is compiled to device
assembly with the library's own flags, and the assembly must hold

* no packed fp32 instructions (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32...):
  the build turns the feature off, and hand-written code must not use them;
* no scalar-cache stores or atomics: device code writes through vector
  stores only;
* no scratch (private segment) use in any kernel: every instance stays in
  registers.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from reverse_linear_recurrence_amd import build as B

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
