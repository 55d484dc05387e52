"""Build librlca.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m reverse_linear_recurrence_amd.build

hipcc cross-compiles without a GPU.  The library lands next to this file, where
the Python binding loads it.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librlca.so")
SOURCES = [os.path.join(CSRC, "rlca.hip")]
DEPS = SOURCES + [os.path.join(CSRC, "scan_kernels.hpp"), os.path.join(INCLUDE, "rlca.h")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build_command(out):
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            # Packed fp32 ops (v_pk_*_f32) stay off: plain scalar fp32 only.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Leading scalar kernel arguments are preloaded into SGPRs.
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC] + SOURCES + ["-o", out]


def up_to_date():
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(d) <= t for d in DEPS)


def build(verbose=False):
    """Compile librlca.so (always) and return its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = build_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
