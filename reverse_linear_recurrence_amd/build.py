"""Build librlca.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m reverse_linear_recurrence_amd.build

hipcc cross-compiles without a GPU.  The library lands next to this file, where
the Python binding loads it.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librlca.so")
# The instrumented build: the same sources with RLCA_TIMESTAMPS defined, so
# that the scan kernels record per-wavefront wall-clock stamps (a measurement
# tool for bench.py; never loaded by default).
LIB_TIMED = os.path.join(PKG, "librlca_timed.so")
# A measurement tool beside the library (not part of it): the streaming
# ceiling of a workload's byte mix, timed by bench.py.
CEILING_SRC = os.path.join(CSRC, "stream_ceiling.hip")
LIB_CEILING = os.path.join(PKG, "libstream_ceiling.so")
# Host code and the kernel tables, compiled in parallel.
SOURCES = [os.path.join(CSRC, n) for n in ("rlca.hip", "kernels_plain.hip", "kernels_window.hip",
                                           "kernels_chain.hip", "kernels_probs.hip",
                                           "kernels_materialized.hip")]
DEPS = SOURCES + [os.path.join(CSRC, n) for n in ("scan_kernels.hpp", "kernel_table.hpp",
                                                   "variants.hpp", "probs_kernels.hpp",
                                                   "materialized.hpp")] + [
    os.path.join(INCLUDE, "rlca.h")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def compile_command(src, obj, timestamps=False):
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-c"] + (
        ["-DRLCA_TIMESTAMPS"] if timestamps else []) + [
            # Packed fp32 ops (v_pk_*_f32) stay off: plain scalar fp32 only.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Leading scalar kernel arguments are preloaded into SGPRs.
            "-mllvm", "-amdgpu-kernarg-preload-count=16",
            # Host code: a stack guard after local arrays, so that a write past
            # an argument table aborts (in the CPU tests) instead of corrupting
            # the caller's stack.
            "-Xarch_host", "-fstack-protector-strong",
            "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC, src, "-o", obj]


def link_command(objs, out):
    return [hipcc(), "--offload-arch=" + ARCH, "-fPIC", "-shared"] + objs + ["-o", out]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l)
    return res.returncode, out


def up_to_date():
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(d) <= t for d in DEPS)


def build(verbose=False, timestamps=False):
    """Compile librlca.so (always; with timestamps, librlca_timed.so) and
    return its path."""
    target = LIB_TIMED if timestamps else LIB
    tag = ".tmp%d%s" % (os.getpid(), "t" if timestamps else "")
    objs = [os.path.join(PKG, os.path.basename(src).replace(".hip", tag + ".o")) for src in SOURCES]
    cmds = [compile_command(src, obj, timestamps) for src, obj in zip(SOURCES, objs)]
    tmp = target + tag
    try:
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, out), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s (%d):\n%s" % (src, rc, out))
            if verbose and out.strip():
                print(out)
        rc, out = _run(link_command(objs, tmp))
        if rc != 0:
            raise RuntimeError("hipcc link failed (%d):\n%s" % (rc, out))
        os.replace(tmp, target)
    finally:
        for f in objs + [tmp]:
            if os.path.exists(f):
                os.remove(f)
    return target


def build_ceiling(verbose=False):
    """Compile libstream_ceiling.so (bench.py's streaming-ceiling leg) and
    return its path."""
    tmp = LIB_CEILING + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wextra",
           CEILING_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        rc, out = _run(cmd)
        if rc != 0:
            raise RuntimeError("hipcc failed on %s (%d):\n%s" % (CEILING_SRC, rc, out))
        os.replace(tmp, LIB_CEILING)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB_CEILING


if __name__ == "__main__":
    if "--ceiling" in sys.argv[1:]:
        print(build_ceiling(verbose=True))
    else:
        print(build(verbose=True, timestamps="--timestamps" in sys.argv[1:]))
    sys.exit(0)
