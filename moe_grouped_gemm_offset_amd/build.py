"""Builds libgg_moe.so (the HIP library) in-tree for gfx950, and beside it
libgg_peak.so (the MFMA rate probe the benchmark loads).

Each translation unit under csrc/ is compiled by hipcc in parallel into
_build/, then linked into moe_grouped_gemm_offset_amd/libgg_moe.so.  No GPU is
needed: hipcc cross-compiles the gfx950 code objects.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgg_moe.so")
PEAK_LIB = os.path.join(HERE, "libgg_peak.so")
PEAK_SOURCE = ("gg_peak.hip", "gg_peak", [])
# (source, object name, defines): the instantiation sources are compiled
# once per kernel family member (activation, B major), in parallel
SOURCES = [(f, os.path.splitext(f)[0], []) for f in
           ("gg_api.cpp", "gg_prologue.hip", "gg_wgrad.hip", "gg_wgrad_mx.hip", "gg_dglu.hip",
            "gg_dglu_mx.hip", "gg_dsrelu.hip")]
SOURCES += [("gg_dglu_mx_inst.hip", f"gg_dglu_mx_a{act}{'k' if bk else 'n'}",
             [f"-DGG_ACT={act}", f"-DGG_BK={bk}"]) for act in range(3) for bk in (1, 0)]
SOURCES += [("gg_dsrelu_inst.hip", f"gg_dsrelu_{'k' if bk else 'n'}", [f"-DGG_BK={bk}"])
            for bk in (1, 0)]
ARCH = os.environ.get("GG_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgg_moe)")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # no packed-fp32 instructions anywhere in this library
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # the fused epilogues walk every accumulator register with
            # compile-time indices; without a higher limit LLVM leaves the
            # loop rolled and demotes the accumulators to scratch memory
            "-mllvm", "-pragma-unroll-threshold=1000000",
            # buffers are reinterpreted (bf16/fp8 bytes as 32-bit words, LDS
            # staging written as floats and read as vectors): no type-based
            # alias assumptions
            "-fno-strict-aliasing",
            # atomics stay as written: every atomic here is issued by one
            # lane or hits per-lane addresses, so the rewrite into a
            # wave-wide scan buys nothing, and it awaits the returned value
            # where the rewrite ends (the wgrad kernel's queue request must
            # stay in flight through half of an epilogue)
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(entry):
    src, name, defines = entry
    obj = os.path.join(BUILD, name + ".o")
    cmd = [hipcc(), *flags(), *defines, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs=None):
    """Compile every source, link libgg_moe.so and libgg_peak.so; returns the
    path of libgg_moe.so."""
    os.makedirs(BUILD, exist_ok=True)
    entries = SOURCES + [PEAK_SOURCE]
    jobs = jobs or min(len(entries), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, entries))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
