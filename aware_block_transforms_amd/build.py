"""Build libwush.so in-tree: HIP kernels for gfx950 plus the host-side builder.

Usage:  python -m aware_block_transforms_amd.build   (or build() from Python)

Every HIP source is compiled with
  * --offload-arch=gfx950 (CDNA4 only; no other targets, no CUDA path),
  * -ffp-contract=off (no implicit FMA contraction: the transform's FMA chain
    is written with explicit fmaf and nothing else may be fused),
  * packed fp32 ops disabled for the device (v_pk_*_f32 are never emitted).
The host builder (fp64 Cholesky / Jacobi) is plain C++17 compiled by g++.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libwush.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

HIP_SOURCES = ["transform_quant.hip", "gemm_mxfp4.hip", "gemm_nv_int4.hip", "gemm_nvfp4.hip", "gemm_int4.hip", "gemm.hip", "loss.hip", "had256.hip", "moments.hip", "builder_dev.hip"]
# matrix-core ceiling probes for bench.py: their own library, none of the method's arithmetic
CEILING_SOURCE = "ceiling.hip"
CEILING_LIB = os.path.join(PKG, "libwush_ceiling.so")
CXX_SOURCES = ["builder.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", f"-I{INCLUDE}"]
# per-source extras: the transform kernels read each MFMA result with the
# vector ALU right away, so their accumulators live in ordinary VGPRs (in
# AGPRs every value would cost a v_accvgpr_read first)
HIP_EXTRA = {"transform_quant.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    # keep real warnings visible, drop the host-pass note about the device-only feature flag
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    return msg


def build(verbose=False):
    """Compile every source and link libwush.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *HIP_EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj])
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for msg in ex.map(_run, jobs):
            if msg and verbose:
                print(msg)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"])
    os.replace(tmp, LIB)
    tmp = CEILING_LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, CEILING_SOURCE)])
    os.replace(tmp, CEILING_LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
