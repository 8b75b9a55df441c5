"""Compile libpa.so (the gfx950 HIP kernels and their C ABI) in place.

    python -m paged_kv_cache_380_amd.build [--verbose]

Every ``csrc/*.hip`` file is compiled with hipcc and every host-only
``csrc/*.cpp`` file with the host C++ compiler to an object under ``_build/``
(in parallel); the objects are linked into ``paged_kv_cache_380_amd/libpa.so``.
The build always recompiles. Packed-FP32 instruction selection is turned off
for all device code.
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source additions. The matrix-core decode keeps its MFMA accumulators in
# ordinary VGPRs: with the default AGPR form the compiler copied all 32
# accumulators out of and back into AGPRs on every block.
FILE_FLAGS = {
    "pa_decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def cxx() -> str:
    return os.environ.get("CXX") or shutil.which("g++") or "c++"


def hipcc() -> str:
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(x for x in (r.stdout, r.stderr) if x)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected.
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    host_srcs = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))  # host-only C++ (no device code)
    objs = [os.path.join(BUILD, os.path.basename(s).rsplit(".", 1)[0] + ".o") for s in srcs + host_srcs]
    cmds = [[cc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(s), []), *extra_flags, "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    cmds += [[cxx(), *CXX_FLAGS, "-c", s, "-o", o] for s, o in zip(host_srcs, objs[len(srcs):])]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        futs = [ex.submit(_run, c, verbose) for c in cmds]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(verbose=args.verbose))
