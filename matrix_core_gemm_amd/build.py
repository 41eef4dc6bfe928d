"""Build the gfx950 HIP library in-tree: matrix_core_gemm_amd/_libmcg.so.

Every source is compiled by hipcc for gfx950 only; objects go to
matrix_core_gemm_amd/_build/ and are linked into one shared library that the
Python binding loads with ctypes.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "_libmcg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gemm_dense.hip", "gemm_skinny_n.hip", "gemm_skinny_m.hip", "gemm_stream.hip", "gemm_fast.hip", "gemm_fast_mid.hip", "gemm_fast_sk.hip", "gemm_fast_mid_sk.hip", "gemm_sparse.hip",
           "gemm_sparse_fast.hip", "gemm_f64.hip", "numerics.hip", "mfma_probe.hip", "api.cpp"]
HEADERS = ["arch_gfx950.hpp", "frag_layout.hpp", "tile_io.hpp", "fast_tiles.hpp", "tile_order.hpp", "gemm_fast_kernel.hpp", "gemm_kernels.hpp", "dense_general.hpp", "sparse_ops.hpp"]

# Packed fp32 VALU forms are disabled for all device code (hipcc's host pass
# reports the feature as unknown, which is harmless).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


# Per-file device flags.  The binary64 kernel keeps its MFMA accumulators in VGPRs:
# with the default AGPR form the compiler copies them between register files around
# the K loop, which costs a third of the FP64 matrix rate.  (The other kernels were
# measured both ways: the VGPR form gains nothing there.)
EXTRA = {"gemm_f64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _needs(obj: str, src: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [src] + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(HERE, "..", "include", "mcg.h")]
    return any(os.path.getmtime(d) > t for d in deps if os.path.exists(d))


def build(force: bool = True, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s + ".o")
        objs.append(obj)
        if force or _needs(obj, src):
            cmd = [HIPCC, *COMMON, *EXTRA.get(s, []), "-c", src, "-o", obj]
            if s.endswith(".hip"):
                cmd[1:1] = ["-x", "hip"]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # drop the known-harmless host-pass feature warning
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((s, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for s, text in failed:
            sys.stderr.write(f"--- {s} ---\n{text}\n")
        raise RuntimeError("HIP build failed: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv, verbose=True))
