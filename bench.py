"""Benchmark of the matrix-core GEMM hot path on one MI355X.

One timed step is one pass over every entry point of the hot path on its
full-size synthetic workload (8192^3 for every GEMM):
  gemm_dense  bf16 x bf16 -> f32   (A row-major, B column-major, C ~ N(0,1), alpha = beta = 1)
  gemm_dense  f16  x f16  -> f32   (same recipe)
  gemm_dense  i8   x i8   -> i32   (C uniform int in [-2^20, 2^20], alpha = beta = 1)
  gemm_dense  e4m3 x e4m3 -> f32   (per-tensor scales, C = 0)
  gemm_dense  e4m3 x e5m2 -> f32   (per-tensor scales, C = 0)
  compress24  bf16 8192 x 8192     (2:4 compressor)
  gemm_sparse24 bf16 (2:4 A) x bf16 -> f32
  gemm_dense  bf16 x bf16 -> bf16  (C and D in bfloat16, alpha = beta = 1)
  gemm_dense  skinny bf16 32768 x 16 x 8192 and 16 x 32768 x 8192 (C absent): HBM-bound
  gemm_sparse24 int8 (2:4 A) x int8 -> i32 and e4m3 (2:4 A) x e4m3 -> f32 (C absent)
  gemm_dense  f64  x f64  -> f64   (binary64, A row-major, B column-major, C ~ N(0,1), alpha = beta = 1)
Each call is bracketed by HIP events on the stream it is launched on, so every
kernel's average duration is measured live.  `value` is the dense bf16 8192^3
rate (TFLOP/s); the per-dtype rates the metric asks for are in `per_dtype`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (TOPS int8) at 8192³ per dtype + % of MI355X MFMA peak"
# MI355X published dense peaks (TFLOP/s or TOPS) and HBM bandwidth (GB/s)
PEAK = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "i8": 5000.0, "f64": 78.6}
HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the dense bf16 8192^3 kernel, from two rocprofv3 --pmc
# passes (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000; the factors make a plain 1 GiB
# copy kernel read as 1 GiB).  Valid only for the kernel sources they were taken
# with (the kernel's files and its argument block): when their hash differs,
# traffic is reported as null.
KERNEL_SOURCES = ("gemm_fast_kernel.hpp", "gemm_fast.hip", "fast_tiles.hpp", "arch_gfx950.hpp")
TRAFFIC_MEASURED = {
    "sources_sha256": "1890032682344e3f9d2e464b54dc92cbbe82a1053e3b3e73c6cde3f500027891",
    "read_bytes": 1810 * 2**20, "write_bytes": 256 * 2**20,
}


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "matrix_core_gemm_amd", "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    # the DenseArgs block of the shared header (the rest of it declares other kernels)
    text = open(os.path.join(csrc, "gemm_kernels.hpp"), "rb").read()
    start = text.index(b"struct DenseArgs {")
    h.update(text[start:text.index(b"};", start) + 2])
    return h.hexdigest()


def measured_traffic():
    if kernel_sources_hash() != TRAFFIC_MEASURED["sources_sha256"]:
        return None
    return TRAFFIC_MEASURED["read_bytes"] + TRAFFIC_MEASURED["write_bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--size", type=int, default=8192)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", default="", help="comma list of entries to run (profiling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import matrix_core_gemm_amd as mcg
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    n = args.size
    M = N = K = n
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    t0 = time.time()
    log(f"generating inputs (n = {n}) ...")
    ops = {}
    for dt in ("bf16", "f16"):
        A = W.operand("A", dt, M, K, "normal", "k_contig")
        B = W.operand("B", dt, K, N, "normal", "k_contig")
        ops[dt] = (dev(A.codes), A.ld, dev(B.codes), B.ld, 1.0, 1.0)
        if dt == "bf16":
            host_bf16 = (A, B)
    C = dev(W.c_matrix(M, N, "normal"))
    Ci = dev(W.c_matrix(M, N, "int20"))
    A = W.operand("A", "i8", M, K, "int8", "k_contig")
    B = W.operand("B", "i8", K, N, "int8", "k_contig")
    ops["i8"] = (dev(A.codes), A.ld, dev(B.codes), B.ld, 1.0, 1.0)
    A8 = W.operand("A", "e4m3", M, K, "normal", "k_contig", fp8_scaled=True)
    B8 = W.operand("B", "e4m3", K, N, "normal", "k_contig", fp8_scaled=True)
    B85 = W.operand("B", "e5m2", K, N, "normal", "k_contig", fp8_scaled=True)
    dA8 = dev(A8.codes)
    ops["e4m3xe4m3"] = (dA8, A8.ld, dev(B8.codes), B8.ld, A8.scale, B8.scale)
    ops["e4m3xe5m2"] = (dA8, A8.ld, dev(B85.codes), B85.ld, A8.scale, B85.scale)
    As = dev(W.sparse24_dense("bf16", M, K))
    Bs = ops["bf16"][2]
    vals = torch.empty((M, K // 2), dtype=torch.int16, device="cuda")
    idx = torch.empty((M, (K + 31) // 32), dtype=torch.int32, device="cuda")
    # 8-bit 2:4 operands, compressed on the device before timing
    sp8 = {}
    for dt, B_ in (("i8", ops["i8"][2]), ("e4m3", ops["e4m3xe4m3"][2])):
        A_ = dev(W.sparse24_dense(dt, M, K, dist="int8" if dt == "i8" else "normal"))
        v_ = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
        i_ = torch.empty((M, (K + 31) // 32), dtype=torch.int32, device="cuda")
        mcg.compress24(dt, M, K, A_, K, v_, K // 2, i_, i_.shape[1], None)
        del A_
        sp8[dt] = (v_, i_, B_)
    D = torch.empty((M, N), dtype=torch.float32, device="cuda")
    Di = torch.empty((M, N), dtype=torch.int32, device="cuda")
    # bfloat16 C and D for the 16-bit output entry
    C16 = C.to(torch.bfloat16).view(torch.int16)
    D16 = torch.empty((M, N), dtype=torch.int16, device="cuda")
    # skinny problems: the wide operand (4n x n bf16 ~ N(0,1)) drawn on the device
    SK = (4 * n, 16)
    g = torch.Generator(device="cuda").manual_seed(W.SEED_A)
    Wide = torch.randn((SK[0], K), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    Narrow = torch.randn((SK[1], K), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    Dsk = torch.empty((SK[0], SK[1]), dtype=torch.float32, device="cuda")
    # binary64 operands ~ N(0,1), drawn on the device
    A64 = torch.randn((M, K), generator=g, dtype=torch.float64, device="cuda")
    B64 = torch.randn((N, K), generator=g, dtype=torch.float64, device="cuda")  # column-major K x N
    C64 = torch.randn((M, N), generator=g, dtype=torch.float64, device="cuda")
    D64 = torch.empty((M, N), dtype=torch.float64, device="cuda")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream()
    s = stream.cuda_stream

    def call(name):
        if name in ("bf16", "f16"):
            a, lda, b, ldb, sa, sb = ops[name]
            mcg.gemm_dense(name, name, 0, 0, M, N, K, a, lda, b, ldb, C, D, N, "f32", 1.0, 1.0,
                           stream=s)
        elif name == "i8":
            a, lda, b, ldb, sa, sb = ops[name]
            mcg.gemm_dense("i8", "i8", 0, 0, M, N, K, a, lda, b, ldb, Ci, Di, N, "i32", 1, 1, stream=s)
        elif name.startswith("e4m3x"):
            a, lda, b, ldb, sa, sb = ops[name]
            mcg.gemm_dense("e4m3", name.split("x")[1], 0, 0, M, N, K, a, lda, b, ldb, None, D, N, "f32",
                           1.0, 0.0, sa, sb, stream=s)
        elif name == "compress24":
            mcg.compress24("bf16", M, K, As, K, vals, K // 2, idx, idx.shape[1], None, stream=s)
        elif name == "sparse24":
            mcg.gemm_sparse24("bf16", "bf16", 0, M, N, K, vals, K // 2, idx, idx.shape[1], Bs, K, None,
                              D, N, "f32", 1.0, 0.0, stream=s)
        elif name == "sparse24_i8":
            v_, i_, B_ = sp8["i8"]
            mcg.gemm_sparse24("i8", "i8", 0, M, N, K, v_, K // 2, i_, i_.shape[1], B_, K, None, Di, N,
                              "i32", 1, 0, stream=s)
        elif name == "sparse24_e4m3":
            v_, i_, B_ = sp8["e4m3"]
            mcg.gemm_sparse24("e4m3", "e4m3", 0, M, N, K, v_, K // 2, i_, i_.shape[1], B_, K, None, D, N,
                              "f32", B8.scale, 0.0, stream=s)
        elif name == "bf16_out":
            a, lda, b, ldb, sa, sb = ops["bf16"]
            mcg.gemm_dense("bf16", "bf16", 0, 0, M, N, K, a, lda, b, ldb, C16, D16, N, "bf16", 1.0, 1.0,
                           stream=s)
        elif name == "skinny_n16":  # A = Wide (M = 4n), B = Narrow (N = 16, column-major)
            mcg.gemm_dense("bf16", "bf16", 0, 0, SK[0], SK[1], K, Wide, K, Narrow, K, None, Dsk, SK[1],
                           "f32", 1.0, 0.0, stream=s)
        elif name == "f64":
            mcg.gemm_dense("f64", "f64", 0, 0, M, N, K, A64, K, B64, K, C64, D64, N, "f64", 1.0, 1.0, stream=s)
        elif name == "skinny_m16":  # A = Narrow (M = 16), B = Wide (N = 4n, column-major)
            mcg.gemm_dense("bf16", "bf16", 0, 0, SK[1], SK[0], K, Narrow, K, Wide, K, None, Dsk, SK[0],
                           "f32", 1.0, 0.0, stream=s)

    names = ["bf16", "f16", "i8", "e4m3xe4m3", "e4m3xe5m2", "compress24", "sparse24", "bf16_out",
             "skinny_n16", "skinny_m16", "sparse24_i8", "sparse24_e4m3", "f64"]
    if args.only:
        keep = set(args.only.split(","))
        names = [x for x in names if x in keep or x == "compress24" and "sparse24" in keep]
    ev = {x: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for x in names}

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for x in names:
                call(x)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for step in range(args.steps):
            for x in names:
                ev[x][step][0].record(stream)
                call(x)
                ev[x][step][1].record(stream)
        torch.cuda.synchronize()
        t_end = time.perf_counter()

    ms = {x: float(np.mean([a.elapsed_time(b) for a, b in ev[x]])) for x in names}
    flops = 2.0 * M * N * K
    per = {}
    for x in names:
        t = ms[x] * 1e-3
        if x == "compress24":
            nbytes = M * K * 2 + M * K // 2 * 2 + M * ((K + 31) // 32) * 4
            per[x] = {"GB/s": nbytes / t / 1e9, "ms": ms[x], "frac_of_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBS,
                      "bytes": nbytes}
        elif x.startswith("skinny"):
            nbytes = SK[0] * K * 2 + SK[1] * K * 2 + SK[0] * SK[1] * 4
            shape = (SK[0], SK[1], K) if x == "skinny_n16" else (SK[1], SK[0], K)
            per[x] = {"GB/s": nbytes / t / 1e9, "ms": ms[x], "frac_of_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBS,
                      "bytes": nbytes, "TFLOP/s": 2.0 * SK[0] * SK[1] * K / t / 1e12, "MxNxK": shape}
        elif x == "bf16_out":
            tf = flops / t / 1e12
            per[x] = {"TFLOP/s": tf, "ms": ms[x], "peak": PEAK["bf16"], "frac_of_peak": tf / PEAK["bf16"]}
        elif x in ("sparse24_i8", "sparse24_e4m3"):
            tf = flops / t / 1e12
            dense = "i8" if x == "sparse24_i8" else "e4m3xe4m3"
            pk = PEAK["i8"] if x == "sparse24_i8" else PEAK["fp8"]
            u = "TOPS" if x == "sparse24_i8" else "TFLOP/s"
            per[x] = {f"{u}_dense_equiv": tf, f"{u}_algorithmic": tf / 2, "ms": ms[x],
                      "frac_of_dense_peak": tf / pk,
                      f"vs_dense_{dense}": tf / (flops / (ms[dense] * 1e-3) / 1e12) if dense in ms else None}
        elif x == "sparse24":
            tf = flops / t / 1e12
            per[x] = {"TFLOP/s_dense_equiv": tf, "TFLOP/s_algorithmic": tf / 2, "ms": ms[x],
                      "frac_of_dense_bf16_peak": tf / PEAK["bf16"],
                      "vs_dense_bf16": tf / (flops / (ms["bf16"] * 1e-3) / 1e12) if "bf16" in ms else None}
        else:
            pk = PEAK["fp8"] if x.startswith("e4m3") else PEAK[x]
            tf = flops / t / 1e12
            per[x] = {("TOPS" if x == "i8" else "TFLOP/s"): tf, "ms": ms[x], "peak": pk, "frac_of_peak": tf / pk}
    head = "bf16" if "bf16" in names else names[0]
    value = flops / (ms[head] * 1e-3) / 1e12 if head != "compress24" else per[head]["GB/s"]

    # CPU oracle baseline: whole rows of D of the bf16 workload, timed on the host cores
    cpu = None
    if not args.no_cpu:
        import oracle
        A, B = host_bf16
        nthr = oracle.max_threads()
        t1 = time.perf_counter()
        rows, cols = np.zeros(N, np.int64), np.arange(N, dtype=np.int64)
        oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes,
                          B.ld, rows=rows, cols=cols)
        one = time.perf_counter() - t1
        nrows = max(1, min(M, int(args.cpu_seconds / max(one, 1e-6))))
        rr = np.repeat(np.arange(nrows, dtype=np.int64) * (M // nrows), N)
        cc = np.tile(np.arange(N, dtype=np.int64), nrows)
        t1 = time.perf_counter()
        oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", M, N, K, A.codes, A.ld, B.codes,
                          B.ld, rows=rr, cols=cc)
        tcpu = time.perf_counter() - t1
        cpu = {"value": 2.0 * nrows * N * K / tcpu / 1e12, "unit": "TFLOP/s", "cores": nthr,
               "kind": "oracle",
               "sample": f"{nrows} whole rows ({nrows * N} outputs, K={K}) of the dense bf16 {n}^3 "
                         f"workload; {tcpu:.1f} s on {nthr} threads ({platform.processor() or 'host'})"}

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (t_end - t_start) * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"dense bf16 GEMM {n}x{n}x{n}, A row-major, B column-major, "
                               f"C ~ N(0,1) fp32, alpha=beta=1, fp32 out; step = all "
                               f"{len(names)} hot-path calls at {n}^3",
                   "M": M, "N": N, "K": K, "entries": names},
        "roofline": {"bound": "mfma", "achieved": value, "peak": PEAK["bf16"], "unit": "TFLOP/s",
                     "frac": value / PEAK["bf16"], "traffic": measured_traffic() if head == "bf16" and n == 8192 else None,
                     "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes": (2 * M * K + 2 * K * N + 8 * M * N),
                     "kernel": "mcg::fast::gemm_fast_kernel<BF16, 0, 0, 256> (256x256 tile, 8-wave ping-pong)", "kernel_ms": ms.get(head)},
        "cpu_baseline": cpu,
        "per_dtype": per,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
