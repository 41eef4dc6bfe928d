"""Benchmark of the matrix-core GEMM hot path on one MI355X.

One timed step is one pass over every entry point of the hot path on its
synthetic workload:
  gemm_dense  bf16 x bf16 -> f32, 8192^3, all four A/B storage orders
              (C ~ N(0,1), alpha = beta = 1); the A row-major / B column-major
              pair is the headline `value`
  gemm_dense  f16  x f16  -> f32, 8192^3, all four storage orders (same recipe)
  gemm_dense  bf16 x bf16 -> f32, 256^3, uniform[-1, 1], beta = 0 (launch-bound:
              one event pair brackets a batch of back-to-back launches)
  gemm_dense  i8   x i8   -> i32, 4096^3 and 8192^3 (C uniform int in
              [-2^20, 2^20], alpha = beta = 1)
  gemm_dense  e4m3 x e4m3 and e4m3 x e5m2 -> f32, 8192^3 (per-tensor scales, C = 0)
  compress24  bf16 8192 x 8192     (2:4 compressor)
  gemm_sparse24 bf16 / int8 / e4m3 (2:4 A), 8192^3, C absent
  gemm_dense  bf16 x bf16 -> bf16, 8192^3 (C and D in bfloat16)
  gemm_dense  skinny bf16 32768 x 16 x 8192 and 16 x 32768 x 8192 (HBM-bound)
  gemm_dense  f64  x f64  -> f64, 8192^3 (binary64, C ~ N(0,1))
  gemm_dense_ws bf16 7168^3, 6144^3, 5120^3, 1024 x 2048 x 8192, 1280 x 1280 x
              8192 (shapes whose last round of tiles is short: the stream-K form
              where the plan takes it; leading blocks of the 8192^2 operands)
  gemm_sparse24_ws bf16 2048 x 2048 x 8192 (the 2:4 stream-K form)
Each call (or batch) is bracketed by HIP events recorded on the stream it is
launched on, so every kernel's average duration is measured live.

After the timed steps every entry runs once more and sampled outputs (whole
rows and random elements) are compared with the CPU oracle, the same
acceptance test as the parity tests; the oracle is also timed per workload on
the host cores (the CPU baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only a,b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s (TOPS int8) at 8192³ per dtype + % of MI355X MFMA peak"
# MI355X published dense peaks (TFLOP/s or TOPS) and HBM bandwidth (GB/s); the
# 2:4 sparse instructions run at twice the dense rate of their input type
PEAK = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0, "i8": 5000.0, "f64": 78.6}
SPARSE_PEAK = {"bf16": 5000.0, "i8": 10000.0, "fp8": 10000.0}
HBM_PEAK_GBS = 8000.0
SMALL_BATCH = 50  # launches of the 256^3 workload per event pair (one HIP graph replay)

# HBM bytes per launch of the dense bf16 8192^3 kernel, from two rocprofv3 --pmc
# passes (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000; the factors make a plain 1 GiB
# copy kernel read as 1 GiB).  Valid only for the kernel sources they were taken
# with (the kernel's files and its argument block): when their hash differs,
# traffic is reported as null.
KERNEL_SOURCES = ("gemm_fast_kernel.hpp", "gemm_fast.hip", "fast_tiles.hpp", "tile_order.hpp", "arch_gfx950.hpp",
                  "frag_layout.hpp")
TRAFFIC_MEASURED = {
    "sources_sha256": "d2bd7e997c58ed70c470bffb29292b832d46764f0828d0e2ddab74c24619da70",
    "read_bytes": 1806 * 2**20, "write_bytes": 256 * 2**20,
}

LAYOUT_NAMES = {("k_contig", "k_contig"): "Arow_Bcol", ("k_contig", "mn_contig"): "Arow_Brow",
                ("mn_contig", "k_contig"): "Acol_Bcol", ("mn_contig", "mn_contig"): "Acol_Brow"}


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


def host_cpu():
    """CPU model name and socket count from /proc/cpuinfo."""
    model, sockets = "unknown", set()
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and model == "unknown":
                model = v
            elif k == "physical id":
                sockets.add(v)
    except OSError:
        pass
    return model, max(1, len(sockets))


class Entry:
    """One hot-path call: its arguments on the device and on the host (for the
    oracle), and how its rate is reported."""

    def __init__(self, name, kind, **kw):
        self.name, self.kind = name, kind
        self.__dict__.update(kw)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-parity", action="store_true", help="skip the sampled oracle comparison")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time for the headline workload's CPU baseline (others: a fifth)")
    ap.add_argument("--only", default="", help="comma list of entries to run (profiling)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the matrix-core rate probe on each entry's operand bits")
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
    n = 8192
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    only = set(args.only.split(",")) if args.only else None
    want = lambda x: only is None or x in only

    t0 = time.time()
    log("generating inputs ...")
    E = {}
    C_h = W.c_matrix(n, n, "normal")
    C = dev(C_h)
    D = torch.empty((n, n), dtype=torch.float32, device="cuda")
    Di = torch.empty((n, n), dtype=torch.int32, device="cuda")

    # dense bf16 / f16, 8192^3, the four storage orders.  The same N(0,1) buffers
    # serve every order (M = N = K): read column-major they are another N(0,1)
    # matrix of the same shape.
    for dt in ("bf16", "f16"):
        A = W.operand("A", dt, n, n, "normal", "k_contig")
        B = W.operand("B", dt, n, n, "normal", "k_contig")
        dA, dB = dev(A.codes), dev(B.codes)
        for lay, tag in LAYOUT_NAMES.items():
            name = dt if tag == "Arow_Bcol" else f"{dt}_{tag}"
            if want(name) or name == "bf16":
                E[name] = Entry(name, "dense", dtA=dt, dtB=dt, layA=lay[0], layB=lay[1], M=n, N=n, K=n,
                                A=dA, B=dB, hA=A.codes, hB=B.codes, lda=n, ldb=n, C=C, hC=C_h, D=D,
                                out="f32", alpha=1.0, beta=1.0, sA=1.0, sB=1.0, peak=PEAK[dt], unit="TFLOP/s")
    # shapes whose last round of tiles is short, on gemm_dense_ws (stream-K form
    # where the plan takes it): leading blocks of the 8192^2 bf16 operands
    # (lda = ldb = 8192), no C, binary32 D
    wsbuf = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    eh = E["bf16"]
    for m_, n_, k_ in ((7168, 7168, 7168), (6144, 6144, 6144), (5120, 5120, 5120), (1024, 2048, 8192),
                       (1280, 1280, 8192)):
        name = f"bf16_{m_}" if m_ == n_ == k_ else f"bf16_{m_}x{n_}x{k_}"
        if not want(name):
            continue
        need = mcg.dense_workspace_bytes("bf16", "k_contig", "k_contig", m_, n_, k_, eh.A, n, eh.B, n)
        E[name] = Entry(name, "dense", dtA="bf16", dtB="bf16", layA="k_contig", layB="k_contig", M=m_, N=n_, K=k_,
                        A=eh.A, B=eh.B, hA=eh.hA, hB=eh.hB, lda=n, ldb=n, C=None, hC=None,
                        D=D.view(-1)[:m_ * n_].view(m_, n_), out="f32", alpha=1.0, beta=0.0, sA=1.0, sB=1.0,
                        peak=PEAK["bf16"], unit="TFLOP/s", ws=wsbuf, ws_bytes=need)
    # bf16 256^3 (launch-bound)
    As = W.operand("A", "bf16", 256, 256, "uniform", "k_contig")
    Bs_ = W.operand("B", "bf16", 256, 256, "uniform", "k_contig")
    Dsm = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    E["bf16_256"] = Entry("bf16_256", "dense", dtA="bf16", dtB="bf16", layA="k_contig", layB="k_contig",
                          M=256, N=256, K=256, A=dev(As.codes), B=dev(Bs_.codes), hA=As.codes, hB=Bs_.codes,
                          lda=256, ldb=256, C=None, hC=None, D=Dsm, out="f32", alpha=1.0, beta=0.0, sA=1.0,
                          sB=1.0, peak=PEAK["bf16"], unit="TFLOP/s", batch=SMALL_BATCH)
    # int8 4096^3 and 8192^3
    for m_ in (4096, n):
        A = W.operand("A", "i8", m_, m_, "int8", "k_contig")
        B = W.operand("B", "i8", m_, m_, "int8", "k_contig")
        Ch = W.c_matrix(m_, m_, "int20")
        name = "i8" if m_ == n else f"i8_{m_}"
        E[name] = Entry(name, "dense", dtA="i8", dtB="i8", layA="k_contig", layB="k_contig", M=m_, N=m_,
                        K=m_, A=dev(A.codes), B=dev(B.codes), hA=A.codes, hB=B.codes, lda=m_, ldb=m_,
                        C=dev(Ch), hC=Ch, D=Di if m_ == n else torch.empty((m_, m_), dtype=torch.int32,
                                                                          device="cuda"),
                        out="i32", alpha=1, beta=1, sA=1.0, sB=1.0, peak=PEAK["i8"], unit="TOPS")
    # fp8 pairs
    A8 = W.operand("A", "e4m3", n, n, "normal", "k_contig", fp8_scaled=True)
    dA8 = dev(A8.codes)
    for dtb in ("e4m3", "e5m2"):
        B8 = W.operand("B", dtb, n, n, "normal", "k_contig", fp8_scaled=True)
        name = f"e4m3x{dtb}"
        E[name] = Entry(name, "dense", dtA="e4m3", dtB=dtb, layA="k_contig", layB="k_contig", M=n, N=n, K=n,
                        A=dA8, B=dev(B8.codes), hA=A8.codes, hB=B8.codes, lda=n, ldb=n, C=None, hC=None, D=D,
                        out="f32", alpha=1.0, beta=0.0, sA=A8.scale, sB=B8.scale, peak=PEAK["fp8"],
                        unit="TFLOP/s")
    # bf16 with bfloat16 C and D
    C16 = C.to(torch.bfloat16).view(torch.int16)
    kw = {k: v for k, v in E["bf16"].__dict__.items() if k not in ("name", "kind")}
    kw.update(C=C16, hC=C16.cpu().numpy().view(np.uint16), out="bf16",
              D=torch.empty((n, n), dtype=torch.int16, device="cuda"))
    E["bf16_out"] = Entry("bf16_out", "dense", **kw)
    # 2:4 sparse: bf16 compressed on the device inside the step (compress24 is
    # itself timed); 8-bit operands compressed once before timing
    Ad_h = W.sparse24_dense("bf16", n, n)
    Ad = dev(Ad_h)
    vals = torch.empty((n, n // 2), dtype=torch.int16, device="cuda")
    idx = torch.empty((n, n // 32), dtype=torch.int32, device="cuda")
    E["compress24"] = Entry("compress24", "compress", dt="bf16", M=n, K=n, A=Ad, hA=Ad_h, vals=vals, idx=idx,
                            nbytes=n * n * 2 + n * n // 2 * 2 + n * (n // 32) * 4)
    E["sparse24"] = Entry("sparse24", "sparse", dtA="bf16", dtB="bf16", M=n, N=n, K=n, vals=vals, idx=idx,
                          B=E["bf16"].B, hB=E["bf16"].hB, ldb=n, D=D, out="f32", alpha=1.0, beta=0.0,
                          dense="bf16", peak=PEAK["bf16"], speak=SPARSE_PEAK["bf16"], unit="TFLOP/s")
    for dt, dense in (("i8", "i8"), ("e4m3", "e4m3xe4m3")):
        name = f"sparse24_{dt}"
        if not want(name):
            continue
        A_ = dev(W.sparse24_dense(dt, n, n, dist="int8" if dt == "i8" else "normal"))
        v_ = torch.empty((n, n // 2), dtype=torch.uint8, device="cuda")
        i_ = torch.empty((n, n // 32), dtype=torch.int32, device="cuda")
        mcg.compress24(dt, n, n, A_, n, v_, n // 2, i_, n // 32, None)
        del A_
        eb = E[dense]
        E[name] = Entry(name, "sparse", dtA=dt, dtB=eb.dtB, M=n, N=n, K=n, vals=v_, idx=i_, B=eb.B, hB=eb.hB,
                        ldb=n, D=Di if dt == "i8" else D, out="i32" if dt == "i8" else "f32",
                        alpha=1 if dt == "i8" else eb.sB, beta=0, dense=dense,
                        peak=PEAK["i8" if dt == "i8" else "fp8"], speak=SPARSE_PEAK["i8" if dt == "i8" else "fp8"],
                        unit="TOPS" if dt == "i8" else "TFLOP/s")
    # 2:4 bf16 2048^2 x 8192 on gemm_sparse24_ws (stream-K form): leading blocks
    # of the 8192^3 entry's compressed A (lda_c = n / 2, ld_idx = n / 32) and B
    if want("sparse24_2048x2048x8192"):
        m_, n_, k_ = 2048, 2048, 8192
        es = E["sparse24"]
        need = mcg.sparse24_workspace_bytes("bf16", "k_contig", m_, n_, k_, vals, n // 2, idx, n // 32, es.B, n)
        E["sparse24_2048x2048x8192"] = Entry(
            "sparse24_2048x2048x8192", "sparse", dtA="bf16", dtB="bf16", M=m_, N=n_, K=k_, vals=vals, idx=idx,
            B=es.B, hB=es.hB, ldb=n, D=D.view(-1)[:m_ * n_].view(m_, n_), out="f32", alpha=1.0, beta=0.0,
            dense=None, peak=PEAK["bf16"], speak=SPARSE_PEAK["bf16"], unit="TFLOP/s", ws=wsbuf, ws_bytes=need,
            lda_c=n // 2, ld_idx=n // 32)
    # skinny problems: the wide operand (4n x n bf16 ~ N(0,1)) drawn on the device
    g = torch.Generator(device="cuda").manual_seed(W.SEED_A)
    Wide = torch.randn((4 * n, n), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    Narrow = torch.randn((16, n), generator=g, device="cuda").to(torch.bfloat16).view(torch.int16)
    Dsk = torch.empty((4 * n, 16), dtype=torch.float32, device="cuda")
    for name, (A_, B_, M_, N_) in (("skinny_n16", (Wide, Narrow, 4 * n, 16)),
                                   ("skinny_m16", (Narrow, Wide, 16, 4 * n))):
        E[name] = Entry(name, "skinny", dtA="bf16", dtB="bf16", layA="k_contig", layB="k_contig", M=M_, N=N_,
                        K=n, A=A_, B=B_, lda=n, ldb=n, C=None, D=Dsk, out="f32", alpha=1.0, beta=0.0, sA=1.0,
                        sB=1.0, nbytes=(4 * n * n + 16 * n) * 2 + 4 * n * 16 * 4)
    # binary64 operands ~ N(0,1), drawn on the device
    if want("f64"):
        A64 = torch.randn((n, n), generator=g, dtype=torch.float64, device="cuda")
        B64 = torch.randn((n, n), generator=g, dtype=torch.float64, device="cuda")  # column-major K x N
        C64 = torch.randn((n, n), generator=g, dtype=torch.float64, device="cuda")
        E["f64"] = Entry("f64", "f64", M=n, N=n, K=n, A=A64, B=B64, C=C64,
                         D=torch.empty((n, n), dtype=torch.float64, device="cuda"), alpha=1.0, beta=1.0,
                         peak=PEAK["f64"], unit="TFLOP/s")
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    stream = torch.cuda.Stream()
    s = stream.cuda_stream

    def call(e):
        if e.kind == "dense" and getattr(e, "ws", None) is not None:
            mcg.gemm_dense_ws(e.dtA, e.dtB, e.layA, e.layB, e.M, e.N, e.K, e.A, e.lda, e.B, e.ldb, e.C, e.D, e.N,
                              e.out, e.alpha, e.beta, e.sA, e.sB, workspace=e.ws, workspace_bytes=e.ws_bytes,
                              stream=s)
        elif e.kind in ("dense", "skinny"):
            mcg.gemm_dense(e.dtA, e.dtB, e.layA, e.layB, e.M, e.N, e.K, e.A, e.lda, e.B, e.ldb, e.C, e.D, e.N,
                           e.out, e.alpha, e.beta, e.sA, e.sB, stream=s)
        elif e.kind == "compress":
            mcg.compress24(e.dt, e.M, e.K, e.A, e.K, e.vals, e.K // 2, e.idx, e.K // 32, None, stream=s)
        elif e.kind == "sparse" and getattr(e, "ws", None) is not None:
            mcg.gemm_sparse24_ws(e.dtA, e.dtB, "k_contig", e.M, e.N, e.K, e.vals, e.lda_c, e.idx, e.ld_idx, e.B,
                                 e.ldb, None, e.D, e.N, e.out, e.alpha, e.beta, workspace=e.ws,
                                 workspace_bytes=e.ws_bytes, stream=s)
        elif e.kind == "sparse":
            mcg.gemm_sparse24(e.dtA, e.dtB, "k_contig", e.M, e.N, e.K, e.vals, e.K // 2, e.idx, e.K // 32, e.B,
                              e.ldb, None, e.D, e.N, e.out, e.alpha, e.beta, stream=s)
        elif e.kind == "f64":
            mcg.gemm_dense("f64", "f64", 0, 0, e.M, e.N, e.K, e.A, e.K, e.B, e.K, e.C, e.D, e.N, "f64", e.alpha,
                           e.beta, stream=s)

    order = ["bf16", "f16", "bf16_Arow_Brow", "bf16_Acol_Bcol", "bf16_Acol_Brow", "f16_Arow_Brow",
             "f16_Acol_Bcol", "f16_Acol_Brow", "bf16_256", "i8_4096", "i8", "e4m3xe4m3", "e4m3xe5m2",
             "compress24", "sparse24", "bf16_out", "skinny_n16", "skinny_m16", "sparse24_i8", "sparse24_e4m3",
             "f64", "bf16_7168", "bf16_6144", "bf16_5120", "bf16_1024x2048x8192", "bf16_1280x1280x8192",
             "sparse24_2048x2048x8192"]
    names = [x for x in order if x in E and (only is None or x in only or x == "compress24" and "sparse24" in only)]
    ev = {x: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] for x in names}

    def run(e):
        g = getattr(e, "graph", None)
        if g is not None:
            g.replay()
            return
        for _ in range(getattr(e, "batch", 1)):
            call(e)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            for x in names:
                run(E[x])
        torch.cuda.synchronize()
        # Launch-bound entries (a batch of back-to-back calls per step) replay the
        # batch from a HIP graph captured once: the library only launches kernels
        # on the caller's stream, so the calls capture as they are, and each step
        # then measures the kernels rather than the Python loop that issues them.
        # The eager rate is reported beside it.
        eager_us = {}
        for x in names:
            e = E[x]
            if getattr(e, "batch", 1) > 1:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(e.batch):
                    call(e)
                e1.record(stream)
                torch.cuda.synchronize()
                eager_us[x] = e0.elapsed_time(e1) * 1e3 / e.batch
                e.graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(e.graph, stream=stream):
                    for _ in range(e.batch):
                        call(e)
                e.graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for step in range(args.steps):
            for x in names:
                ev[x][step][0].record(stream)
                run(E[x])
                ev[x][step][1].record(stream)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
    log(f"timed {args.steps} steps in {t_end - t_start:.2f} s")

    # average duration of one call, ms
    ms = {x: float(np.mean([a.elapsed_time(b) for a, b in ev[x]])) / getattr(E[x], "batch", 1) for x in names}
    per = {}
    for x in names:
        e, t = E[x], ms[x] * 1e-3
        if e.kind in ("compress", "skinny"):
            per[x] = {"GB/s": e.nbytes / t / 1e9, "ms": ms[x], "frac_of_hbm_peak": e.nbytes / t / 1e9 / HBM_PEAK_GBS,
                      "bytes": e.nbytes}
            if e.kind == "skinny":
                per[x].update({"TFLOP/s": 2.0 * e.M * e.N * e.K / t / 1e12, "MxNxK": (e.M, e.N, e.K)})
            continue
        tf = 2.0 * e.M * e.N * e.K / t / 1e12
        if e.kind == "sparse":
            d = {f"{e.unit}_dense_equiv": tf, f"{e.unit}_algorithmic": tf / 2, "ms": ms[x],
                 "frac_of_sparse_peak": tf / e.speak, "sparse_peak": e.speak, "frac_of_dense_peak": tf / e.peak}
            if e.dense in ms:
                d[f"vs_dense_{e.dense}"] = tf / (2.0 * e.M * e.N * e.K / (ms[e.dense] * 1e-3) / 1e12)
            if getattr(e, "ws", None) is not None:
                d["MxNxK"] = (e.M, e.N, e.K)
                d["stream_k_workspace_MiB"] = e.ws_bytes / 2**20
            per[x] = d
        else:
            per[x] = {e.unit: tf, "ms": ms[x], "peak": e.peak, "frac_of_peak": tf / e.peak,
                      "MxNxK": (e.M, e.N, e.K)}
            if e.kind == "dense":
                per[x]["layout"] = LAYOUT_NAMES[(e.layA, e.layB)]
            if x in eager_us:
                per[x].update({"launches_per_step": e.batch, "replayed_from_hip_graph": True,
                               "eager_us_per_launch": eager_us[x],
                               "eager_" + e.unit: 2.0 * e.M * e.N * e.K / (eager_us[x] * 1e-6) / 1e12})
            if getattr(e, "ws", None) is not None:
                per[x]["stream_k_workspace_MiB"] = e.ws_bytes / 2**20  # 0: whole tiles only
    head = "bf16" if "bf16" in names else names[0]
    value = per[head].get("TFLOP/s", per[head].get("TOPS", per[head].get("GB/s")))

    # ---------------------------------------------------------------- matrix-core ceiling
    # The published peaks hold at the peak clock; under full matrix-core load the
    # clock depends on the operand bits.  mcg_mfma_probe runs each entry's
    # instruction in the kernels' arrangement on fragments of that entry's own
    # operands, with no other traffic: the rate no data-movement schedule can
    # exceed for those bits (after the timed steps, outside their events).
    ceiling = None
    if not args.no_ceiling:
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        sink = torch.empty(ncu * 512, device="cuda")
        clocks = torch.zeros(2 * ncu, dtype=torch.int64, device="cuda")
        # dense k of one instruction: mfma 32x32x{16,32,64}; smfmac 32x32x{32,64,64}
        kd = {0: {"bf16": 16, "f16": 16, "i8": 32, "e4m3": 64, "e5m2": 64},
              1: {"bf16": 32, "f16": 32, "i8": 64, "e4m3": 64, "e5m2": 64}}
        instr = 16384
        cache = {}

        def probe(dtA, dtB, sparse, a, b, idx):
            key = (dtA, dtB, sparse, a.data_ptr(), b.data_ptr())
            if key not in cache:
                times = []
                with torch.cuda.stream(stream):
                    mcg.mfma_probe(dtA, dtB, sparse, a, b, idx, instr, ncu, sink, clocks, stream=s)
                    for _ in range(3):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        mcg.mfma_probe(dtA, dtB, sparse, a, b, idx, instr, ncu, sink, clocks, stream=s)
                        e1.record(stream)
                        times.append((e0, e1))
                torch.cuda.synchronize()
                t = sorted(a_.elapsed_time(b_) for a_, b_ in times)[1] * 1e-3
                c = clocks.view(ncu, 2).double().cpu()
                flops = ncu * 8 * instr * 2 * 32 * 32 * kd[sparse][dtA]
                cache[key] = (flops / t / 1e12, float((c[:, 0] / c[:, 1]).mean()) * 0.1)
            return cache[key]

        for x in names:
            e = E[x]
            if e.kind == "dense" and e.dtA in kd[0]:
                rate, ghz = probe(e.dtA, e.dtB, 0, e.A, e.B, None)
                got = per[x][e.unit]
            elif e.kind == "sparse":
                rate, ghz = probe(e.dtA, e.dtB, 1, e.vals, e.B, e.idx)
                got = per[x][f"{e.unit}_dense_equiv"]
            else:
                continue
            pk = e.speak if e.kind == "sparse" else e.peak
            per[x]["mfma_ceiling"] = {"value": rate, "unit": e.unit + ("_dense_equiv" if e.kind == "sparse" else ""),
                                      "clock_ghz": ghz, "frac_of_peak": rate / pk}
            per[x]["frac_of_ceiling"] = got / rate
        if head in per and "mfma_ceiling" in per[head]:
            ceiling = dict(per[head]["mfma_ceiling"])
            ceiling.update({"achieved_frac_of_ceiling": per[head]["frac_of_ceiling"],
                            "probe": f"mcg_mfma_probe: {instr} instructions per wavefront, {ncu} workgroups "
                                     "of 8 wavefronts, fragments from the entry's own operands"})
        log(f"matrix-core ceiling on the headline operands: {ceiling}")

    # ---------------------------------------------------------------- parity
    # Every entry once more; sampled outputs against the oracle (the acceptance
    # test of the parity tests: the float bound, or bit-exact integers / codes).
    parity = None
    if not args.no_parity:
        import oracle
        parity = {}
        t_par = time.perf_counter()
        for x in names:
            e = E[x]
            D_ = getattr(e, "D", None)
            with torch.cuda.stream(stream):
                if D_ is not None:  # a stale or unwritten output must not pass
                    D_.fill_({torch.int32: 0x7FC00000, torch.int16: 0x7FC0}.get(D_.dtype, float("nan")))
                call(e)
            torch.cuda.synchronize()
            if e.kind == "compress":
                rows = np.arange(0, e.M, 97)
                v, i, nv = oracle.compress24(e.dt, e.hA[rows])
                ok = (nv == 0 and np.array_equal(e.vals.cpu().numpy().view(np.uint16)[rows], v)
                      and np.array_equal(e.idx.cpu().numpy().view(np.uint32)[rows], i))
                parity[x] = {"ok": bool(ok), "rows": len(rows), "exact": True}
                continue
            rows, cols = W.sample_coords(e.M, e.N, n_random=1024, full_rows=(e.M - 1,))
            if e.kind == "skinny":
                hA = e.A.cpu().numpy().view(np.uint16)
                hB = e.B.cpu().numpy().view(np.uint16)
                dg = e.D.cpu().numpy().reshape(-1)[rows * e.N + cols]
                ref, sm = oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", e.M, e.N, e.K, hA, e.lda,
                                            hB, e.ldb, rows=rows, cols=cols)
                r = oracle.check_float(dg, ref, sm, e.K)
            elif e.kind == "f64":
                hA, hB, hC = e.A.cpu().numpy(), e.B.cpu().numpy(), e.C.cpu().numpy()
                dg = e.D.cpu().numpy()[rows, cols]
                ref, sm = oracle.gemm_f64("k_contig", "k_contig", e.M, e.N, e.K, hA, e.K, hB, e.K, hC, e.N,
                                          e.alpha, e.beta, rows=rows, cols=cols)
                r = oracle.check_f64(dg, ref, sm, e.K, e.alpha, e.beta, hC[rows, cols])
            elif e.kind == "sparse":
                hv = e.vals.cpu().numpy().view(oracle.CODE_NP[e.dtA])
                hi = e.idx.cpu().numpy().view(np.uint32)
                ref, sm = oracle.gemm_sparse24(e.dtA, e.dtB, "k_contig", e.M, e.N, e.K, hv, hi, e.hB, e.ldb,
                                               alpha=e.alpha, beta=0.0, rows=rows, cols=cols, out=e.out)
                dg = e.D.cpu().numpy()[rows, cols]
                r = (oracle.check_exact(dg, ref) if e.dtA == "i8"
                     else oracle.check_float(dg, ref, sm, e.K, e.alpha))
            else:
                dD = e.D.cpu().numpy()
                if e.out == "bf16":
                    dg = (dD.view(np.uint16).astype(np.uint32) << 16).view(np.float32)[rows, cols]
                else:
                    dg = dD[rows, cols]
                if e.dtA == "i8":
                    ref = oracle.gemm_i8(e.layA, e.layB, e.M, e.N, e.K, e.hA, e.lda, e.hB, e.ldb, e.hC, e.N,
                                         e.alpha, e.beta, rows=rows, cols=cols)
                    r = oracle.check_exact(dg, ref)
                else:
                    ref, sm = oracle.gemm_float(e.dtA, e.dtB, e.layA, e.layB, e.M, e.N, e.K, e.hA, e.lda, e.hB,
                                                e.ldb, e.hC, e.N, e.alpha, e.beta, e.sA, e.sB, rows=rows,
                                                cols=cols, out=e.out)
                    cc = None
                    if e.beta != 0:
                        cc = e.hC[rows, cols]
                        if e.out == "bf16":
                            cc = (cc.astype(np.uint32) << 16).view(np.float32)
                    r = oracle.check_float(dg, ref, sm, e.K, e.alpha, e.sA, e.sB, e.beta, cc, out=e.out)
            parity[x] = {"ok": bool(r["ok"]), "outputs": r["n"], "exact": "max_ratio" not in r}
            if "max_ratio" in r:
                parity[x]["max_err_over_bound"] = r["max_ratio"]
            if not r["ok"]:
                log(f"PARITY FAILURE {x}: {r}")
        parity = {"all_ok": all(v["ok"] for v in parity.values()),
                  "sample": "per entry: its last row and 1024 random outputs (compress24: every 97th row), "
                            "recomputed by the oracle; float results within the acceptance bound, "
                            "integers and codes bit-exact",
                  "seconds": time.perf_counter() - t_par, "entries": parity}
        log(f"parity: all_ok = {parity['all_ok']} ({parity['seconds']:.1f} s)")

    # ---------------------------------------------------------------- CPU baseline
    # The oracle as it stands, all host threads, on whole rows of each workload
    # (bounded time), plus the 256^3 workload whole and single-threaded.
    cpu = None
    if not args.no_cpu:
        import oracle
        model, sockets = host_cpu()
        nthr = oracle.max_threads()

        def time_rows(e, budget):
            def run_rows(nrows):
                rr = np.repeat(np.arange(nrows, dtype=np.int64) * (e.M // nrows), e.N)
                cc = np.tile(np.arange(e.N, dtype=np.int64), nrows)
                t1 = time.perf_counter()
                if e.kind == "sparse":
                    oracle.gemm_sparse24(e.dtA, e.dtB, "k_contig", e.M, e.N, e.K, e.hv, e.hi, e.hB, e.ldb,
                                         alpha=e.alpha, rows=rr, cols=cc, out=e.out)
                elif e.dtA == "i8":
                    oracle.gemm_i8(e.layA, e.layB, e.M, e.N, e.K, e.hA, e.lda, e.hB, e.ldb, e.hC, e.N, e.alpha,
                                   e.beta, rows=rr, cols=cc)
                else:
                    oracle.gemm_float(e.dtA, e.dtB, e.layA, e.layB, e.M, e.N, e.K, e.hA, e.lda, e.hB, e.ldb,
                                      e.hC, e.N, e.alpha, e.beta, e.sA, e.sB, rows=rr, cols=cc)
                return time.perf_counter() - t1
            one = run_rows(1)
            nrows = max(1, min(e.M, int(budget / max(one, 1e-6))))
            t = run_rows(nrows)
            rate = 2.0 * nrows * e.N * e.K / t / 1e12
            return {"value": rate, "unit": "TOPS" if e.dtA == "i8" else "TFLOP/s", "seconds": t,
                    "sample": f"{nrows} whole rows ({nrows * e.N} outputs) of {e.M}x{e.N}x{e.K}",
                    "gpu_over_cpu": per[e.name][e.unit if e.kind != "sparse" else f"{e.unit}_dense_equiv"] / rate
                    if e.name in per else None}

        per_cfg = {}
        eh = E["bf16"]
        per_cfg["bf16_8192"] = time_rows(eh, args.cpu_seconds)
        for key, x in (("i8_4096", "i8_4096"), ("e4m3xe4m3_8192", "e4m3xe4m3"), ("sparse24_bf16_8192", "sparse24")):
            if x not in E:
                continue
            e = E[x]
            if e.kind == "sparse":
                e.hv = e.vals.cpu().numpy().view(oracle.CODE_NP[e.dtA])
                e.hi = e.idx.cpu().numpy().view(np.uint32)
            per_cfg[key] = time_rows(e, args.cpu_seconds / 5)
        # 256^3 whole, all threads and one thread
        e = E["bf16_256"]
        for tag, thr in (("bf16_256", nthr), ("bf16_256_1thread", 1)):
            oracle.set_threads(thr)
            t1 = time.perf_counter()
            reps = 0
            while reps < 3 or time.perf_counter() - t1 < 0.5:
                oracle.gemm_float("bf16", "bf16", "k_contig", "k_contig", 256, 256, 256, e.hA, 256, e.hB, 256)
                reps += 1
            t = (time.perf_counter() - t1) / reps
            per_cfg[tag] = {"value": 2.0 * 256 ** 3 / t / 1e12, "unit": "TFLOP/s", "seconds": t, "threads": thr,
                            "sample": "the whole 256^3 product",
                            "gpu_over_cpu": per["bf16_256"]["TFLOP/s"] / (2.0 * 256 ** 3 / t / 1e12)
                            if "bf16_256" in per else None}
        oracle.set_threads(nthr)
        h = per_cfg["bf16_8192"]
        cpu = {"value": h["value"], "unit": "TFLOP/s", "cores": nthr, "kind": "oracle",
               "sample": f"{h['sample']} of the dense bf16 8192^3 workload (K-contiguous pair, with C); "
                         f"{h['seconds']:.1f} s on {nthr} threads",
               "cpu_model": model, "sockets": sockets, "per_workload": per_cfg}

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
                               f"{len(names)} hot-path entries (per_dtype)",
                   "M": n, "N": n, "K": n, "entries": names},
        "roofline": {"bound": "mfma", "achieved": value, "peak": PEAK["bf16"], "unit": "TFLOP/s",
                     "frac": value / PEAK["bf16"], "traffic": measured_traffic() if head == "bf16" else None,
                     "traffic_unit": "HBM bytes per launch",
                     "algorithmic_bytes": (2 * n * n + 2 * n * n + 8 * n * n),
                     "kernel": "mcg::fast::gemm_fast_kernel<BF16, 0, 0, 256> (256x256 tile, 8-wave ping-pong)",
                     "kernel_ms": ms.get(head)},
        "cpu_baseline": cpu,
        "mfma_ceiling": ceiling,
        "parity": parity,
        "per_dtype": per,
    }
    print(json.dumps(res), flush=True)
    if parity is not None and not parity["all_ok"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
