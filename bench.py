#!/usr/bin/env python3
"""Throughput of the CSR SpMM / SDDMM hot path on one MI355X.

A step is one pass of the whole hot path over the Transformer-FFN workload
(A 2048x512 at 90 % sparsity, row lengths N(51.2, 5.12); B 512x256; companion
SDDMM with dY 2048x256 and X 512x256): CSR row offsets and the row swizzle
from the row lengths (one launch), SpMM C = A B and SDDMM dA = (dY X^T) at
A's entries -- three kernels, captured in a HIP graph and replayed.  Inputs are resident in
HBM before timing starts.

Prints one JSON line:
  value        useful GFLOP/s of the step, (2 nnz n + 2 nnz d) / step time
  roofline     the SpMM kernel: algorithmic (compulsory) bytes per launch over
               its average launch duration, against 8 TB/s HBM peak
  cpu_baseline the C oracle timed on this host's cores on the same inputs
  kernels      per-kernel average durations, GFLOP/s and GB/s

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SpMM/SDDMM GFLOP/s (2·nnz·N) + HBM GB/s vs roofline at 90% sparsity"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X FP32 vector, published (counts packed FP32)
FP32_FMA_PEAK_TFLOPS = 78.6      # 256 CU x 64 FMA/clk x 2 x 2.4 GHz: unpacked FMA (the build's)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spmm_sddmm_transformer_ffn_traffic.json")
STREAM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spmm_lds_hbm_stream_traffic.json")
CSRC = os.path.join(ROOT, "unstructured_sparse_linear_csr_amd", "csrc")


# The sources a measured launch is built from: its kernel's file, the files
# whose variant selection sets its parameters, the entry points, and every
# header.  A counter record stays valid while these hash the same.
PAIR_SOURCES = ("fused.hip", "spmm.hip", "sddmm.hip", "sp_api.hip")
STREAM_SOURCES = ("spmm.hip", "sp_api.hip")


def kernel_source_sha256(sources=None) -> str:
    """Hash of the named kernel source files plus every header (names and
    contents, sorted); every .hip and .h file when `sources` is None."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith(".h") or (name.endswith(".hip") and (sources is None or name in sources)):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def log(msg: str) -> None:
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--kernel-reps", type=int, default=200,
                    help="back-to-back launches per kernel for per-kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakeven", action="store_true",
                    help="skip the LSTM-sized sparsity sweep against dense GEMM")
    ap.add_argument("--suite", metavar="JSONL", default=None,
                    help="also time every workload (warm and cold caches) and "
                         "write one JSON record per kernel run to this file")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the streaming-regime SpMM (CSR far beyond the caches)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the probe kernels that measure this GPU's stream-read, "
                         "row-gather and launch ceilings")
    ap.add_argument("--profile-stream", action="store_true",
                    help="with --profile-launches: also launch the streaming-regime SpMM")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="only run this many eager launches of each kernel "
                         "(for rocprofv3 counter passes) and exit")
    return ap.parse_args()


def host_info() -> dict:
    model = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def spmm_bytes(m, k, n, nnz) -> int:
    """Compulsory bytes of one SpMM: CSR values and columns, row offsets and
    row order, B read once, C written once."""
    return 8 * nnz + 4 * (m + 1) + 4 * m + 4 * k * n + 4 * m * n


def sddmm_bytes(m, k, d, nnz) -> int:
    """Compulsory bytes of one SDDMM: X and Y read once, columns read, outputs
    written, row offsets and row order."""
    return 4 * m * d + 4 * k * d + 4 * nnz + 4 * nnz + 4 * (m + 1) + 4 * m


def traffic_record(path=TRAFFIC_FILE):
    """Measured HBM bytes per launch from the committed counter passes, if
    they were taken on the current kernel sources."""
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = kernel_source_sha256(rec.get("kernel_sources"))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def graph_time_us(torch, fn, reps: int) -> float:
    """Average launch duration of `fn` over `reps` back-to-back launches
    captured in one HIP graph, timed with events on the launch stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def cold_time_us(torch, fn, flush, reps: int = 10) -> float:
    """Median duration of single launches of `fn`, each after writing a
    buffer larger than the chip's caches (so operands come from HBM)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        flush.add_(1.0)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(times))


def latency_us(torch, fn, reps: int = 50) -> float:
    """Median duration of single eager launches of `fn` with its operands warm
    in the caches, each timed alone with events on the launch stream: what one
    call costs when it is not batched into a graph."""
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(times))


def spmm_record(name, m, k, n, nnz, us, extra=None) -> dict:
    s = us * 1e-6
    rec = {"record": "spmm", "workload": name, "m": m, "k": k, "n": n, "nnz": nnz,
           "us": us, "gflops": 2.0 * nnz * n / s / 1e9,
           "compulsory_gbs": spmm_bytes(m, k, n, nnz) / s / 1e9,
           "gather_gbs": 4.0 * nnz * n / s / 1e9}
    rec["hbm_frac"] = rec["compulsory_gbs"] / HBM_PEAK_GBS
    rec["fp32_fma_frac"] = rec["gflops"] / (FP32_FMA_PEAK_TFLOPS * 1e3)
    if extra:
        rec.update(extra)
    return rec


def upload_csr(torch, sp, dev, rl):
    """Device CSR of row lists: lengths, columns and values uploaded, offsets
    and the swizzled row order computed on the device."""
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    lengths, cols, vals = up(rl.lengths), up(rl.cols), up(rl.values)
    ro = torch.empty(rl.m + 1, dtype=torch.int32, device=dev)
    sp.sp_csr_offsets_from_lengths(rl.m, lengths, ro)
    ri = torch.empty(rl.m, dtype=torch.int32, device=dev)
    sp.sp_row_swizzle(rl.m, ro, ri)
    return ro, ri, cols, vals


def lstm_breakeven(torch, sp, inputs, dev, reps=50, records=None, flush=None):
    """SpMM time at each LSTM-sized sparsity next to a dense fp32 GEMM of the
    same shape; the break-even sparsity is where t_sparse / t_dense crosses 1,
    interpolated linearly between sweep points."""
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.set_float32_matmul_precision("highest")
    times = {}
    dense_us = None
    for s in inputs.LSTM_SPARSITIES:
        w = inputs.lstm(s)
        a = w["a"]
        m, k, n = w["m"], w["k"], w["n"]
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b = torch.from_numpy(w["b"]).to(dev)
        c = torch.empty(m, n, device=dev)
        fn = lambda: sp.sp_spmm(m, k, n, a.nnz, ri, vals, ro, cols, b, c)
        times[s] = graph_time_us(torch, fn, reps)
        if records is not None:
            cold = cold_time_us(torch, fn, flush) if flush is not None else None
            records.append(spmm_record(w["name"], m, k, n, a.nnz, times[s],
                                       {"sparsity": s, "cold_us": cold}))
        if dense_us is None:
            # The dense operand of the comparison: A with every entry present.
            dense_a = torch.from_numpy(inputs.random_dense(5, m, k, std=0.02)).to(dev)
            dfn = lambda: torch.mm(dense_a, b, out=c)
            dense_us = graph_time_us(torch, dfn, reps)
            if records is not None:
                records.append({"record": "dense_gemm", "workload": "lstm_8192x2048x128_dense",
                                "m": m, "k": k, "n": n, "us": dense_us,
                                "gflops": 2.0 * m * k * n / (dense_us * 1e-6) / 1e9,
                                "precision": "fp32 (TF32 off, matmul precision 'highest')"})
        log(f"lstm s={s}: spmm {times[s]:.2f} us (dense {dense_us:.2f} us)")
    ratio = {s: t / dense_us for s, t in times.items()}
    sps = sorted(ratio)
    breakeven = None
    for lo, hi in zip(sps, sps[1:]):
        if (ratio[lo] - 1.0) * (ratio[hi] - 1.0) <= 0 and ratio[lo] != ratio[hi]:
            breakeven = lo + (1.0 - ratio[lo]) * (hi - lo) / (ratio[hi] - ratio[lo])
            break
    return {"dense_fp32_gemm_us": dense_us, "spmm_us": {str(s): t for s, t in times.items()},
            "sparse_over_dense": {str(s): r for s, r in ratio.items()},
            "breakeven_sparsity": breakeven,
            "note": ("sparsity where SpMM time equals dense fp32 GEMM time, "
                     "linearly interpolated; null if the sweep has no crossing")}


def stream_setup(torch, sp, inputs, dev, dtype=None):
    """The streaming regime: A 65536 x 8192 at 90 % sparsity (53.7 M entries,
    430 MB of CSR, far beyond L2 and MALL), B 8192 x 4 held in LDS, natural
    row order; values and B fp32, or of the 16-bit torch `dtype`.  Returns
    (launch, workload description)."""
    w = inputs.hbm_stream(n=4)
    a = w["a"]
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ro = up(np.concatenate([[0], np.cumsum(a.lengths)]).astype(np.int32))
    cols, vals, b = up(a.cols), up(a.values), up(w["b"])
    c = torch.empty(w["m"], w["n"], device=dev)
    m, k, n, nnz = w["m"], w["k"], w["n"], a.nnz
    if dtype is None:
        fn = lambda: sp.sp_spmm(m, k, n, nnz, None, vals, ro, cols, b, c)
    else:
        vals, b = vals.to(dtype), b.to(dtype)
        fn = lambda: sp.sp_spmm_ex(m, k, n, nnz, None, vals, ro, cols, b, c)
    return fn, {"workload": w["name"], "m": m, "k": k, "n": n, "nnz": nnz}


def stream_record(torch, sp, inputs, dev) -> dict:
    """Average launch time of the streaming-regime SpMM (graph of 20
    launches, events on the launch stream) against the HBM roofline."""
    fn, desc = stream_setup(torch, sp, inputs, dev)
    us = graph_time_us(torch, fn, 20)
    alg = spmm_bytes(desc["m"], desc["k"], desc["n"], desc["nnz"])
    gbs = alg / (us * 1e-6) / 1e9
    rec = {**desc, "kernel": "spmm (B in LDS)", "avg_us": us,
           "gflops": 2.0 * desc["nnz"] * desc["n"] / (us * 1e-6) / 1e9,
           "algorithmic_bytes_per_launch": alg, "achieved_gbs": gbs,
           "frac_hbm_peak": gbs / HBM_PEAK_GBS,
           "traffic": traffic_record(STREAM_TRAFFIC_FILE)}
    del fn
    # the same matrix with bf16 values and B: 6 bytes per entry
    fn, desc = stream_setup(torch, sp, inputs, dev, torch.bfloat16)
    us = graph_time_us(torch, fn, 20)
    alg = (6 * desc["nnz"] + 4 * (desc["m"] + 1) + 2 * desc["k"] * desc["n"]
           + 4 * desc["m"] * desc["n"])
    gbs = alg / (us * 1e-6) / 1e9
    rec["bf16"] = {"avg_us": us, "algorithmic_bytes_per_launch": alg, "achieved_gbs": gbs,
                   "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                   "note": "values and B in bf16, fp32 arithmetic and C; 6 bytes per entry"}
    return rec


def backward_records(torch, sp, inputs, dev, w, flush) -> list:
    """Transpose of A (structure and values), the values-only update, and the
    backward product dX = A^T dY, for one workload."""
    a = w["a"]
    m, k, n, nnz = w["m"], w["k"], w["n"], a.nnz
    ro, _, cols, vals = upload_csr(torch, sp, dev, a)
    ws = torch.empty(sp.sp_csr_transpose_workspace(m, k, nnz), dtype=torch.uint8, device=dev)
    t_ro = torch.empty(k + 1, dtype=torch.int32, device=dev)
    t_ci = torch.empty(nnz, dtype=torch.int32, device=dev)
    t_v = torch.empty(nnz, device=dev)
    t_p = torch.empty(nnz, dtype=torch.int32, device=dev)
    t_ri = torch.empty(k, dtype=torch.int32, device=dev)
    tfn = lambda: sp.sp_csr_transpose(m, k, nnz, ro, cols, vals, t_ro, t_ci, t_v, t_p, ws)
    us_t = graph_time_us(torch, tfn, 20)
    tfn()
    sp.sp_row_swizzle(k, t_ro, t_ri)
    vfn = lambda: sp.sp_csr_transpose_values(nnz, t_p, vals, t_v)
    dy = torch.from_numpy(inputs.random_dense(7, m, n)).to(dev)
    dx = torch.empty(k, n, device=dev)
    bfn = lambda: sp.sp_spmm(k, m, n, nnz, t_ri, t_v, t_ro, t_ci, dy, dx)
    us_b = graph_time_us(torch, bfn, 50)
    return [{"record": "csr_transpose", "workload": w["name"], "m": m, "k": k, "nnz": nnz,
             "us": us_t, "entries_per_s": nnz / (us_t * 1e-6)},
            {"record": "csr_transpose_values", "workload": w["name"], "nnz": nnz,
             "us": graph_time_us(torch, vfn, 50)},
            spmm_record(w["name"] + "_backward_AT_dY", k, m, n, nnz, us_b,
                        {"cold_us": cold_time_us(torch, bfn, flush), "swizzle": True})]


def lowp_records(torch, sp, inputs, dev, flush) -> list:
    """SpMM and SDDMM with 16-bit operands on the FFN, LSTM 90 % and ResNet
    shapes and the attention pair; bytes counted at 2 per operand element."""
    recs = []
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    for tdt, tag in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        for w in (inputs.transformer_ffn(), inputs.lstm(0.9), inputs.resnet_1x1()):
            a = w["a"]
            m, k, n, nnz = w["m"], w["k"], w["n"], a.nnz
            ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
            v16, b16 = vals.to(tdt), up(w["b"]).to(tdt)
            c = torch.empty(m, n, device=dev)
            fn = lambda: sp.sp_spmm_ex(m, k, n, nnz, ri, v16, ro, cols, b16, c)
            us = graph_time_us(torch, fn, 50)
            byts = 6 * nnz + 8 * m + 4 + 2 * k * n + 4 * m * n
            recs.append({"record": "spmm_" + tag, "workload": w["name"], "m": m, "k": k,
                         "n": n, "nnz": nnz, "us": us,
                         "gflops": 2.0 * nnz * n / (us * 1e-6) / 1e9,
                         "compulsory_gbs": byts / (us * 1e-6) / 1e9,
                         "cold_us": cold_time_us(torch, fn, flush)})
            if "x" in w:
                d = w["d"]
                x16, y16 = up(w["x"]).to(tdt), up(w["y"]).to(tdt)
                out = torch.empty(nnz, device=dev)
                sfn = lambda: sp.sp_sddmm_ex(m, k, d, nnz, ri, ro, cols, x16, y16, 1.0, out)
                us = graph_time_us(torch, sfn, 50)
                recs.append({"record": "sddmm_" + tag, "workload": w["name"], "m": m, "k": k,
                             "d": d, "nnz": nnz, "us": us,
                             "gflops": 2.0 * nnz * d / (us * 1e-6) / 1e9,
                             "cold_us": cold_time_us(torch, sfn, flush)})
        w = inputs.sparse_attention()
        bh, seq, hd = w["batch"], w["seq"], w["head_dim"]
        mk = up(w["mask"])
        ro = torch.empty(seq + 1, dtype=torch.int32, device=dev)
        sp.sp_csr_count_dense(seq, seq, mk, ro)
        nnz = int(ro[seq].item())
        cols = torch.empty(nnz, dtype=torch.int32, device=dev)
        sp.sp_csr_fill_dense(seq, seq, mk, None, ro, cols, None)
        ri = torch.empty(seq, dtype=torch.int32, device=dev)
        sp.sp_row_swizzle(seq, ro, ri)
        q, kk, vv = up(w["q"]).to(tdt), up(w["k"]).to(tdt), up(w["v"]).to(tdt)
        s_out = torch.empty(bh, nnz, device=dev)
        p16 = torch.full((bh, nnz), 1.0 / 80.0, device=dev).to(tdt)
        o = torch.empty(bh, seq, hd, device=dev)
        sfn = lambda: sp.sp_sddmm_ex(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out, bh,
                                     seq * hd, seq * hd, nnz)
        pfn = lambda: sp.sp_spmm_ex(seq, seq, hd, nnz, ri, p16, ro, cols, vv, o, bh, nnz,
                                    seq * hd, seq * hd)
        afn = lambda: sp.sp_sparse_attention(seq, seq, hd, nnz, ri, ro, cols, q, kk, vv, 0.125, o,
                                             bh, seq * hd, seq * hd, seq * hd, seq * hd)
        for kind, fn in (("sddmm_batched_" + tag, sfn), ("spmm_batched_" + tag, pfn),
                         ("attention_one_pass_" + tag, afn)):
            us = graph_time_us(torch, fn, 20)
            flops = (4.0 if kind.startswith("attention") else 2.0) * bh * nnz * hd
            recs.append({"record": kind, "workload": w["name"], "batch": bh, "seq": seq,
                         "head_dim": hd, "nnz_per_head": nnz, "us": us,
                         "gflops": flops / (us * 1e-6) / 1e9,
                         "cold_us": cold_time_us(torch, fn, flush)})
    return recs


def run_suite(torch, sp, inputs, dev, path: str) -> None:
    """Every workload, warm (graph back-to-back) and cold (after flushing the
    caches), one JSON record per kernel run."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB > caches
    flush.zero_()
    recs = []
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    # Transformer FFN SpMM + SDDMM, and the lognormal imbalance variant with
    # and without the swizzled row order.
    for w in (inputs.transformer_ffn(), inputs.imbalance()):
        a = w["a"]
        m, k, n, d = w["m"], w["k"], w["n"], w["d"]
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b, x, y = up(w["b"]), up(w["x"]), up(w["y"])
        c = torch.empty(m, n, device=dev)
        out = torch.empty(a.nnz, device=dev)
        for swz in (True, False):
            order = ri if swz else None
            fn = lambda: sp.sp_spmm(m, k, n, a.nnz, order, vals, ro, cols, b, c)
            recs.append(spmm_record(w["name"], m, k, n, a.nnz, graph_time_us(torch, fn, 200),
                                    {"swizzle": swz, "cold_us": cold_time_us(torch, fn, flush)}))
            bfn = lambda: sp.sp_spmm_balanced(m, k, n, a.nnz, order, vals, ro, cols, b, c)
            recs.append(spmm_record(w["name"], m, k, n, a.nnz, graph_time_us(torch, bfn, 200),
                                    {"swizzle": swz, "kernel": "balanced",
                                     "cold_us": cold_time_us(torch, bfn, flush)}))
            sfn = lambda: sp.sp_sddmm(m, k, d, a.nnz, order, ro, cols, x, y, out)
            us = graph_time_us(torch, sfn, 200)
            recs.append({"record": "sddmm", "workload": w["name"], "m": m, "k": k, "d": d,
                         "nnz": a.nnz, "swizzle": swz, "us": us,
                         "cold_us": cold_time_us(torch, sfn, flush),
                         "gflops": 2.0 * a.nnz * d / (us * 1e-6) / 1e9,
                         "compulsory_gbs": sddmm_bytes(m, k, d, a.nnz) / (us * 1e-6) / 1e9})
            bsfn = lambda: sp.sp_sddmm_balanced(m, k, d, a.nnz, order, ro, cols, x, y, out)
            us = graph_time_us(torch, bsfn, 200)
            recs.append({"record": "sddmm", "workload": w["name"], "m": m, "k": k, "d": d,
                         "nnz": a.nnz, "swizzle": swz, "kernel": "balanced", "us": us,
                         "cold_us": cold_time_us(torch, bsfn, flush),
                         "gflops": 2.0 * a.nnz * d / (us * 1e-6) / 1e9,
                         "compulsory_gbs": sddmm_bytes(m, k, d, a.nnz) / (us * 1e-6) / 1e9})
        recs.append({"record": "row_swizzle", "workload": w["name"], "m": m,
                     "us": graph_time_us(torch, lambda: sp.sp_row_swizzle(m, ro, ri), 200)})
        if w["name"] != inputs.transformer_ffn()["name"]:
            continue
        # General SDDMM on the same shapes: the mask's values as the element-wise
        # scale and accumulation into the previous output, with Y stored k x d
        # and d x k.
        # (d x k once more with a workspace: Y transposed there first).
        y_dk = y.t().contiguous()
        ws = torch.empty(sp.sp_sddmm_general_workspace(k, d), dtype=torch.uint8, device=dev)
        for layout, yy, wsp, name in ((sp.SP_Y_KD, y, None, "kd"), (sp.SP_Y_DK, y_dk, None, "dk"),
                                      (sp.SP_Y_DK, y_dk, ws, "dk_workspace")):
            gfn = lambda: sp.sp_sddmm_general(m, k, d, a.nnz, ri, ro, cols, vals, x, yy,
                                              layout, 0.5, 1.0, out, workspace=wsp)
            us = graph_time_us(torch, gfn, 200)
            recs.append({"record": "sddmm_general", "workload": w["name"], "m": m, "k": k,
                         "d": d, "nnz": a.nnz, "y_layout": name, "mask_values": True,
                         "beta": 1.0, "us": us,
                         "cold_us": cold_time_us(torch, gfn, flush),
                         "gflops": 2.0 * a.nnz * d / (us * 1e-6) / 1e9,
                         "compulsory_gbs": (sddmm_bytes(m, k, d, a.nnz) + 8 * a.nnz)
                         / (us * 1e-6) / 1e9})
    # Backward pass of a sparse layer: A^T in CSR (once per structure; the
    # values of a new A follow through the permutation), then dX = A^T dY on
    # the swizzled rows of A^T.
    for w in (inputs.transformer_ffn(), inputs.lstm(0.9)):
        recs.extend(backward_records(torch, sp, inputs, dev, w, flush))
    # Mixed precision: values and B (X and Y) in 16-bit, fp32 arithmetic.
    recs.extend(lowp_records(torch, sp, inputs, dev, flush))
    # ResNet-50 1x1 conv
    w = inputs.resnet_1x1()
    a = w["a"]
    ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
    b = up(w["b"])
    c = torch.empty(w["m"], w["n"], device=dev)
    fn = lambda: sp.sp_spmm(w["m"], w["k"], w["n"], a.nnz, ri, vals, ro, cols, b, c)
    recs.append(spmm_record(w["name"], w["m"], w["k"], w["n"], a.nnz, graph_time_us(torch, fn, 50),
                            {"cold_us": cold_time_us(torch, fn, flush)}))
    # LSTM sweep with the dense comparison
    be = lstm_breakeven(torch, sp, inputs, dev, records=recs, flush=flush)
    recs.append({"record": "breakeven", **be})
    # Sparse attention over one shared mask: batched SDDMM (scores, scale
    # 1/8), the row softmax in place, batched SpMM (P V), each alone and the
    # three as one graph; and the scores with K given d x k.
    w = inputs.sparse_attention()
    bh, seq, hd = w["batch"], w["seq"], w["head_dim"]
    mk = up(w["mask"])
    ro = torch.empty(seq + 1, dtype=torch.int32, device=dev)
    sp.sp_csr_count_dense(seq, seq, mk, ro)
    nnz = int(ro[seq].item())
    cols = torch.empty(nnz, dtype=torch.int32, device=dev)
    sp.sp_csr_fill_dense(seq, seq, mk, None, ro, cols, None)
    ri = torch.empty(seq, dtype=torch.int32, device=dev)
    sp.sp_row_swizzle(seq, ro, ri)
    q, kk, v = up(w["q"]), up(w["k"]), up(w["v"])
    s_out = torch.empty(bh, nnz, device=dev)
    p_vals = torch.full((bh, nnz), 1.0 / 80.0, device=dev)
    o = torch.empty(bh, seq, hd, device=dev)
    sfn = lambda: sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                      bh, seq * hd, seq * hd, nnz)
    pfn = lambda: sp.sp_spmm_batched(seq, seq, hd, nnz, ri, p_vals, ro, cols, v, o, bh,
                                     nnz, seq * hd, seq * hd)
    kt = kk.transpose(1, 2).contiguous()
    tfn = lambda: sp.sp_sddmm_general(seq, seq, hd, nnz, ri, ro, cols, None, q, kt,
                                      sp.SP_Y_DK, 0.125, 0.0, s_out, bh, 0, seq * hd,
                                      seq * hd, nnz)
    kt_ws = torch.empty(sp.sp_sddmm_general_workspace(seq, hd, bh, seq * hd),
                        dtype=torch.uint8, device=dev)
    twfn = lambda: sp.sp_sddmm_general(seq, seq, hd, nnz, ri, ro, cols, None, q, kt,
                                       sp.SP_Y_DK, 0.125, 0.0, s_out, bh, 0, seq * hd,
                                       seq * hd, nnz, workspace=kt_ws)
    smfn = lambda: sp.sp_csr_row_softmax(seq, nnz, ri, ro, s_out, s_out, bh, nnz, nnz)

    def attention():
        sfn()
        smfn()
        sp.sp_spmm_batched(seq, seq, hd, nnz, ri, s_out, ro, cols, v, o, bh, nnz, seq * hd,
                           seq * hd)

    fsfn = lambda: sp.sp_sddmm_softmax(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                       bh, seq * hd, seq * hd, nnz)

    def attention_fused():
        fsfn()
        sp.sp_spmm_batched(seq, seq, hd, nnz, ri, s_out, ro, cols, v, o, bh, nnz, seq * hd,
                           seq * hd)

    vfn = lambda: sp.sp_sparse_attention(seq, seq, hd, nnz, ri, ro, cols, q, kk, v, 0.125, o,
                                         bh, seq * hd, seq * hd, seq * hd, seq * hd)
    for kind, fn in (("sddmm_batched", sfn), ("sddmm_general_dk_batched", tfn),
                     ("sddmm_general_dk_workspace_batched", twfn),
                     ("row_softmax_batched", smfn), ("sddmm_softmax_batched", fsfn),
                     ("spmm_batched", pfn), ("attention_all_device", attention),
                     ("attention_all_device_fused_scores", attention_fused),
                     ("attention_one_pass", vfn)):
        us = graph_time_us(torch, fn, 20)
        flops = 2.0 * bh * nnz * hd
        if kind == "row_softmax_batched":
            flops = 0.0
            byts = bh * 8 * nnz + 8 * seq
        elif kind.startswith("attention_"):
            flops = 4.0 * bh * nnz * hd
            byts = bh * (sddmm_bytes(seq, seq, hd, nnz) + 8 * nnz
                         + spmm_bytes(seq, seq, hd, nnz))
        else:
            byts = bh * (sddmm_bytes(seq, seq, hd, nnz) if kind.startswith("sddmm")
                         else spmm_bytes(seq, seq, hd, nnz))
        recs.append({"record": kind, "workload": w["name"], "batch": bh, "seq": seq,
                     "head_dim": hd, "nnz_per_head": nnz, "us": us,
                     "cold_us": cold_time_us(torch, fn, flush),
                     "gflops": flops / (us * 1e-6) / 1e9,
                     "compulsory_gbs": byts / (us * 1e-6) / 1e9})
    # Single-launch latency where launch overhead exceeds the roofline time:
    # the tiny problem (256x256 at 80 %), the Transformer FFN and the LSTM
    # layer at 98 %, one eager call at a time beside the graph-batched average.
    lat = []
    wt = inputs.tiny()
    at = sp.csr_from_dense(up(wt["mask"]), up(wt["dense_values"]))
    sp.row_swizzle(at)
    bt, xt, yt = up(wt["b"]), up(wt["x"]), up(wt["y"])
    ct = torch.empty(wt["m"], wt["n"], device=dev)
    ot = torch.empty(at.nnz, device=dev)
    lat.append((wt["name"], "spmm", at.nnz,
                lambda: sp.sp_spmm(at.m, at.k, wt["n"], at.nnz, at.row_indices, at.values,
                                   at.row_offsets, at.col_indices, bt, ct)))
    lat.append((wt["name"], "sddmm", at.nnz,
                lambda: sp.sp_sddmm(at.m, at.k, wt["d"], at.nnz, at.row_indices,
                                    at.row_offsets, at.col_indices, xt, yt, ot)))
    wf = inputs.transformer_ffn()
    rof, rif, colf, valf = upload_csr(torch, sp, dev, wf["a"])
    bf, xf, yf = up(wf["b"]), up(wf["x"]), up(wf["y"])
    cf = torch.empty(wf["m"], wf["n"], device=dev)
    of = torch.empty(wf["a"].nnz, device=dev)
    nf = wf["a"].nnz
    lat.append((wf["name"], "spmm", nf,
                lambda: sp.sp_spmm(wf["m"], wf["k"], wf["n"], nf, rif, valf, rof, colf, bf, cf)))
    lat.append((wf["name"], "sddmm", nf,
                lambda: sp.sp_sddmm(wf["m"], wf["k"], wf["d"], nf, rif, rof, colf, xf, yf, of)))
    wl = inputs.lstm(0.98)
    rol, ril, coll, vall = upload_csr(torch, sp, dev, wl["a"])
    bl = up(wl["b"])
    cl = torch.empty(wl["m"], wl["n"], device=dev)
    nl = wl["a"].nnz
    lat.append((wl["name"], "spmm", nl,
                lambda: sp.sp_spmm(wl["m"], wl["k"], wl["n"], nl, ril, vall, rol, coll, bl, cl)))
    for name, kern, nnz, fn in lat:
        recs.append({"record": "latency", "workload": name, "kernel": kern, "nnz": nnz,
                     "single_us": latency_us(torch, fn), "graph_us": graph_time_us(torch, fn, 200)})
    # The streaming regime: CSR far larger than every cache, n = 8 and n = 4
    # (B in LDS), natural and swizzled row order.
    for n_cols in (8, 4):
        w = inputs.hbm_stream(n=n_cols)
        a = w["a"]
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b = up(w["b"])
        c = torch.empty(w["m"], w["n"], device=dev)
        for order in (None, ri):
            fn = lambda: sp.sp_spmm(w["m"], w["k"], w["n"], a.nnz, order, vals, ro, cols, b, c)
            recs.append(spmm_record(w["name"], w["m"], w["k"], w["n"], a.nnz,
                                    graph_time_us(torch, fn, 20),
                                    {"cold_us": cold_time_us(torch, fn, flush),
                                     "csr_bytes": 8 * a.nnz, "swizzle": order is not None}))
        # 16-bit values and B: the CSR streams 6 bytes per entry
        for tag, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
            v16, b16 = vals.to(tdt), b.to(tdt)
            fn = lambda: sp.sp_spmm_ex(w["m"], w["k"], w["n"], a.nnz, None, v16, ro, cols,
                                       b16, c)
            us = graph_time_us(torch, fn, 20)
            byts = 6 * a.nnz + 4 * (w["m"] + 1) + 2 * w["k"] * w["n"] + 4 * w["m"] * w["n"]
            recs.append({"record": "spmm_" + tag, "workload": w["name"], "m": w["m"],
                         "k": w["k"], "n": w["n"], "nnz": a.nnz, "us": us,
                         "cold_us": cold_time_us(torch, fn, flush),
                         "gflops": 2.0 * a.nnz * w["n"] / (us * 1e-6) / 1e9,
                         "compulsory_gbs": byts / (us * 1e-6) / 1e9,
                         "hbm_frac": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS})
            del v16, b16
        del a, ro, ri, cols, vals
    with open(path, "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")
    for r in recs:
        log(json.dumps({kk: (round(vv, 3) if isinstance(vv, float) else vv)
                        for kk, vv in r.items() if not isinstance(vv, dict)}))


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(SpMM shards by rows of A or columns of B, attention by head, with no "
              "exchange; only the one-GPU share is implemented)", file=sys.stderr)
        return 2

    import torch
    from unstructured_sparse_linear_csr_amd import binding as sp
    from unstructured_sparse_linear_csr_amd import inputs

    assert torch.cuda.is_available(), "needs an MI355X"
    torch.cuda.set_device(0)
    dev = "cuda:0"
    sp.lib()

    w = inputs.transformer_ffn()
    a = w["a"]
    m, k, n, d, nnz = w["m"], w["k"], w["n"], w["d"], a.nnz
    stats = inputs.row_stats(a.lengths, k)
    log(f"workload {w['name']}: nnz={nnz} stats={stats}")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    lengths, cols, vals = up(a.lengths), up(a.cols), up(a.values)
    b, x, y = up(w["b"]), up(w["x"]), up(w["y"])
    ro = torch.empty(m + 1, dtype=torch.int32, device=dev)
    ri = torch.empty(m, dtype=torch.int32, device=dev)
    c = torch.empty(m, n, dtype=torch.float32, device=dev)
    out = torch.empty(nnz, dtype=torch.float32, device=dev)

    def k_build():
        sp.sp_csr_build_from_lengths(m, lengths, ro, ri)

    def k_offsets():
        sp.sp_csr_offsets_from_lengths(m, lengths, ro)

    def k_swizzle():
        sp.sp_row_swizzle(m, ro, ri)

    def k_spmm():
        sp.sp_spmm(m, k, n, nnz, ri, vals, ro, cols, b, c)

    def k_sddmm():
        sp.sp_sddmm(m, k, d, nnz, ri, ro, cols, x, y, out)

    def k_fused():
        sp.sp_spmm_sddmm(m, k, n, nnz, ri, vals, ro, cols, b, c, m, k, d, nnz, ri, ro, cols, x,
                         y, 1.0, out)

    def step():
        k_build()
        k_fused()

    if args.profile_launches:
        step()
        torch.cuda.synchronize()
        for fn in (k_build, k_offsets, k_swizzle, k_spmm, k_sddmm, k_fused):
            for _ in range(args.profile_launches):
                fn()
        if args.profile_stream:
            fn, _ = stream_setup(torch, sp, inputs, dev)
            for _ in range(args.profile_launches):
                fn()
        # a plain copy of known size, to calibrate the byte counters
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(args.profile_launches):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("profile launches done")
        return 0

    def capture(fn, reps):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        return g

    # ---- the timed steps: W warmup steps, then exactly K steps
    g_warm = capture(step, max(args.warmup, 1))
    g_steps = capture(step, args.steps)
    g_warm.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    flops_step = 2.0 * nnz * n + 2.0 * nnz * d
    gflops = flops_step / (ms_per_step * 1e-3) / 1e9
    log(f"step: {ms_per_step * 1e3:.2f} us  {gflops:.1f} GFLOP/s")

    # ---- per-kernel average launch duration: R back-to-back launches in a
    # graph on the stream the kernels run on, bracketed by events
    kernel_us = {}
    for name, fn in (("csr_build_from_lengths", k_build),
                     ("csr_offsets_from_lengths", k_offsets), ("row_swizzle", k_swizzle),
                     ("spmm", k_spmm), ("sddmm", k_sddmm), ("spmm_sddmm", k_fused)):
        g = capture(fn, args.kernel_reps)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        kernel_us[name] = e0.elapsed_time(e1) * 1e3 / args.kernel_reps
        log(f"kernel {name}: {kernel_us[name]:.2f} us")

    sb = spmm_bytes(m, k, n, nnz)
    db = sddmm_bytes(m, k, d, nnz)
    spmm_s = kernel_us["spmm"] * 1e-6
    sddmm_s = kernel_us["sddmm"] * 1e-6
    kernels = {
        "spmm": {"avg_us": kernel_us["spmm"],
                 "gflops": 2.0 * nnz * n / spmm_s / 1e9,
                 "compulsory_gbs": sb / spmm_s / 1e9,
                 "gather_gbs": 4.0 * nnz * n / spmm_s / 1e9},
        "sddmm": {"avg_us": kernel_us["sddmm"],
                  "gflops": 2.0 * nnz * d / sddmm_s / 1e9,
                  "compulsory_gbs": db / sddmm_s / 1e9,
                  "gather_gbs": 4.0 * nnz * d / sddmm_s / 1e9},
        "spmm_sddmm": {"avg_us": kernel_us["spmm_sddmm"],
                       "gflops": flops_step / (kernel_us["spmm_sddmm"] * 1e-6) / 1e9,
                       "note": "the SpMM and the SDDMM in one launch (in the step)"},
        "csr_build_from_lengths": {"avg_us": kernel_us["csr_build_from_lengths"],
                                   "note": "offsets and swizzled order in one launch (in the step)"},
        "row_swizzle": {"avg_us": kernel_us["row_swizzle"], "note": "standalone, not in the step"},
        "csr_offsets_from_lengths": {"avg_us": kernel_us["csr_offsets_from_lengths"],
                                     "note": "standalone, not in the step"},
    }
    for kk in ("spmm", "sddmm"):
        kernels[kk]["frac_fp32_fma_peak"] = kernels[kk]["gflops"] / (FP32_FMA_PEAK_TFLOPS * 1e3)
    # The step's dominant kernel: the SpMM and the SDDMM in one launch; its
    # algorithmic bytes are the two problems' compulsory bytes.
    fused_s = kernel_us["spmm_sddmm"] * 1e-6
    kernels["spmm_sddmm"]["compulsory_gbs"] = (sb + db) / fused_s / 1e9
    achieved = kernels["spmm_sddmm"]["compulsory_gbs"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_record(),
                "kernel": "spmm_sddmm", "algorithmic_bytes_per_launch": sb + db,
                "avg_launch_us": kernel_us["spmm_sddmm"]}

    result = {
        "metric": METRIC, "value": gflops, "unit": "GFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded numpy PCG64, seed 0)",
        "config": {"workload": w["name"], "m": m, "k": k, "n": n, "d": d, "nnz": nnz,
                   "sparsity": stats["sparsity"], "mean_row_length": stats["mean_row_length"],
                   "row_length_cov": stats["row_length_cov"],
                   "step": ("csr_build_from_lengths (offsets + row swizzle), then spmm and "
                            "sddmm in one launch (sp_spmm_sddmm)"),
                   "launch": "HIP graph of the K steps", "flops_per_step": flops_step},
        "roofline": roofline,
        "kernels": kernels,
    }

    if not args.no_breakeven:
        result["breakeven"] = lstm_breakeven(torch, sp, inputs, dev)

    if not args.no_stream:
        result["streaming"] = stream_record(torch, sp, inputs, dev)
        log(f"streaming spmm: {result['streaming']['avg_us']:.1f} us "
            f"{result['streaming']['achieved_gbs']:.0f} GB/s "
            f"({100 * result['streaming']['frac_hbm_peak']:.1f} % of HBM peak); bf16 "
            f"{result['streaming']['bf16']['avg_us']:.1f} us "
            f"({100 * result['streaming']['bf16']['frac_hbm_peak']:.1f} %)")

    if not args.no_ceilings:
        # The same byte count as the streaming SpMM's CSR, and the FFN SpMM's B.
        from unstructured_sparse_linear_csr_amd import probes
        result["ceilings"] = probes.measure(torch, stream_bytes=431164900,
                                            b_bytes=512 * 256 * 4)
        ceil = result["ceilings"]
        log(f"ceilings: stream read {ceil['stream_read_gbs']:.0f} GB/s (two arrays side by "
            f"side {ceil['stream_read2_gbs']:.0f} GB/s); 1 KB row gathers "
            + ", ".join(f"{k} {v:.1f} TB/s" for k, v in ceil["row_gather_tbs"].items())
            + f"; empty launch {ceil['launch_floor_us']:.2f} us")

    if args.suite:
        run_suite(torch, sp, inputs, dev, args.suite)

    # ---- CPU baseline: the oracle on this host, same inputs, one thread
    if not args.no_cpu_baseline:
        import oracle
        torch.cuda.synchronize()
        c_gpu = c.cpu().numpy()
        out_gpu = out.cpu().numpy()
        ro_gpu = ro.cpu().numpy()
        ri_gpu = ri.cpu().numpy()
        reps = 0
        t0 = time.perf_counter()
        cpu0 = time.process_time()
        while True:
            ro_o = oracle.csr_offsets_from_lengths(a.lengths)
            ri_o = oracle.row_swizzle(ro_o)
            c_o, c_abs = oracle.spmm(m, k, n, ro_o, a.cols, a.values, w["b"])
            s_o, s_abs = oracle.sddmm(m, k, d, ro_o, a.cols, w["x"], w["y"])
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        wall = time.perf_counter() - t0
        cpu_used = time.process_time() - cpu0
        per_step = wall / reps
        result["cpu_baseline"] = {
            "value": flops_step / per_step / 1e9, "unit": "GFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"the full step (offsets, swizzle, SpMM, SDDMM) on the same "
                       f"workload, repeated {reps} times in {wall:.1f} s "
                       f"({cpu_used:.1f} s CPU); single-threaded C, double accumulation"),
            "ms_per_step": per_step * 1e3, **host_info()}
        with np.errstate(divide="ignore", invalid="ignore"):
            spmm_ratio = float(np.max(np.abs(c_gpu - c_o) / (1e-5 * c_abs)))
            sddmm_ratio = float(np.max(np.abs(out_gpu - s_o) / (1e-5 * s_abs)))
        result["parity"] = {
            "row_offsets_bit_exact": bool(np.array_equal(ro_gpu, ro_o)),
            "row_swizzle_bit_exact": bool(np.array_equal(ri_gpu, ri_o)),
            "spmm_max_err_over_bound": spmm_ratio,
            "sddmm_max_err_over_bound": sddmm_ratio}
        log(f"cpu baseline: {result['cpu_baseline']['value']:.3f} GFLOP/s; "
            f"parity {result['parity']}")

    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
