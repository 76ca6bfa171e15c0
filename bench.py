#!/usr/bin/env python3
"""Throughput of the CSR SpMM / SDDMM hot path on one MI355X.

A step is one pass of the whole hot path over the Transformer-FFN workload
(A 2048x512 at 90 % sparsity, row lengths N(51.2, 5.12); B 512x256; companion
SDDMM with dY 2048x256 and X 512x256): CSR row offsets and the row swizzle
from the row lengths (one launch), then SpMM C = A B and SDDMM dA = (dY X^T)
at A's entries in one launch, captured in a HIP graph and replayed.  Inputs
are resident in HBM before timing starts.

Prints one JSON line:
  value        useful GFLOP/s of the step, (2 nnz n + 2 nnz d) / step time
  roofline     the step's dominant launch (SpMM + SDDMM): algorithmic
               (compulsory) bytes per launch over its average launch duration,
               against 8 TB/s HBM peak
  cpu_baseline the C oracle timed on this host's cores on the same inputs
  kernels      per-kernel average durations, GFLOP/s and GB/s
  records      every seeded workload (tiny, Transformer FFN, ResNet-50 1x1,
               LSTM sweep, sparse attention x 32 heads, lognormal imbalance,
               row swizzle at 65,536 and 1.1 M rows): warm and cold (after a
               1 GiB write) times, GFLOP/s, compulsory GB/s and the fraction of
               min(FP32 peak, arithmetic intensity x HBM peak), the smaller
               term named
  breakeven    LSTM-sized SpMM against dense fp32 GEMM
  streaming    a 430 MB-CSR SpMM where HBM bandwidth binds

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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload records (tiny, FFN, ResNet, attention, "
                         "imbalance, swizzle, latency)")
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
    ap.add_argument("--profile-workloads", default="ffn",
                    help="with --profile-launches: comma-separated workloads to launch -- "
                         "ffn (the step's kernels), resnet, lstm90, lstm50, attention; "
                         "resnet_wide, lstm50_wide: the same SpMM as a 2-entry batch, "
                         "which takes the wide kernel; stream8: the streaming-regime "
                         "SpMM with B 8 columns wide (two column slices); ffn_dk, "
                         "attention_dk: the general SDDMM with Y stored d x k and no "
                         "workspace; imbalance: the lognormal-row SpMM (swizzled, "
                         "natural) and SDDMM; transpose: the LSTM layer's CSR transpose")
    ap.add_argument("--profile-cold", action="store_true",
                    help="with --profile-launches: write a 1 GiB buffer before every "
                         "launch, so the byte counters see HBM traffic")
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


def roofline_of(flops: float, byts: float, us: float) -> dict:
    """Achieved rate of one kernel run against the published roofline: the
    attainable rate is min(FP32 vector peak, arithmetic intensity x HBM peak)
    over the run's compulsory bytes; `bound` names the smaller term.  The
    build's unpacked-FMA ceiling (78.6 TFLOP/s) is given beside it."""
    s = us * 1e-6
    gflops = flops / s / 1e9
    gbs = byts / s / 1e9
    if flops == 0:  # pure data movement (the row softmax): the HBM roof alone
        return {"gflops": 0.0, "compulsory_gbs": gbs, "ai_flop_per_byte": 0.0,
                "attainable_gflops": None, "bound": "hbm", "frac": gbs / HBM_PEAK_GBS,
                "frac_hbm_peak": gbs / HBM_PEAK_GBS, "frac_fp32_unpacked": 0.0}
    ai = flops / byts
    hbm_term = ai * HBM_PEAK_GBS                     # GFLOP/s
    fp32_term = FP32_VECTOR_PEAK_TFLOPS * 1e3
    attainable = min(hbm_term, fp32_term)
    return {"gflops": gflops, "compulsory_gbs": gbs,
            "ai_flop_per_byte": ai, "attainable_gflops": attainable,
            "bound": "hbm" if hbm_term < fp32_term else "fp32",
            "frac": gflops / attainable,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "frac_fp32_unpacked": gflops / (FP32_FMA_PEAK_TFLOPS * 1e3)}


def kernel_record(torch, config, kind, workload, fn, flops, byts, flush, reps, extra=None):
    """Warm (graph of back-to-back launches) and cold (single launches after a
    1 GiB write) timings of one kernel run, with its roofline figures."""
    us = graph_time_us(torch, fn, reps)
    rec = {"config": config, "kernel": kind, "workload": workload, "us": us,
           "cold_us": cold_time_us(torch, fn, flush) if flush is not None else None,
           "flops": flops, "compulsory_bytes": byts}
    rec.update(roofline_of(flops, byts, us))
    if extra:
        rec.update(extra)
    log(f"[{config}] {kind} {workload}: {us:.2f} us warm, "
        f"{rec['cold_us'] or 0:.2f} us cold, {rec['gflops']:.0f} GFLOP/s, "
        f"{100 * rec['frac']:.1f} % of the {rec['bound']} roof")
    return rec


def config_records(torch, sp, inputs, dev, flush) -> list:
    """One record per kernel run of each seeded workload: tiny SpMM and SDDMM;
    Transformer-FFN SpMM and SDDMM alone; ResNet-50 1x1 SpMM; sparse attention
    over 32 heads (scores, row softmax, weighted sum, and the one-pass form);
    the lognormal-row imbalance SpMM and SDDMM swizzled, natural and balanced;
    the row swizzle at 65,536 and 1.1 M rows (rank sort and radix sort); and
    single-launch latencies.  The LSTM sweep is recorded by lstm_breakeven."""
    recs = []
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    def kname(m, k, n, nnz, vals, cols, b, c, order):
        # the kernel the timed call (same row order) runs
        return sp.sp_spmm_kernel_name(m, k, n, nnz, vals, cols, b, c, row_indices=order)

    # ---- tiny (256 x 256, p = 0.2): SpMM n = 64, SDDMM d = 32
    wt = inputs.tiny()
    at = sp.csr_from_dense(up(wt["mask"]), up(wt["dense_values"]))
    sp.row_swizzle(at)
    bt, xt, yt = up(wt["b"]), up(wt["x"]), up(wt["y"])
    ct = torch.empty(wt["m"], wt["n"], device=dev)
    ot = torch.empty(at.nnz, device=dev)
    fns = {
        "spmm": lambda: sp.sp_spmm(at.m, at.k, wt["n"], at.nnz, at.row_indices, at.values,
                                   at.row_offsets, at.col_indices, bt, ct),
        "sddmm": lambda: sp.sp_sddmm(at.m, at.k, wt["d"], at.nnz, at.row_indices,
                                     at.row_offsets, at.col_indices, xt, yt, ot)}
    recs.append(kernel_record(torch, "tiny", "spmm", wt["name"], fns["spmm"],
                              2.0 * at.nnz * wt["n"], spmm_bytes(at.m, at.k, wt["n"], at.nnz),
                              flush, 200, {"m": at.m, "k": at.k, "n": wt["n"], "nnz": at.nnz,
                                           "single_launch_us": latency_us(torch, fns["spmm"]),
                                           "variant": kname(at.m, at.k, wt["n"], at.nnz,
                                                            at.values, at.col_indices, bt, ct,
                                                            at.row_indices)}))
    recs.append(kernel_record(torch, "tiny", "sddmm", wt["name"], fns["sddmm"],
                              2.0 * at.nnz * wt["d"], sddmm_bytes(at.m, at.k, wt["d"], at.nnz),
                              flush, 200, {"m": at.m, "k": at.k, "d": wt["d"], "nnz": at.nnz,
                                           "single_launch_us": latency_us(torch, fns["sddmm"])}))

    # ---- Transformer FFN (2048 x 512 at 90 %): the SpMM and the SDDMM alone,
    # and the imbalance workload (lognormal rows): swizzled, natural, balanced
    for w, cfg in ((inputs.transformer_ffn(), "transformer_ffn"),
                   (inputs.imbalance(), "imbalance")):
        a = w["a"]
        m, k, n, d, nnz = w["m"], w["k"], w["n"], w["d"], a.nnz
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b, x, y = up(w["b"]), up(w["x"]), up(w["y"])
        c = torch.empty(m, n, device=dev)
        out = torch.empty(nnz, device=dev)
        orders = ((True, False) if cfg == "imbalance" else (True,))
        for swz in orders:
            order = ri if swz else None
            tag = {"swizzle": swz, "m": m, "k": k, "n": n, "d": d, "nnz": nnz}
            fn = lambda: sp.sp_spmm(m, k, n, nnz, order, vals, ro, cols, b, c)
            ex = dict(tag, variant=kname(m, k, n, nnz, vals, cols, b, c, order))
            if cfg != "imbalance":
                ex["single_launch_us"] = latency_us(torch, fn)
            recs.append(kernel_record(torch, cfg, "spmm", w["name"], fn, 2.0 * nnz * n,
                                      spmm_bytes(m, k, n, nnz), flush, 200, ex))
            sfn = lambda: sp.sp_sddmm(m, k, d, nnz, order, ro, cols, x, y, out)
            ex = dict(tag)
            if cfg != "imbalance":
                ex["single_launch_us"] = latency_us(torch, sfn)
            recs.append(kernel_record(torch, cfg, "sddmm", w["name"], sfn, 2.0 * nnz * d,
                                      sddmm_bytes(m, k, d, nnz), flush, 200, ex))
            if cfg == "imbalance":
                bfn = lambda: sp.sp_spmm_balanced(m, k, n, nnz, order, vals, ro, cols, b, c)
                recs.append(kernel_record(torch, cfg, "spmm_balanced", w["name"], bfn,
                                          2.0 * nnz * n, spmm_bytes(m, k, n, nnz), flush, 200,
                                          tag))
                bsfn = lambda: sp.sp_sddmm_balanced(m, k, d, nnz, order, ro, cols, x, y, out)
                recs.append(kernel_record(torch, cfg, "sddmm_balanced", w["name"], bsfn,
                                          2.0 * nnz * d, sddmm_bytes(m, k, d, nnz), flush, 200,
                                          tag))

    # ---- ResNet-50 1x1 conv (1024 x 256 at 70 %, N = 6272)
    w = inputs.resnet_1x1()
    a = w["a"]
    m, k, n, nnz = w["m"], w["k"], w["n"], a.nnz
    ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
    b = up(w["b"])
    c = torch.empty(m, n, device=dev)
    fn = lambda: sp.sp_spmm(m, k, n, nnz, ri, vals, ro, cols, b, c)
    recs.append(kernel_record(torch, "resnet50_1x1", "spmm", w["name"], fn, 2.0 * nnz * n,
                              spmm_bytes(m, k, n, nnz), flush, 50,
                              {"m": m, "k": k, "n": n, "nnz": nnz,
                               "variant": kname(m, k, n, nnz, vals, cols, b, c, ri)}))
    del b, c

    # ---- sparse attention: 32 (batch, head) pairs over one 4096 x 4096 mask
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
    tag = {"batch": bh, "seq": seq, "head_dim": hd, "nnz_per_head": nnz}
    sfn = lambda: sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                      bh, seq * hd, seq * hd, nnz)
    smfn = lambda: sp.sp_csr_row_softmax(seq, nnz, ri, ro, s_out, s_out, bh, nnz, nnz)
    pfn = lambda: sp.sp_spmm_batched(seq, seq, hd, nnz, ri, p_vals, ro, cols, v, o, bh, nnz,
                                     seq * hd, seq * hd)
    afn = lambda: sp.sp_sparse_attention(seq, seq, hd, nnz, ri, ro, cols, q, kk, v, 0.125, o,
                                         bh, seq * hd, seq * hd, seq * hd, seq * hd)
    sb, pb = sddmm_bytes(seq, seq, hd, nnz), spmm_bytes(seq, seq, hd, nnz)
    recs.append(kernel_record(torch, "sparse_attention", "sddmm_x32", w["name"], sfn,
                              2.0 * bh * nnz * hd, bh * sb, flush, 20, tag))
    # the softmax moves 8 bytes per entry (read, write) and does no FMA work
    recs.append(kernel_record(torch, "sparse_attention", "row_softmax_x32", w["name"], smfn,
                              0.0, bh * 8.0 * nnz + 8 * seq, flush, 20, tag))
    # scores and their row softmax in one launch: the SDDMM's traffic
    fsfn = lambda: sp.sp_sddmm_softmax(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                       bh, seq * hd, seq * hd, nnz)
    recs.append(kernel_record(torch, "sparse_attention", "sddmm_softmax_x32", w["name"], fsfn,
                              2.0 * bh * nnz * hd, bh * sb, flush, 20, tag))
    recs.append(kernel_record(torch, "sparse_attention", "spmm_x32", w["name"], pfn,
                              2.0 * bh * nnz * hd, bh * pb, flush, 20, tag))
    recs.append(kernel_record(torch, "sparse_attention", "attention_one_pass_x32", w["name"], afn,
                              4.0 * bh * nnz * hd, bh * (4 * seq * hd * 3 + 4 * seq * hd
                                                         + 4 * nnz + 8 * seq), flush, 20, tag))
    del q, kk, v, s_out, p_vals, o

    # ---- the row swizzle of many rows: the rank sort (no workspace) against
    # the radix sort (workspace form), at 65,536 and 1,100,000 rows
    for m, seed in ((65536, 31), (1100000, 32)):
        k = 8192
        lengths = np.random.default_rng(seed).integers(0, 1639, m).astype(np.int32)
        ro = torch.empty(m + 1, dtype=torch.int32, device=dev)
        sp.sp_csr_offsets_from_lengths(m, up(lengths), ro)
        ri = torch.empty(m, dtype=torch.int32, device=dev)
        ws = torch.empty(sp.sp_row_swizzle_workspace(m), dtype=torch.uint8, device=dev)
        radix = lambda: sp.sp_row_swizzle_ws(m, k, ro, ri, ws)
        rank = lambda: sp.sp_row_swizzle(m, ro, ri)
        rec = {"config": "row_swizzle", "kernel": "row_swizzle", "m": m, "k": k,
               "radix_us": graph_time_us(torch, radix, 20),
               "rank_us": graph_time_us(torch, rank, 3 if m > 100000 else 10)}
        log(f"[row_swizzle] m={m}: radix {rec['radix_us']:.1f} us, rank {rec['rank_us']:.1f} us")
        recs.append(rec)

    # ---- single-launch latency at 98 % sparsity (LSTM layer)
    wl = inputs.lstm(0.98)
    rol, ril, coll, vall = upload_csr(torch, sp, dev, wl["a"])
    bl = up(wl["b"])
    cl = torch.empty(wl["m"], wl["n"], device=dev)
    nl = wl["a"].nnz
    fn = lambda: sp.sp_spmm(wl["m"], wl["k"], wl["n"], nl, ril, vall, rol, coll, bl, cl)
    recs.append({"config": "lstm", "kernel": "spmm_latency", "workload": wl["name"],
                 "single_launch_us": latency_us(torch, fn), "graph_us": graph_time_us(torch, fn, 200)})
    return recs


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
        if records is not None:
            rec = kernel_record(torch, "lstm", "spmm", w["name"], fn, 2.0 * a.nnz * n,
                                spmm_bytes(m, k, n, a.nnz), flush, reps,
                                {"sparsity": s, "m": m, "k": k, "n": n, "nnz": a.nnz,
                                 "variant": sp.sp_spmm_kernel_name(m, k, n, a.nnz, vals, cols,
                                                                   b, c, row_indices=ri)})
            records.append(rec)
            times[s] = rec["us"]
        else:
            times[s] = graph_time_us(torch, fn, reps)
        if dense_us is None:
            # The dense operand of the comparison: A with every entry present.
            dense_a = torch.from_numpy(inputs.random_dense(5, m, k, std=0.02)).to(dev)
            dfn = lambda: torch.mm(dense_a, b, out=c)
            dense_us = graph_time_us(torch, dfn, reps)
            if records is not None:
                records.append({"config": "lstm", "kernel": "dense_gemm",
                                "workload": "lstm_8192x2048x128_dense",
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


def profile_workload_fns(torch, sp, inputs, dev, wanted):
    """Launch functions of the named workloads, for rocprofv3 passes: resnet
    (the ResNet-50 1x1 SpMM), lstm90 / lstm50 (the LSTM-sized SpMM at 90 % and
    50 %), attention (the four sparse-attention kernels over 32 heads),
    resnet_wide / lstm50_wide (the SpMM on the wide kernel, as a 2-entry
    batch), and ffn_dk / attention_dk (the general SDDMM with Y stored d x k,
    no workspace)."""
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    fns = []

    def imbalance_fns():
        # lognormal rows: the SpMM swizzled (the balanced kernel) and natural
        # (the wide kernel), and the SDDMM swizzled (windows on four waves)
        if "imbalance" not in wanted:
            return []
        w = inputs.imbalance()
        a = w["a"]
        m, k, n, d, nnz = w["m"], w["k"], w["n"], w["d"], a.nnz
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b, x, y = up(w["b"]), up(w["x"]), up(w["y"])
        c = torch.empty(m, n, device=dev)
        out = torch.empty(nnz, device=dev)
        return [lambda: sp.sp_spmm(m, k, n, nnz, ri, vals, ro, cols, b, c),
                lambda: sp.sp_spmm(m, k, n, nnz, None, vals, ro, cols, b, c),
                lambda: sp.sp_sddmm(m, k, d, nnz, ri, ro, cols, x, y, out)]

    gens = {"resnet": inputs.resnet_1x1, "lstm90": lambda: inputs.lstm(0.9),
            "lstm50": lambda: inputs.lstm(0.5)}
    for name, gen in gens.items():
        # "<name>_wide": the same problem twice as a 2-entry batch (shared A
        # and B), which never takes the panel kernel: the wide kernel's
        # counters for the problem are half the dispatch's
        for wide in (False, True):
            if (name + ("_wide" if wide else "")) not in wanted:
                continue
            w = gen()
            a = w["a"]
            ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
            b = up(w["b"])
            m, k, n, nnz = w["m"], w["k"], w["n"], a.nnz
            if wide:
                c = torch.empty(2, m, n, device=dev)
                fns.append(lambda m=m, k=k, n=n, nnz=nnz, ri=ri, vals=vals, ro=ro, cols=cols,
                           b=b, c=c: sp.sp_spmm_batched(m, k, n, nnz, ri, vals, ro, cols, b, c,
                                                        2, 0, 0, m * n))
            else:
                c = torch.empty(m, n, device=dev)
                fns.append(lambda m=m, k=k, n=n, nnz=nnz, ri=ri, vals=vals, ro=ro, cols=cols,
                           b=b, c=c: sp.sp_spmm(m, k, n, nnz, ri, vals, ro, cols, b, c))
    if "ffn_dk" in wanted:
        # the general SDDMM on the FFN shapes, Y stored d x k, no workspace
        w = inputs.transformer_ffn()
        a = w["a"]
        m, k, d = w["m"], w["k"], w["d"]
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        x, y_dk = up(w["x"]), up(w["y"]).t().contiguous()
        out = torch.zeros(a.nnz, device=dev)
        fns.append(lambda: sp.sp_sddmm_general(m, k, d, a.nnz, ri, ro, cols, vals, x, y_dk,
                                               sp.SP_Y_DK, 0.5, 1.0, out))
    if "attention" in wanted or "attention_dk" in wanted:
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
        if "attention_dk" in wanted:
            # the scores with K stored d x k per head, no workspace
            kt = kk.transpose(1, 2).contiguous()
            fns.append(lambda: sp.sp_sddmm_general(seq, seq, hd, nnz, ri, ro, cols, None, q,
                                                   kt, sp.SP_Y_DK, 0.125, 0.0, s_out, bh, 0,
                                                   seq * hd, seq * hd, nnz))
        if "attention" not in wanted:
            return fns + imbalance_fns()
        fns += [lambda: sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125,
                                            s_out, bh, seq * hd, seq * hd, nnz),
                lambda: sp.sp_csr_row_softmax(seq, nnz, ri, ro, s_out, s_out, bh, nnz, nnz),
                lambda: sp.sp_spmm_batched(seq, seq, hd, nnz, ri, p_vals, ro, cols, v, o, bh,
                                           nnz, seq * hd, seq * hd),
                lambda: sp.sp_sparse_attention(seq, seq, hd, nnz, ri, ro, cols, q, kk, v,
                                               0.125, o, bh, seq * hd, seq * hd, seq * hd,
                                               seq * hd),
                lambda: sp.sp_sddmm_softmax(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125,
                                            s_out, bh, seq * hd, seq * hd, nnz)]
    return fns + imbalance_fns()


def stream_setup(torch, sp, inputs, dev, dtype=None, n=4):
    """The streaming regime: A 65536 x 8192 at 90 % sparsity (53.7 M entries,
    430 MB of CSR, far beyond L2 and MALL), B 8192 x n held in LDS (n = 8:
    in two column slices), natural row order; values and B fp32, or of the
    16-bit torch `dtype`.  Returns (launch, workload description)."""
    w = inputs.hbm_stream(n=n)
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
    """Beyond the default records: the general SDDMM (mask values, accumulation,
    Y stored k x d / d x k, with and without a workspace), the backward pass
    (transpose, values, A^T dY), 16-bit operands, the sparse-attention
    compositions (scores with K given d x k, scores + softmax in one pass, the
    all-device pipelines) and the streaming SpMM at n = 8 and 4.  Warm (graph
    back-to-back) and cold (after flushing the caches), one JSON record per
    kernel run."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB > caches
    flush.zero_()
    recs = []
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    # General SDDMM on the Transformer-FFN shapes: the mask's values as the
    # element-wise scale and accumulation into the previous output, with Y
    # stored k x d and d x k (d x k once more with a workspace: Y transposed
    # there first).
    w = inputs.transformer_ffn()
    a = w["a"]
    m, k, d = w["m"], w["k"], w["d"]
    ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
    x, y = up(w["x"]), up(w["y"])
    out = torch.empty(a.nnz, device=dev)
    y_dk = y.t().contiguous()
    ws = torch.empty(sp.sp_sddmm_general_workspace(k, d), dtype=torch.uint8, device=dev)
    for layout, yy, wsp, name in ((sp.SP_Y_KD, y, None, "kd"), (sp.SP_Y_DK, y_dk, None, "dk"),
                                  (sp.SP_Y_DK, y_dk, ws, "dk_workspace")):
        gfn = lambda: sp.sp_sddmm_general(m, k, d, a.nnz, ri, ro, cols, vals, x, yy,
                                          layout, 0.5, 1.0, out, workspace=wsp)
        recs.append(kernel_record(torch, "transformer_ffn", "sddmm_general_" + name, w["name"],
                                  gfn, 2.0 * a.nnz * d, sddmm_bytes(m, k, d, a.nnz) + 8 * a.nnz,
                                  flush, 200, {"mask_values": True, "beta": 1.0}))
    # Backward pass of a sparse layer: A^T in CSR (once per structure; the
    # values of a new A follow through the permutation), then dX = A^T dY on
    # the swizzled rows of A^T.
    for w in (inputs.transformer_ffn(), inputs.lstm(0.9)):
        recs.extend(backward_records(torch, sp, inputs, dev, w, flush))
    # Mixed precision: values and B (X and Y) in 16-bit, fp32 arithmetic.
    recs.extend(lowp_records(torch, sp, inputs, dev, flush))
    # Sparse attention compositions over one shared mask.
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
    o = torch.empty(bh, seq, hd, device=dev)
    kt = kk.transpose(1, 2).contiguous()
    tfn = lambda: sp.sp_sddmm_general(seq, seq, hd, nnz, ri, ro, cols, None, q, kt,
                                      sp.SP_Y_DK, 0.125, 0.0, s_out, bh, 0, seq * hd,
                                      seq * hd, nnz)
    kt_ws = torch.empty(sp.sp_sddmm_general_workspace(seq, hd, bh, seq * hd),
                        dtype=torch.uint8, device=dev)
    twfn = lambda: sp.sp_sddmm_general(seq, seq, hd, nnz, ri, ro, cols, None, q, kt,
                                       sp.SP_Y_DK, 0.125, 0.0, s_out, bh, 0, seq * hd,
                                       seq * hd, nnz, workspace=kt_ws)
    sfn = lambda: sp.sp_sddmm_batched(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                      bh, seq * hd, seq * hd, nnz)
    smfn = lambda: sp.sp_csr_row_softmax(seq, nnz, ri, ro, s_out, s_out, bh, nnz, nnz)
    fsfn = lambda: sp.sp_sddmm_softmax(seq, seq, hd, nnz, ri, ro, cols, q, kk, 0.125, s_out,
                                       bh, seq * hd, seq * hd, nnz)
    pv = lambda: sp.sp_spmm_batched(seq, seq, hd, nnz, ri, s_out, ro, cols, v, o, bh, nnz,
                                    seq * hd, seq * hd)

    def attention():
        sfn()
        smfn()
        pv()

    def attention_fused():
        fsfn()
        pv()

    sb, pb = sddmm_bytes(seq, seq, hd, nnz), spmm_bytes(seq, seq, hd, nnz)
    for kind, fn, flops, byts in (
            ("sddmm_general_dk_x32", tfn, 2.0 * bh * nnz * hd, bh * sb),
            ("sddmm_general_dk_workspace_x32", twfn, 2.0 * bh * nnz * hd, bh * sb),
            ("attention_all_device_x32", attention, 4.0 * bh * nnz * hd,
             bh * (sb + 8 * nnz + pb)),
            ("attention_all_device_fused_scores_x32", attention_fused, 4.0 * bh * nnz * hd,
             bh * (sb + pb))):
        recs.append(kernel_record(torch, "sparse_attention", kind, w["name"], fn, flops, byts,
                                  flush, 20, {"batch": bh, "seq": seq, "head_dim": hd,
                                              "nnz_per_head": nnz}))
    del q, kk, v, kt, s_out, o, kt_ws
    # The streaming regime: CSR far larger than every cache, n = 8 and n = 4
    # (B in LDS), natural and swizzled row order, fp32 and 16-bit.
    for n_cols in (8, 4):
        w = inputs.hbm_stream(n=n_cols)
        a = w["a"]
        ro, ri, cols, vals = upload_csr(torch, sp, dev, a)
        b = up(w["b"])
        c = torch.empty(w["m"], w["n"], device=dev)
        for order in (None, ri):
            fn = lambda: sp.sp_spmm(w["m"], w["k"], w["n"], a.nnz, order, vals, ro, cols, b, c)
            recs.append(kernel_record(torch, "hbm_stream", "spmm", w["name"], fn,
                                      2.0 * a.nnz * w["n"],
                                      spmm_bytes(w["m"], w["k"], w["n"], a.nnz), flush, 20,
                                      {"swizzle": order is not None}))
        for tag, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
            v16, b16 = vals.to(tdt), b.to(tdt)
            fn = lambda: sp.sp_spmm_ex(w["m"], w["k"], w["n"], a.nnz, None, v16, ro, cols,
                                       b16, c)
            byts = 6 * a.nnz + 4 * (w["m"] + 1) + 2 * w["k"] * w["n"] + 4 * w["m"] * w["n"]
            recs.append(kernel_record(torch, "hbm_stream", "spmm_" + tag, w["name"], fn,
                                      2.0 * a.nnz * w["n"], byts, flush, 20))
            del v16, b16
        del a, ro, ri, cols, vals
    with open(path, "w") as f:
        for r in recs:
            f.write(json.dumps(r) + "\n")


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
        flush = None
        if args.profile_cold:
            flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
            flush.zero_()

        def launches(fn):
            for _ in range(args.profile_launches):
                if flush is not None:
                    flush.add_(1.0)
                fn()

        wanted = set(args.profile_workloads.split(","))
        if "ffn" in wanted:
            for fn in (k_build, k_offsets, k_swizzle, k_spmm, k_sddmm, k_fused):
                launches(fn)
        for fn in profile_workload_fns(torch, sp, inputs, dev, wanted):
            launches(fn)
        if args.profile_stream:
            fn, _ = stream_setup(torch, sp, inputs, dev)
            launches(fn)
        if "stream8" in wanted:
            fn, _ = stream_setup(torch, sp, inputs, dev, n=8)
            launches(fn)
        if "transpose" in wanted:
            # the CSR transpose of the LSTM layer at 90 % (radix method: a
            # chain of launches per call)
            w = inputs.lstm(0.9)
            a = w["a"]
            m, k, nnz = w["m"], w["k"], a.nnz
            ro, _, cols, vals = upload_csr(torch, sp, dev, a)
            ws = torch.empty(sp.sp_csr_transpose_workspace(m, k, nnz), dtype=torch.uint8,
                             device=dev)
            t_ro = torch.empty(k + 1, dtype=torch.int32, device=dev)
            t_ci = torch.empty(nnz, dtype=torch.int32, device=dev)
            t_v = torch.empty(nnz, device=dev)
            t_p = torch.empty(nnz, dtype=torch.int32, device=dev)
            launches(lambda: sp.sp_csr_transpose(m, k, nnz, ro, cols, vals, t_ro, t_ci, t_v,
                                                 t_p, ws))
        # a plain copy of known size, to calibrate the byte counters
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        launches(lambda: dst.copy_(src))
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

    # Every seeded workload, warm and cold, against its roofline; the LSTM
    # sweep with its dense comparison gives the break-even sparsity.
    flush = None
    if not args.no_configs or not args.no_breakeven:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB > L2 + MALL
        flush.zero_()
    records = []
    if not args.no_configs:
        records.extend(config_records(torch, sp, inputs, dev, flush))
    if not args.no_breakeven:
        result["breakeven"] = lstm_breakeven(torch, sp, inputs, dev, records=records, flush=flush)
    if records:
        result["records"] = records
    del flush

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
