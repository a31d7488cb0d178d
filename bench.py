#!/usr/bin/env python3
"""Throughput of the block-scaled FP8 GEMM path on one MI355X.

Default workload: the dense FP8 NT sweep, M in {64, 128, 4096} x (N, K) in
{(2112,7168), (24576,1536), (32768,512), (7168,16384), (4096,7168), (7168,2048)}
with 1x128 activation / 128x128 weight scales and bf16 output, synthetic
seeded inputs (moe_grouped_matmul_amd.workloads).  One step = for each of the
18 shapes: quantise the fp32 activations (dg_quant_1x128) and run the GEMM
(dg_fp8_gemm_nt).  Weights are quantised once beforehand (offline, as in
inference).  Every shape rotates over enough copies of its buffers that each
call reads cold HBM (> 2x the 256 MB Infinity Cache per shape).

Timing: every step is captured into a HIP graph (one per rotation index) and
the timed region replays them back to back, so no host launch gaps enter the
measurement; per-shape kernel times come from graphs of back-to-back launches
over all rotating buffer sets, timed with HIP events on the launch stream.

Output: one JSON line with the whole-step FP8 TFLOPS, per-shape GEMM TFLOPS,
GB/s and fraction of the MI355X roofline, the dominant kernel's roofline, and
the CPU oracle timed on a bounded sample of the same workload.

The default run also times the M-grouped calls beside the step (not part of
`value`): the contiguous form (8 experts, tokens per expert uniform in
[1, 8192], (N, K) in {(4096, 7168), (7168, 2048)}), the masked form
(32 experts x 256 rows, masked_m uniform in [0, 256], same (N, K)) and its
decode-sized configuration (32 experts x 128 rows, masked_m uniform in
[0, 128]), each call over rotating buffer sets; their rows join `per_shape`
and `roofline_by_form` holds one roofline per form (--no-grouped skips them).

Other workloads: --workload large | small (one dense shape), contiguous | masked
(the M-grouped forms as the timed step), masked_decode (the masked form with
32 experts x 128 rows, masked_m uniform in [0, 128]), bf16 | acc | kgrouped |
ue8m0 (the BF16, accumulating, K-grouped and UE8M0-scale variants).
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA (published, no sparsity)
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA (published, no sparsity)
ROTATE_BYTES = 768 << 20  # per-shape rotation footprint (3x the 256 MB MALL)
CPU_SAMPLE_ROWS = 2048  # rows per shape in the CPU-oracle baseline sample
COPY_CAL_BYTES = 1 << 30  # plain device copy used to calibrate the HBM byte counters
# HBM bytes per launch of the dominant kernel, measured with rocprofv3 FETCH_SIZE /
# WRITE_SIZE counters (calibrated against a plain copy) and recorded together with
# a hash of the kernel's sources (code only, comments stripped): reported only
# while that code is unchanged.
TRAFFIC_RECORDS = {
    "sweep": os.path.join(ROOT, "profiles", "traffic_fp8_gemm_wide_kernel_dense_sweep.md"),
    "masked": os.path.join(ROOT, "profiles", "traffic_fp8_gemm_persistent_kernel_masked_4096x7168.md"),
    "masked_decode": os.path.join(ROOT, "profiles", "traffic_fp8_gemm_persistent_kernel_masked_decode_4096x7168.md"),
    "contiguous": os.path.join(ROOT, "profiles", "traffic_fp8_gemm_wide_kernel_contiguous_4096x7168.md"),
}
CLOCK_RECORDS = {
    "fp8_gemm_wide_kernel": os.path.join(ROOT, "profiles", "counters_fp8_gemm_wide_kernel_4096x7168x16384.md"),
}
KERNEL_SOURCES = ("moe_grouped_matmul_amd/csrc/gemm_persist.hip", "moe_grouped_matmul_amd/csrc/gemm_wide.hip",
                  "moe_grouped_matmul_amd/csrc/gemm_common.hpp",
                  "moe_grouped_matmul_amd/csrc/dg_internal.hpp", "moe_grouped_matmul_amd/csrc/api.cpp",
                  "moe_grouped_matmul_amd/build.py")


def _code_only(text, python):
    """Source text with comments and blank space removed, so a record stays
    tied to the code that was measured and not to its comments.  C-family
    files: // and /* */ comments outside string and character literals;
    Python: lines that are only a comment."""
    if python:
        lines = [l.rstrip() for l in text.splitlines() if l.strip() and not l.lstrip().startswith("#")]
        return "\n".join(lines)
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            k = text.find("*/", i + 2)
            i = n if k < 0 else k + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return "\n".join(" ".join(l.split()) for l in "".join(out).splitlines() if l.strip())


def kernel_source_hash():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_code_only(f.read(), rel.endswith(".py")).encode())
    return h.hexdigest()


def _record_fields(path, kernel):
    """The "- key: value" fields of a committed counter record, or None when the
    record is missing, is for another kernel, or predates the sources."""
    try:
        with open(path) as f:
            fields = dict(l.strip()[2:].split(": ", 1) for l in f if l.startswith("- ") and ": " in l)
    except OSError:
        return None
    if fields.get("kernel") != kernel or fields.get("source_sha256") != kernel_source_hash():
        return None
    return fields


def recorded_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter record, or None when the
    record is missing, is for another kernel/workload, or predates the sources."""
    fields = _record_fields(TRAFFIC_RECORDS[workload], kernel) if workload in TRAFFIC_RECORDS else None
    if fields is None or fields.get("workload") != workload:
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def recorded_clock(kernel):
    """Achieved shader clock and MFMA-busy fraction of a kernel from its committed
    rocprofv3 counter record (SQ_BUSY_CYCLES over the 32 shader engines against
    the dispatch time; SQ_VALU_MFMA_BUSY_CYCLES over the 1024 SIMDs), or None.
    The clock's published peak, 2.4 GHz, underlies the 5.0 PF FP8 peak."""
    fields = _record_fields(CLOCK_RECORDS[kernel], kernel) if kernel in CLOCK_RECORDS else None
    if fields is None:
        return None
    try:
        return dict(clock_ghz=float(fields["clock_ghz"]), clock_peak_ghz=2.4, mfma_busy=float(fields["mfma_busy"]),
                    clock_record=os.path.relpath(CLOCK_RECORDS[kernel], ROOT) + " (" + fields["workload"] + ")")
    except (KeyError, ValueError):
        return None


def dense_work(M, N, K):
    """Algorithmic FLOPs and HBM bytes of one dense call (valid rows only)."""
    flops = 2.0 * M * N * K
    nbytes = M * K + 4 * M * (K // 128) + N * K + 4 * ((N + 127) // 128) * (K // 128) + 2 * M * N
    return flops, float(nbytes)


def grouped_work(rows_per_group, N, K, index_bytes):
    flops = 0.0
    nbytes = float(index_bytes)
    for r in rows_per_group:
        if r <= 0:
            continue
        flops += 2.0 * r * N * K
        nbytes += r * K + 4 * r * (K // 128) + N * K + 4 * ((N + 127) // 128) * (K // 128) + 2 * r * N
    return flops, nbytes


def roof_time_us(flops, nbytes):
    return max(flops / (PEAK_FP8_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sweep", choices=["sweep", "large", "small", "contiguous", "masked",
                                                              "masked_decode", "bf16", "acc", "kgrouped", "ue8m0"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-grouped", action="store_true",
                    help="sweep only: skip the per-call timing of the contiguous and masked calls")
    ap.add_argument("--shapes", default="",
                    help="comma-separated indices into the workload's shape list (default: all; the sweep has 18, "
                         "the grouped workloads 2)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (reference dispatch for HBM byte counters)")
    return ap.parse_args()


class Timer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.torch.cuda.current_stream())
        return e


def capture(torch, fn):
    """Capture fn's launches into a HIP graph (replayed back to back on the GPU,
    so the timed region holds no host launch gaps)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graph(torch, timer, g, reps):
    """Average milliseconds of one replay of g over reps replays (after one untimed)."""
    g.replay()
    torch.cuda.synchronize()
    e0 = timer.ev()
    for _ in range(reps):
        g.replay()
    e1 = timer.ev()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def timed_steps(torch, timer, step, args):
    """Milliseconds per step (and wall seconds) over exactly args.steps steps,
    step indices warmup .. warmup + steps - 1, captured into one HIP graph so
    the GPU runs them back to back with no host or graph-launch gap between
    steps; one untimed replay first, the timed replay bracketed by device
    synchronisation."""
    g = capture(torch, lambda: [step(args.warmup + i) for i in range(args.steps)])
    g.replay()
    torch.cuda.synchronize()
    t0 = timer.ev()
    w0 = time.perf_counter()
    g.replay()
    t1 = timer.ev()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = t0.elapsed_time(t1) / args.steps
    del g
    return ms, wall


PER_SHAPE_LAUNCHES = 16  # minimum launches per per-shape timing graph (cycling over the rotating buffer sets)
PER_SHAPE_REPS = 5       # timed replays of each per-shape graph


def run_dense(args, torch, dg, workloads):
    dev = torch.device("cuda:0")
    shapes = workloads.CONFIGS["dense_sweep"] if args.workload == "sweep" else \
        workloads.CONFIGS["dense_large"] if args.workload == "large" else workloads.CONFIGS["dense_small"]
    if args.shapes:
        shapes = [shapes[int(i)] for i in args.shapes.split(",")]
    prepared = []
    for s in shapes:
        M, N, K = s["M"], s["N"], s["K"]
        a32, b32 = workloads.dense(M, N, K, s["seed"])
        A32 = torch.from_numpy(a32).to(dev)
        B32 = torch.from_numpy(b32).to(dev)
        B8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
        SB = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=dev)
        dg.dg_quant_128x128(B32, B8, SB)  # offline weight quantisation
        del B32
        per_set = A32.numel() * 4 + M * K + 4 * M * (K // 128) + N * K + SB.numel() * 4 + 2 * M * N
        nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
        sets = []
        for i in range(nsets):
            sets.append(dict(
                a32=A32 if i == 0 else A32.clone(),
                a8=torch.empty((M, K), dtype=torch.uint8, device=dev),
                sa=torch.empty((K // 128, M), dtype=torch.float32, device=dev),
                b8=B8 if i == 0 else B8.clone(),
                sb=SB if i == 0 else SB.clone(),
                d=torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        wsz = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, M, N, K, 1)
        ws = torch.zeros(max(wsz // 4, 1), dtype=torch.float32, device=dev) if wsz else None
        flops, nbytes = dense_work(M, N, K)
        plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT, M, N, K, 1)
        kernel = ("fp8_gemm_wide_kernel" if "kernel=wide" in plan else
                  "fp8_gemm_persistent_kernel<dense>" if "kernel=persistent" in plan else
                  "fp8_gemm_skinny_kernel" if "kernel=skinny" in plan else plan.split()[0] if plan else "?")
        prepared.append(dict(M=M, N=N, K=K, sets=sets, ws=ws, flops=flops, bytes=nbytes, kernel=kernel))
    torch.cuda.synchronize()
    timer = Timer(torch)

    def quant(p, i):
        st = p["sets"][i % len(p["sets"])]
        dg.dg_quant_1x128(st["a32"], st["a8"], st["sa"])

    def gemm(p, i):
        st = p["sets"][i % len(p["sets"])]
        dg.dg_fp8_gemm_nt(st["a8"], st["sa"], st["b8"], st["sb"], st["d"], p["ws"])

    def step(i):
        for p in prepared:
            quant(p, i)
            gemm(p, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # step i runs on buffer set i (mod the set count) of every shape
    ms_per_step, wall = timed_steps(torch, timer, step, args)

    # per-shape kernel times: graphs of back-to-back launches over the rotating sets
    per_shape = []
    for p in prepared:
        launches = max(PER_SHAPE_LAUNCHES, len(p["sets"]))  # every set once per replay: cold HBM
        gq = capture(torch, lambda p=p: [quant(p, i) for i in range(launches)])
        gg = capture(torch, lambda p=p: [gemm(p, i) for i in range(launches)])
        q_ms = time_graph(torch, timer, gq, PER_SHAPE_REPS) / launches
        g_ms = time_graph(torch, timer, gg, PER_SHAPE_REPS) / launches
        del gq, gg
        t_us = g_ms * 1e3
        rt = roof_time_us(p["flops"], p["bytes"])
        per_shape.append(dict(form="dense", M=p["M"], N=p["N"], K=p["K"], gemm_us=round(t_us, 2), quant_us=round(q_ms * 1e3, 2),
                              tflops=round(p["flops"] / t_us / 1e6, 1), gbs=round(p["bytes"] / t_us / 1e3, 1),
                              bound="mfma" if p["flops"] / (PEAK_FP8_TFLOPS * 1e12) >= p["bytes"] / (PEAK_HBM_GBS * 1e9)
                              else "hbm", roof_frac=round(rt / t_us, 4), kernel=p["kernel"]))
    step_flops = sum(p["flops"] for p in prepared)
    # dominant kernel: the one with the largest share of GEMM time
    by_kernel = {}
    for p, r in zip(prepared, per_shape):
        k = by_kernel.setdefault(p["kernel"], dict(us=0.0, flops=0.0, bytes=0.0, n=0))
        k["us"] += r["gemm_us"]
        k["flops"] += p["flops"]
        k["bytes"] += p["bytes"]
        k["n"] += 1
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["us"])
    avg_us = dom["us"] / dom["n"]
    mfma_bound = dom["flops"] / (PEAK_FP8_TFLOPS * 1e12) >= dom["bytes"] / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = dom["flops"] / dom["n"] / avg_us / 1e6
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_FP8_TFLOPS, 4))
    else:
        achieved = dom["bytes"] / dom["n"] / avg_us / 1e3
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    traffic = recorded_traffic(dom_name, args.workload) if not args.shapes else None
    roof.update(traffic=traffic, kernel=dom_name, launches_per_step=dom["n"], avg_launch_us=round(avg_us, 2),
                algorithmic_bytes_per_launch=round(dom["bytes"] / dom["n"]),
                algorithmic_flops_per_launch=round(dom["flops"] / dom["n"]))
    clock = recorded_clock(dom_name)
    if clock:
        roof.update(clock)
    return dict(ms_per_step=ms_per_step, wall_s=wall, step_flops=step_flops, per_shape=per_shape, roofline=roof,
                shapes=[(p["M"], p["N"], p["K"]) for p in prepared])


def run_grouped(args, torch, dg, workloads, form=None, timed=True):
    """M-grouped contiguous (8 experts, tokens per expert uniform in [1, 8192],
    segments padded to 128) or masked (32 experts x 256 capacity, masked_m
    uniform in [0, 256]) GEMMs for both (N, K) pairs.  Activations arrive
    already in e4m3 (as from an expert-parallel dispatch), so a step is the two
    grouped GEMM calls.  form: "contiguous" | "masked" | "masked_decode" (32
    experts x 128 capacity, masked_m uniform in [0, 128]) (default: the workload);
    timed=False measures only the per-call kernel times (graphs of
    back-to-back launches over the rotating sets), as the default sweep run
    does for the grouped forms."""
    dev = torch.device("cuda:0")
    form = form or args.workload
    cfgs = workloads.CONFIGS[form]
    if args.shapes and form == args.workload:
        cfgs = [cfgs[int(i)] for i in args.shapes.split(",")]
    prepared = []
    for c in cfgs:
        G, N, K = c["G"], c["N"], c["K"]
        if form == "contiguous":
            w = workloads.contiguous(G, N, K, c["seed"])
            rows_total = w["m_total"]
            A32 = torch.from_numpy(w["a"]).to(dev)
            q = torch.empty((A32.shape[0], K), dtype=torch.uint8, device=dev)
            s = torch.empty((K // 128, A32.shape[0]), dtype=torch.float32, device=dev)
            dg.dg_quant_1x128(A32, q, s)
            del A32
            rows_idx = torch.from_numpy(w["rows"]).to(dev)
            A8 = torch.full((rows_total, K), workloads.TRAP_CODE, dtype=torch.uint8, device=dev)
            SA = torch.full((K // 128, rows_total), float("nan"), dtype=torch.float32, device=dev)
            A8[rows_idx] = q
            SA[:, rows_idx] = s
            index = torch.from_numpy(w["m_indices"]).to(dev)
            flops, nbytes = grouped_work(w["counts"], N, K, 4 * rows_total)
            d_shape = (rows_total, N)
            counts = [int(x) for x in w["counts"]]
        else:
            max_m = c["max_m"]
            w = workloads.masked(G, max_m, N, K, c["seed"])
            A32 = torch.from_numpy(w["a"]).to(dev)
            q = torch.empty((A32.shape[0], K), dtype=torch.uint8, device=dev)
            s = torch.empty((K // 128, A32.shape[0]), dtype=torch.float32, device=dev)
            dg.dg_quant_1x128(A32, q, s)
            del A32
            rows_idx = torch.from_numpy(w["rows"]).to(dev)
            A8 = torch.full((G * max_m, K), workloads.TRAP_CODE, dtype=torch.uint8, device=dev)
            SAf = torch.full((K // 128, G * max_m), float("nan"), dtype=torch.float32, device=dev)
            A8[rows_idx] = q
            SAf[:, rows_idx] = s
            A8 = A8.view(G, max_m, K)
            SA = SAf.view(K // 128, G, max_m).permute(1, 0, 2).contiguous()
            index = torch.from_numpy(w["masked_m"]).to(dev)
            counts = [int(x) for x in w["masked_m"]]
            flops, nbytes = grouped_work(counts, N, K, 4 * G)
            d_shape = (G, max_m, N)
        B32 = torch.from_numpy(w["b"]).to(dev)
        B8 = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
        SB = torch.empty((G, (N + 127) // 128, K // 128), dtype=torch.float32, device=dev)
        dg.dg_quant_128x128(B32, B8, SB)
        del B32
        per_set = A8.numel() + SA.numel() * 4 + B8.numel() + SB.numel() * 4 + 2 * int(np.prod(d_shape))
        nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
        sets = [dict(a8=A8 if i == 0 else A8.clone(), sa=SA if i == 0 else SA.clone(),
                     b8=B8 if i == 0 else B8.clone(), sb=SB if i == 0 else SB.clone(),
                     d=torch.empty(d_shape, dtype=torch.bfloat16, device=dev)) for i in range(nsets)]
        if form == "contiguous":
            plan = dg.dg_describe_plan(dg.DG_OP_CONTIGUOUS, rows_total, N, K, G)
            kname = ("fp8_gemm_wide_kernel<contiguous>" if "kernel=wide" in plan
                     else "fp8_gemm_persistent_kernel<contiguous>")
        else:
            kname = "fp8_gemm_persistent_kernel<masked>"
        prepared.append(dict(G=G, N=N, K=K, sets=sets, index=index, flops=flops, bytes=nbytes, counts=counts,
                             rows=rows_total if form == "contiguous" else G * c["max_m"], kernel=kname))
    torch.cuda.synchronize()
    timer = Timer(torch)

    def gemm(p, i):
        st = p["sets"][i % len(p["sets"])]
        if form == "contiguous":
            dg.dg_m_grouped_fp8_gemm_nt_contiguous(st["a8"], st["sa"], st["b8"], st["sb"], st["d"], p["index"])
        else:
            dg.dg_m_grouped_fp8_gemm_nt_masked(st["a8"], st["sa"], st["b8"], st["sb"], st["d"], p["index"],
                                               expected_m=128)

    def step(i):
        for p in prepared:
            gemm(p, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, wall = timed_steps(torch, timer, step, args) if timed else (None, None)
    per_shape = []
    for p in prepared:
        launches = max(len(p["sets"]), 4)  # every set once per replay: cold HBM
        gg = capture(torch, lambda p=p: [gemm(p, i) for i in range(launches)])
        t_us = time_graph(torch, timer, gg, PER_SHAPE_REPS) / launches * 1e3
        del gg
        rt = roof_time_us(p["flops"], p["bytes"])
        mf = p["flops"] / (PEAK_FP8_TFLOPS * 1e12) >= p["bytes"] / (PEAK_HBM_GBS * 1e9)
        per_shape.append(dict(form=form, G=p["G"], N=p["N"], K=p["K"], rows=p["rows"],
                              valid_rows=int(sum(max(c, 0) for c in p["counts"])),
                              gemm_us=round(t_us, 2), tflops=round(p["flops"] / t_us / 1e6, 1),
                              gbs=round(p["bytes"] / t_us / 1e3, 1), bound="mfma" if mf else "hbm",
                              roof_frac=round(rt / t_us, 4), kernel=p["kernel"]))
    big = max(per_shape, key=lambda r: r["gemm_us"])
    if big["bound"] == "mfma":
        roof = dict(bound="mfma", achieved=big["tflops"], peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                    frac=round(big["tflops"] / PEAK_FP8_TFLOPS, 4))
    else:
        roof = dict(bound="hbm", achieved=big["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(big["gbs"] / PEAK_HBM_GBS, 4))
    big_p = next(p for p in prepared if p["N"] == big["N"] and p["K"] == big["K"])
    label = f"{big_p['kernel']} ({big['N']}x{big['K']})"
    roof.update(traffic=recorded_traffic(label, form), kernel=label,
                algorithmic_bytes_per_launch=round(big_p["bytes"]),
                algorithmic_flops_per_launch=round(big_p["flops"]),
                avg_launch_us=big["gemm_us"])
    name = {"contiguous": "m_grouped_contiguous_8x_tokens_1to8192", "masked": "m_grouped_masked_32x256",
            "masked_decode": "m_grouped_masked_32x128"}[form]
    config = dict(workload=name, shapes=[f"G={p['G']} N={p['N']} K={p['K']}" for p in prepared],
                  step="grouped GEMM per (N,K) pair", cold_hbm=True)
    return dict(ms_per_step=ms_per_step, wall_s=wall, step_flops=sum(p["flops"] for p in prepared),
                per_shape=per_shape, roofline=roof, name=name, config=config)


def cpu_baseline(shapes, workloads):
    """The CPU oracle as it stands, on the first min(M, CPU_SAMPLE_ROWS) rows of
    each shape: activation quantisation + GEMM timed (weights quantised
    beforehand, untimed), with the BLAS thread pool set to the cores this
    process may run on (os.sched_getaffinity)."""
    import oracle

    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None
    t_total = 0.0
    flops = 0.0
    for (M, N, K), s in shapes:
        rows = min(M, CPU_SAMPLE_ROWS)
        a32, b32 = workloads.dense(rows, N, K, s["seed"])
        qb, sb = oracle.quant_128x128(b32)
        t0 = time.perf_counter()
        qa, sa = oracle.quant_1x128(a32)
        oracle.gemm_nt(qa, sa, qb, sb)
        t_total += time.perf_counter() - t0
        flops += 2.0 * rows * N * K
    if limiter is not None:
        limiter.unregister()
    return dict(value=round(flops / t_total / 1e12, 5), unit="TFLOPS", cores=int(threads), kind="oracle",
                sample=f"first min(M,{CPU_SAMPLE_ROWS}) rows of each of the {len(shapes)} shapes: fp64 oracle 1x128 quantisation "
                       f"+ promoted GEMM + bf16 rounding ({flops / 1e9:.1f} GFLOP in {t_total:.1f} s); "
                       "weights pre-quantised untimed")


def run_bf16(args, torch, dg, workloads):
    """BF16 dense GEMM 4096 x 7168 x 16384 (the second dense workload the
    pages measure): one step = one call over one of the rotating buffer sets."""
    dev = torch.device("cuda:0")
    M, N, K = 4096, 7168, 16384
    a, b = workloads.dense_bf16(M, N, K, seed=500)
    A = torch.from_numpy(a.view(np.int16)).to(dev)
    B = torch.from_numpy(b.view(np.int16)).to(dev)
    per_set = 2 * (M * K + N * K + M * N)
    nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
    sets = [dict(a=A if i == 0 else A.clone(), b=B if i == 0 else B.clone(),
                 d=torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for i in range(nsets)]
    wsz = dg.dg_get_workspace_size(dg.DG_OP_BF16_GEMM_NT, M, N, K, 1)
    ws = torch.zeros(max(wsz // 4, 1), dtype=torch.float32, device=dev) if wsz else None
    timer = Timer(torch)

    def step(i):
        st = sets[i % nsets]
        dg.dg_bf16_gemm_nt(st["a"], st["b"], st["d"], ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, _ = timed_steps(torch, timer, step, args)
    flops = 2.0 * M * N * K
    nbytes = 2.0 * (M * K + N * K + M * N)
    us = ms_per_step * 1e3
    achieved = flops / us / 1e6
    plan = dg.dg_describe_plan(dg.DG_OP_BF16_GEMM_NT, M, N, K, 1)
    kname = "fp8_gemm_wide_kernel<bf16>" if "kernel=wide" in plan else "fp8_gemm_persistent_kernel<bf16>"
    roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_BF16_TFLOPS, 4), traffic=None, kernel=kname,
                launches_per_step=1, avg_launch_us=round(us, 2), algorithmic_bytes_per_launch=round(nbytes),
                algorithmic_flops_per_launch=round(flops))
    per_shape = [dict(M=M, N=N, K=K, gemm_us=round(us, 2), tflops=round(achieved, 1),
                      gbs=round(nbytes / us / 1e3, 1), bound="mfma",
                      roof_frac=round(max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6 / us, 4),
                      kernel=kname)]
    config = dict(workload="dense_bf16_nt_4096x7168x16384", shapes=[f"{M}x{N}x{K}"], out="bf16",
                  step="dg_bf16_gemm_nt", cold_hbm=True)
    return dict(ms_per_step=ms_per_step, step_flops=flops, per_shape=per_shape, roofline=roof, name=config["workload"],
                config=config)


def run_acc(args, torch, dg, workloads):
    """Accumulating FP8 GEMM D = C + A.B^T (fp32 C, D in place) at
    4096 x 7168 x 16384: one step = one call over one rotating buffer set."""
    dev = torch.device("cuda:0")
    M, N, K = 4096, 7168, 16384
    a32, b32 = workloads.dense(M, N, K, 200)
    A32 = torch.from_numpy(a32).to(dev)
    B32 = torch.from_numpy(b32).to(dev)
    A8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    SA = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    B8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
    SB = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=dev)
    dg.dg_quant_1x128(A32, A8, SA)
    dg.dg_quant_128x128(B32, B8, SB)
    del A32, B32
    per_set = M * K + N * K + 4 * M * N
    nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
    sets = [dict(a=A8 if i == 0 else A8.clone(), sa=SA if i == 0 else SA.clone(), b=B8 if i == 0 else B8.clone(),
                 sb=SB if i == 0 else SB.clone(), c=torch.zeros((M, N), dtype=torch.float32, device=dev))
            for i in range(nsets)]
    wsz = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT, M, N, K, 1)
    ws = torch.zeros(max(wsz // 4, 1), dtype=torch.float32, device=dev) if wsz else None
    timer = Timer(torch)

    def step(i):
        st = sets[i % nsets]
        dg.dg_fp8_gemm_nt_acc(st["a"], st["sa"], st["b"], st["sb"], st["c"], st["c"], ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, _ = timed_steps(torch, timer, step, args)
    flops, nbytes = dense_work(M, N, K)
    nbytes += 6.0 * M * N  # fp32 C read and fp32 D written instead of bf16 D
    us = ms_per_step * 1e3
    achieved = flops / us / 1e6
    # the accumulating form takes 256 x 256 tiles by the dense rule
    plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT, M, N, K, 1)
    kname = "fp8_gemm_wide_kernel<acc>" if "kernel=wide" in plan else "fp8_gemm_persistent_kernel<acc>"
    roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_FP8_TFLOPS, 4), traffic=None, kernel=kname,
                launches_per_step=1, avg_launch_us=round(us, 2), algorithmic_bytes_per_launch=round(nbytes),
                algorithmic_flops_per_launch=round(flops))
    per_shape = [dict(M=M, N=N, K=K, gemm_us=round(us, 2), tflops=round(achieved, 1), gbs=round(nbytes / us / 1e3, 1),
                      bound="mfma", roof_frac=round(roof_time_us(flops, nbytes) / us, 4),
                      kernel=kname)]
    config = dict(workload="dense_fp8_nt_acc_4096x7168x16384", shapes=[f"{M}x{N}x{K}"], out="fp32 D = C + A.B^T",
                  step="dg_fp8_gemm_nt_acc (C = D, in place)", cold_hbm=True)
    return dict(ms_per_step=ms_per_step, step_flops=flops, per_shape=per_shape, roofline=roof, name=config["workload"],
                config=config)


UE8M0_DECODE = [(64, 2112, 7168), (128, 7168, 2048)]  # timed per call beside the step


def run_ue8m0(args, torch, dg, workloads):
    """Dense FP8 GEMM with UE8M0 (power-of-two) scales packed four per int32
    at 4096 x 7168 x 16384: one step = one GEMM call over one rotating set.
    Two decode shapes (rows <= 128, the skinny kernel) are timed per call
    beside the step and reported in per_shape only."""
    dev = torch.device("cuda:0")
    timer = Timer(torch)

    def prepare(M, N, K, seed):
        KW = (K // 128 + 3) // 4
        a32, b32 = workloads.dense(M, N, K, seed)
        A32 = torch.from_numpy(a32).to(dev)
        B32 = torch.from_numpy(b32).to(dev)
        A8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
        SA = torch.empty((KW, M), dtype=torch.int32, device=dev)
        B8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
        SB = torch.empty(((N + 127) // 128, KW), dtype=torch.int32, device=dev)
        dg.dg_quant_1x128_ue8m0(A32, A8, SA)
        dg.dg_quant_128x128_ue8m0(B32, B8, SB)
        del A32, B32
        per_set = M * K + N * K + 2 * M * N
        nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
        sets = [dict(a=A8 if i == 0 else A8.clone(), sa=SA if i == 0 else SA.clone(), b=B8 if i == 0 else B8.clone(),
                     sb=SB if i == 0 else SB.clone(), d=torch.empty((M, N), dtype=torch.bfloat16, device=dev))
                for i in range(nsets)]
        wsz = dg.dg_get_workspace_size(dg.DG_OP_GEMM_NT_UE8M0, M, N, K, 1)
        ws = torch.zeros(max(wsz // 4, 1), dtype=torch.float32, device=dev) if wsz else None

        def call(i):
            st = sets[i % nsets]
            dg.dg_fp8_gemm_nt_ue8m0(st["a"], st["sa"], st["b"], st["sb"], st["d"], ws)

        flops = 2.0 * M * N * K
        nbytes = float(M * K + N * K + 4 * M * KW + 4 * ((N + 127) // 128) * KW + 2 * M * N)
        return call, nsets, flops, nbytes

    def row(M, N, K, us, flops, nbytes):
        plan = dg.dg_describe_plan(dg.DG_OP_GEMM_NT_UE8M0, M, N, K, 1)
        kname = ("fp8_gemm_wide_kernel<ue8m0>" if "kernel=wide" in plan else
                 "fp8_gemm_skinny_kernel<ue8m0>" if "kernel=skinny" in plan else "fp8_gemm_persistent_kernel<ue8m0>")
        bound = "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) > flops / (PEAK_FP8_TFLOPS * 1e12) else "mfma"
        return dict(M=M, N=N, K=K, gemm_us=round(us, 2), tflops=round(flops / us / 1e6, 1),
                    gbs=round(nbytes / us / 1e3, 1), bound=bound, roof_frac=round(roof_time_us(flops, nbytes) / us, 4),
                    kernel=kname)

    M, N, K = 4096, 7168, 16384
    step, _, flops, nbytes = prepare(M, N, K, 200)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, _ = timed_steps(torch, timer, step, args)
    us = ms_per_step * 1e3
    achieved = flops / us / 1e6
    per_shape = [row(M, N, K, us, flops, nbytes)]
    roof = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                frac=round(achieved / PEAK_FP8_TFLOPS, 4), traffic=None, kernel=per_shape[0]["kernel"],
                launches_per_step=1, avg_launch_us=round(us, 2), algorithmic_bytes_per_launch=round(nbytes),
                algorithmic_flops_per_launch=round(flops))
    del step
    torch.cuda.empty_cache()
    for (m, n, k) in ([] if args.shapes else UE8M0_DECODE):
        call, nsets, f, b = prepare(m, n, k, 201)
        launches = max(16, nsets)
        g = capture(torch, lambda: [call(i) for i in range(launches)])
        per_shape.append(row(m, n, k, time_graph(torch, timer, g, 5) * 1e3 / launches, f, b))
        del g, call
        torch.cuda.empty_cache()
    config = dict(workload="dense_fp8_nt_ue8m0_4096x7168x16384", shapes=[f"{M}x{N}x{K}"],
                  per_call_only=[f"{m}x{n}x{k}" for (m, n, k) in UE8M0_DECODE] if not args.shapes else [],
                  scales="UE8M0 1x128 activations, 128x128 weights, four codes per int32", out="bf16",
                  step="dg_fp8_gemm_nt_ue8m0", cold_hbm=True)
    return dict(ms_per_step=ms_per_step, step_flops=flops, per_shape=per_shape, roofline=roof, name=config["workload"],
                config=config)


def kgrouped_work(M, N, counts, K):
    """Algorithmic work of one K-grouped call: flops of the valid tokens; bytes
    of both operands and their per-row scales over the padded K layout, fp32 C
    read and D written for every group, and the lengths."""
    G = len(counts)
    flops = 2.0 * M * N * float(sum(counts))
    nbytes = (M + N) * K + 4 * (M + N) * (K // 128) + 8.0 * G * M * N + 4 * G
    return flops, float(nbytes)


def run_kgrouped(args, torch, dg, workloads):
    """K-grouped contiguous weight-gradient GEMMs of 8 local experts (tokens
    per expert uniform in [0, 8192], segments padded to 128): the up
    projection (4096 x 7168) and the down projection (7168 x 2048), each
    accumulated in place into its fp32 gradient (C = D).  A step is the two
    calls."""
    dev = torch.device("cuda:0")
    prepared = []
    for c in workloads.CONFIGS["k_grouped"]:
        G, M, N = c["G"], c["M"], c["N"]
        w = workloads.k_grouped(G, M, N, c["seed"])
        K = int(w["ks"].sum())

        def quant(x):
            X = torch.from_numpy(x).to(dev)
            q = torch.empty(X.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty((K // 128, X.shape[0]), dtype=torch.float32, device=dev)
            dg.dg_quant_1x128(X, q, sc)
            del X
            return q, sc

        A8, SA = quant(w["a"])
        B8, SB = quant(w["b"])
        ks = torch.from_numpy(w["ks"]).to(dev)
        per_set = (M + N) * K + 4 * (M + N) * (K // 128) + 4 * G * M * N
        nsets = max(2, math.ceil(ROTATE_BYTES / per_set))
        sets = [dict(a8=A8 if i == 0 else A8.clone(), sa=SA if i == 0 else SA.clone(),
                     b8=B8 if i == 0 else B8.clone(), sb=SB if i == 0 else SB.clone(),
                     d=torch.zeros((G, M, N), dtype=torch.float32, device=dev)) for i in range(nsets)]
        flops, nbytes = kgrouped_work(M, N, [int(x) for x in w["counts"]], K)
        prepared.append(dict(G=G, M=M, N=N, K=K, sets=sets, ks=ks, flops=flops, bytes=nbytes))
        del w
    torch.cuda.synchronize()
    timer = Timer(torch)

    def gemm(p, i):
        st = p["sets"][i % len(p["sets"])]
        dg.dg_k_grouped_fp8_gemm_nt_contiguous(st["a8"], st["sa"], st["b8"], st["sb"], st["d"], st["d"], p["ks"])

    def step(i):
        for p in prepared:
            gemm(p, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_per_step, _ = timed_steps(torch, timer, step, args)
    per_shape = []
    for p in prepared:
        launches = max(len(p["sets"]), 4)
        gg = capture(torch, lambda p=p: [gemm(p, i) for i in range(launches)])
        t_us = time_graph(torch, timer, gg, PER_SHAPE_REPS) / launches * 1e3
        del gg
        per_shape.append(dict(G=p["G"], M=p["M"], N=p["N"], K=p["K"], gemm_us=round(t_us, 2),
                              tflops=round(p["flops"] / t_us / 1e6, 1), gbs=round(p["bytes"] / t_us / 1e3, 1),
                              bound="mfma", roof_frac=round(roof_time_us(p["flops"], p["bytes"]) / t_us, 4),
                              algorithmic_flops_per_launch=round(p["flops"]),
                              algorithmic_bytes_per_launch=round(p["bytes"])))
    big = max(per_shape, key=lambda r: r["gemm_us"])
    plan = dg.dg_describe_plan(dg.DG_OP_K_GROUPED, big["M"], big["N"], big["K"], big["G"])
    kname = "fp8_gemm_wide_kernel<k_grouped>" if "kernel=wide" in plan else "fp8_gemm_persistent_kernel<k_grouped>"
    roof = dict(bound="mfma", achieved=big["tflops"], peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                frac=round(big["tflops"] / PEAK_FP8_TFLOPS, 4), traffic=None,
                kernel=f"{kname} ({big['M']}x{big['N']})", avg_launch_us=big["gemm_us"])
    name = "k_grouped_wgrad_8x_tokens_0to8192"
    config = dict(workload=name, shapes=[f"G={p['G']} M={p['M']} N={p['N']} K={p['K']}" for p in prepared],
                  out="fp32 D[g] += A_g . B_g^T (in place)", step="dg_k_grouped_fp8_gemm_nt_contiguous per shape",
                  cold_hbm=True)
    return dict(ms_per_step=ms_per_step, step_flops=sum(p["flops"] for p in prepared), per_shape=per_shape,
                roofline=roof, name=name, config=config)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): the FP8 GEMM "
              "path is a per-GPU kernel, and runs over several GPUs are not implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    from moe_grouped_matmul_amd import dg, workloads

    if not os.path.exists(dg.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload in ("sweep", "large", "small"):
        r = run_dense(args, torch, dg, workloads)
        name = {"sweep": "dense_fp8_nt_sweep_18_shapes", "large": "dense_fp8_nt_4096x7168x16384",
                "small": "dense_fp8_nt_64x2112x7168"}[args.workload]
        config = dict(workload=name, shapes=[f"{m}x{n}x{k}" for m, n, k in r["shapes"]],
                      scales="1x128 activations, 128x128 weights, fp32", out="bf16",
                      step="dg_quant_1x128 + dg_fp8_gemm_nt per shape", cold_hbm=True)
        if args.workload == "sweep" and not args.no_grouped and not args.shapes:
            # the two M-grouped forms' calls, timed per call beside the step
            # (not part of `value`): per-call rows and one roofline per form
            r["roofline_by_form"] = {"dense": r["roofline"]}
            grouped_names = []
            for form in ("contiguous", "masked", "masked_decode"):
                torch.cuda.empty_cache()
                g = run_grouped(args, torch, dg, workloads, form=form, timed=False)
                r["per_shape"] = r["per_shape"] + g["per_shape"]
                r["roofline_by_form"][form] = g["roofline"]
                grouped_names.append(g["name"])
            config["per_call_only"] = grouped_names
    elif args.workload in ("bf16", "acc", "kgrouped", "ue8m0"):
        r = {"bf16": run_bf16, "acc": run_acc, "kgrouped": run_kgrouped, "ue8m0": run_ue8m0}[args.workload](
            args, torch, dg, workloads)
        name = r["name"]
        config = r["config"]
    else:
        r = run_grouped(args, torch, dg, workloads)
        name = r["name"]
        config = r["config"]

    value = r["step_flops"] / (r["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": "FP8 TFLOPS + GB/s per shape (dense/contig/masked), % of MI355X roofline",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.workload == "bf16" else "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) / N(0,1/K) bf16 operands)" if args.workload == "bf16" else
                "synthetic (seeded DeepSeek-V3-shaped fp32 sources, quantised on device)",
        "config": config,
        "per_shape": r["per_shape"],
        "roofline": r["roofline"],
    }
    if "roofline_by_form" in r:
        line["roofline_by_form"] = r["roofline_by_form"]
    if not args.no_cpu_baseline and args.workload in ("sweep", "large", "small"):
        shp = workloads.CONFIGS["dense_sweep"] if args.workload == "sweep" else \
            workloads.CONFIGS["dense_large"] if args.workload == "large" else workloads.CONFIGS["dense_small"]
        if args.shapes:
            shp = [shp[int(i)] for i in args.shapes.split(",")]
        line["cpu_baseline"] = cpu_baseline([((s["M"], s["N"], s["K"]), s) for s in shp], workloads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
