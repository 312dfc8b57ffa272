#!/usr/bin/env python3
"""Benchmark of the routed low-bit MoE expert layer on one MI355X.

One step = one pass of the hot path over one batch: routing (top-k +
counting sort) and the expert FFN (V-projections, gate/up + SwiGLU, down,
combine) on a seeded synthetic layer, through moeq_moe_forward (which runs
the gate/up projection beside the routing for decode batches); --no-fused
times moeq_route followed by moeq_expert_ffn.  Default workload: the
Mixtral-shaped decode layer (8 experts, top-2, H 4096, I 14336, 16 tokens,
int3 group-128 codes, rank-32 compensators).  Inputs are resident in HBM
before timing; weights rotate over several packed copies so that no step
finds them in the 256 MB last-level cache.

Prints one JSON line (see the repository's design notes for every field).
"""

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "expert-FFN tokens/s; decode HBM GB/s and prefill TFLOP/s as % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA peak, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
CSRC = os.path.join(ROOT, "bit_quantized_moe_token_amd", "csrc")


def kernel_source_hash():
    """Hash of every kernel source; stored counter readings are used only
    while it matches (any edit of a kernel makes them stale)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", choices=["decode", "prefill", "finegrained", "bitplane", "tiny"],
                   default="decode")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--tokens", type=int, default=0,
                   help="run the workload's layer with this many tokens instead of its own T (the "
                        "workload name and the summaries' file names follow)")
    p.add_argument("--path", type=int, default=0, help="moeq_path (0 = auto)")
    p.add_argument("--split-k", type=int, default=0, help="down-projection K splits (0 = automatic)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (reference kernel for counter scaling)")
    p.add_argument("--summarize-sq", nargs="+", metavar="DIR",
                   help="reduce a kernel trace and an SQ counter pass (MFMA, VALU) of the workload's command "
                        "(and, optionally, a pass of the stall and LDS counters) to "
                        "profiles/counters_<workload>.md")
    p.add_argument("--summarize-trace", metavar="TRACE_DIR",
                   help="no GPU work: reduce a rocprofv3 --kernel-trace --stats folder of the default "
                        "bench command to profiles/kernels_<workload>.md")
    p.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                   help="no GPU work: read two rocprofv3 --pmc output folders (FETCH_SIZE, "
                        "WRITE_SIZE) of a --copy-calibration run (and, optionally, the log of "
                        "the FETCH run's bench line) and record the scaled per-launch HBM "
                        "traffic of each kernel of the workload")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the extra measurements (prefill layer and the other three layers)")
    p.add_argument("--no-others", action="store_true",
                   help="skip the tiny, fine-grained and bit-plane layers (keep the prefill one)")
    p.add_argument("--graph", action="store_true",
                   help="replay each step from a captured HIP graph instead of launching it directly")
    p.add_argument("--no-fused", action="store_true",
                   help="time moeq_route followed by moeq_expert_ffn instead of moeq_moe_forward")
    return p.parse_args()


def build_layers(cfg, seed, copies, formats):
    """Quantize the seeded fp16 weights on the device and pack `copies`
    copies per requested (fmt, bits) variant.  Returns {name: [layers]}."""
    import numpy as np
    import torch
    from bit_quantized_moe_token_amd import moeq
    from synth import gen

    E = cfg["E"]
    blocks = {name: [] for name in formats}
    bits_of = {}
    for name, c in formats.items():
        bits_of[name] = gen.gen_bits(c, seed)
    factors = []
    for e in range(E):
        for blk in range(3):
            W = torch.from_numpy(gen.gen_weight_block(cfg, seed, e, blk)).cuda()
            for name, c in formats.items():
                blocks[name].append(moeq.quantize_block(W, c["fmt"], int(bits_of[name][e, blk]), c["G"]))
            if cfg["r"] and cfg.get("comp") == "svd":
                # rank-r truncation of the RTN residual, fitted on the device
                # (the first format's quantization; INT layers only)
                q = blocks[next(iter(formats))][-1]
                r = cfg["r"]
                l = min(r + 16, 128, *W.shape)
                omega = torch.from_numpy(gen.gen_test_matrix(cfg, seed, e, blk, l)).cuda()
                factors.append(moeq.fit_lowrank(W, q["codes"], q["scales"], q["zeros"], cfg["G"], omega, r, 2))
            elif cfg["r"]:
                f = gen.gen_factors(cfg, seed, e, blk)
                factors.append((torch.from_numpy(f[0]).cuda(), torch.from_numpy(f[1]).cuda()))
            del W
    shared = None
    if cfg.get("rs"):
        shared = []
        for g in range(gen.n_groups(cfg)):
            for blk in range(3):
                f = gen.gen_shared_factors(cfg, seed, g, blk)
                shared.append((torch.from_numpy(f[0]).cuda(), torch.from_numpy(f[1]).cuda()))
    out = {}
    for name, c in formats.items():
        out[name] = [moeq.PackedLayer(E, cfg["H"], cfg["I"], c["G"], c["fmt"], bits_of[name],
                                      blocks[name], factors if cfg["r"] else None, shared,
                                      cfg.get("share", 0))
                     for _ in range(copies[name])]
    torch.cuda.synchronize()
    del blocks
    return out


def algorithmic(cfg, layer, offsets, sorted_pairs, n_comp):
    """Algorithmic bytes and flops of one call from the actual routing:
    per active expert its codes (b bits/weight or top-q planes), fp16 scale
    + 1 B zero per (row, group) or its LUT, fp16 factors of blocks with a
    compensated pair (shared factors once per active group); x and y fp16.
    Flops: 2 m N K per block plus 2 r (N + K) per compensated pair and block.
    Also the bytes of the gate/up kernel alone (codes, metadata and U of the
    gate and up blocks, x read, h written)."""
    import numpy as np
    E, H, I, k, T = cfg["E"], cfg["H"], cfg["I"], cfg["k"], cfg["T"]
    r, rs = cfg["r"], cfg.get("rs", 0)
    counts = np.diff(offsets)
    comp_cnt = np.zeros(E, dtype=np.int64)
    for pos in range(len(sorted_pairs)):
        e = int(np.searchsorted(offsets, pos, side="right") - 1)
        if int(sorted_pairs[pos]) % k < n_comp:
            comp_cnt[e] += 1
    total, flops, gu = 0, 0.0, 0
    groups = set()
    for e in range(E):
        if counts[e] == 0:
            continue
        for blk in range(3):
            N, K = (I, H) if blk < 2 else (H, I)
            b = layer.block_bytes(e, blk)          # codes + metadata + U, V
            fac = (N + K) * r * 2
            body = b - fac
            total += body + (fac if comp_cnt[e] else 0)
            flops += 2.0 * counts[e] * N * K + 2.0 * (r + rs) * (N + K) * comp_cnt[e]
            if blk < 2:
                gu += body + (N * r * 2 if comp_cnt[e] else 0)
        if rs and comp_cnt[e]:
            groups.add(e // cfg["share"])
    for g in groups:
        for blk in range(3):
            total += layer.shared_bytes(g, blk)
            if blk < 2:
                N = I
                gu += N * rs * 2
    P = T * k
    total += 2 * T * H * 2
    gu += T * H * 2 + P * I * 2
    return dict(bytes=int(total), flops=float(flops), gateup_bytes=int(gu),
                active=int((counts > 0).sum()), counts=[int(c) for c in counts])


def time_steps(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def step_distribution(fn, steps):
    """Per-step event pairs on torch's stream (the library launches on it):
    median, p10 and p90 of the step time in ms, next to the block mean."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)

    def q(f):
        return ts[min(len(ts) - 1, int(f * len(ts)))]
    return dict(median=statistics.median(ts), p10=q(0.1), p90=q(0.9), n=len(ts))


def run_workload(cfg, layers_list, seed, steps, warmup, path, profile=True, graph=False, split_k=0, fused=True):
    import numpy as np
    import torch
    from bit_quantized_moe_token_amd import moeq
    from synth import gen

    T, k = cfg["T"], cfg["k"]
    x = torch.from_numpy(gen.gen_x(cfg, seed)).cuda()
    logits = torch.from_numpy(gen.gen_logits(cfg, seed)).cuda()
    rt = moeq.RoutingOut(T, cfg["E"], k, x.device)
    y = torch.empty((T, cfg["H"]), dtype=torch.float16, device=x.device)
    ws = moeq.FfnWorkspace(layers_list[0], T, k, path, split_k, forward=fused)
    R = len(layers_list)

    def step(i):
        # one pass of the hot path: routing and the expert layer
        if fused:
            moeq.moe_forward(layers_list[i % R], logits, x, k, cfg["n_comp"], routing=rt, out=y, ws=ws)
        else:
            moeq.route(logits, k, out=rt)
            moeq.expert_ffn(layers_list[i % R], x, rt, cfg["n_comp"], out=y, ws=ws, path=path, split_k=split_k)

    timed = step
    if graph:
        # one HIP graph per weight copy holding the step's launches (the
        # library's calls enqueue kernels only: no host syncs, no memsets)
        for i in range(R):
            step(i)
        torch.cuda.synchronize()
        graphs = []
        for i in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        torch.cuda.synchronize()

        def timed(i):
            graphs[i % R].replay()

    ms = time_steps(timed, steps, warmup)
    dist = step_distribution(timed, steps)
    prof = {}
    if profile:
        moeq.profile_enable(True)
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        prof = moeq.profile_read()
        moeq.profile_enable(False)
    torch.cuda.synchronize()
    offsets = rt.offsets.cpu().numpy()
    sp = rt.sorted_pairs.cpu().numpy()
    alg = algorithmic(cfg, layers_list[0], offsets, sp, cfg["n_comp"])
    alg["step_ms_dist"] = dist
    return ms, prof, alg


CALIB_BYTES = 1 << 30


def copy_calibration():
    """A plain elementwise copy (negation) of 1 GiB int8, 5 times: it reads
    and writes CALIB_BYTES once each, the reference for scaling counters."""
    import torch
    a = torch.empty(CALIB_BYTES, dtype=torch.int8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(a, out=b)
    torch.cuda.synchronize()


# rocprofv3 kernel names -> the names the library's own profiler uses
# kernel name pattern -> key; the tiled kernels' names contain the streaming
# kernels' names, so they are matched first
KERNEL_KEYS = [("tiled_gateup", "gateup_tiled"), ("tiled_down", "down_tiled"),
               ("gateup_kernel", "gateup_stream"), ("down_kernel", "down_stream"),
               ("route", "route"), ("combine", "combine"), ("neg_kernel", "calibration_copy")]


def route_scaling(reps=20):
    """moeq_route alone on seeded N(0, 1) logits, 128 experts, top-8, at
    batches from 512 to 32768 tokens: beyond 4096 tokens the sort counts
    through a workspace, so its time should grow about linearly."""
    import numpy as np
    import torch
    from bit_quantized_moe_token_amd import moeq
    res = []
    for T in (512, 4096, 8192, 32768):
        logits = torch.from_numpy(np.random.default_rng([0, T]).standard_normal((T, 128)).astype(np.float32)).cuda()
        rt = moeq.RoutingOut(T, 128, 8, logits.device)
        ms = time_steps(lambda i: moeq.route(logits, 8, out=rt), reps, 3)
        res.append(dict(T=T, us=ms * 1e3))
        del logits, rt
    return dict(E=128, k=8, what="moeq_route, mean of %d calls" % reps, batches=res)


def hbm_context(reps=10):
    """Plain torch streaming kernels over 1 GiB (a read-only sum and a copy),
    timed with events on torch's stream: what simple streaming code reaches
    on this GPU, as context for the HBM fractions (the peak stays 8 TB/s)."""
    import torch
    n = 1 << 28                                    # 1 GiB of fp32
    a = torch.full((n,), 1.0, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)

    def med(fn):
        ts = []
        for i in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        return statistics.median(ts)

    t_read = med(lambda: a.sum())
    t_copy = med(lambda: b.copy_(a))
    del a, b
    torch.cuda.empty_cache()
    read = (n * 4) / t_read / 1e9
    copy = (2 * n * 4) / t_copy / 1e9
    return dict(read_GBps=read, read_frac=read / HBM_PEAK_GBS, copy_GBps=copy, copy_frac=copy / HBM_PEAK_GBS,
                bytes=n * 4, what="torch sum (read) and copy_ (read + write) of 1 GiB fp32, median of %d" % reps)


def _read_pmc(folder, counter):
    """Per-kernel list of per-dispatch values of `counter` (KiB) from the
    counter_collection.csv files under `folder`."""
    import csv
    import glob
    per_dispatch = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    for fn in files:
        with open(fn) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                key = next((k for pat, k in KERNEL_KEYS if pat in name), None)
                if key is None and "lowrank" in name:
                    key = "lowrank_project"
                if key is None:
                    continue
                d = (fn, row.get("Dispatch_Id"), key)      # rows of one dispatch add up
                per_dispatch[d] = per_dispatch.get(d, 0.0) + float(row["Counter_Value"])
    vals = {}
    for (_, _, key), v in per_dispatch.items():
        vals.setdefault(key, []).append(v)
    return vals


SQ_KEYS = [("tiled_gateup", "gateup_tiled"), ("tiled_down", "down_tiled"), ("gateup_kernel", "gateup_stream"),
           ("down_kernel", "down_stream"), ("lowrank", "lowrank_project"), ("route", "route"), ("combine", "combine")]
SQ_COUNTERS = ["SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_WAVES", "SQ_BUSY_CYCLES",
               "GRBM_GUI_ACTIVE"]
# the optional second pass: where the waves' cycles go, and the LDS
SQ_STALL_COUNTERS = ["SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY",
                     "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"]
MFMA_FLOPS = 16 * 16 * 32 * 2      # every MFMA of these kernels is v_mfma_f32_16x16x32_f16
N_SIMD = 256 * 4
N_XCD = 8                           # GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs


def _sq_key(name):
    return next((k for pat, k in SQ_KEYS if pat in name), None)


def _read_sq(folder, names):
    """Per kernel key, per counter: the per-dispatch values under folder."""
    import csv
    import glob
    per = {}
    for fn in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(fn)):
            key = _sq_key(row.get("Kernel_Name", ""))
            if key is None or row.get("Counter_Name") not in names:
                continue
            d = (fn, row["Dispatch_Id"], key, row["Counter_Name"])
            per[d] = per.get(d, 0.0) + float(row["Counter_Value"])
    vals = {}
    for (_, _, key, cn), v in per.items():
        vals.setdefault(key, {}).setdefault(cn, []).append(v)
    return vals


def summarize_sq(workload, trace_dir, sq_dir, stall_dir=None):
    """MFMA and VALU counters per kernel from one rocprofv3 --pmc pass
    (SQ_COUNTERS) and the kernel trace of the same command: MFMA
    instructions x 16384 flops over the mean duration (counter TFLOP/s), the
    MFMA-busy share of SIMD cycles, the clock the GPU-active cycle count
    implies.  Writes profiles/counters_<workload>.md."""
    import csv
    import glob
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    dur = {}
    for row in csv.DictReader(open(stats[0])):
        key = _sq_key(row["Name"])
        if key:
            c, t = dur.get(key, (0, 0.0))
            dur[key] = (c + int(row["Calls"]), t + float(row["TotalDurationNs"]))
    vals = _read_sq(sq_dir, SQ_COUNTERS)
    lines = [f"# MFMA and VALU counters per kernel, {workload}", "",
             "Two runs of the same command (a kernel trace, then one counter pass with "
             f"{' '.join(SQ_COUNTERS)}) and their reduction:", "", "```",
             f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o kt --output-format csv -- "
             f"python3 bench.py {workload_ref(workload)[1]} --steps 5 --warmup 2 --no-cpu-baseline --no-extra",
             f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -d {sq_dir} -o pmc --output-format csv -- "
             f"python3 bench.py {workload_ref(workload)[1]} --steps 5 --warmup 2 --no-cpu-baseline --no-extra",
             f"python3 bench.py {workload_ref(workload)[1]} --summarize-sq {trace_dir} {sq_dir}", "```", "",
             "Per dispatch (means). MFMA TFLOP/s = SQ_INSTS_MFMA x 16384 / mean duration (every MFMA here is "
             "16x16x32 fp16; padding rows and the low-rank MFMAs count). GRBM_GUI_ACTIVE sums the 8 XCDs' "
             "active cycles, so the clock = GRBM_GUI_ACTIVE / 8 / mean duration, and MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs): the share of the MFMA peak at "
             "that clock (it agrees with MFMA TFLOP/s over the peak scaled to the clock). Clock and busy "
             "figures of kernels of a few microseconds are dominated by launch and drain.", "",
             "| kernel | dispatches | mean us | MFMA instr | MFMA TFLOP/s | of 2.5 PF | MFMA busy | VALU instr | "
             "waves | clock GHz |", "|---|---|---|---|---|---|---|---|---|---|"]
    stat = statistics.mean
    for key in [k for _, k in SQ_KEYS]:
        if key not in vals or key not in dur:
            continue
        v = {cn: stat(x) for cn, x in vals[key].items()}
        us = dur[key][1] / dur[key][0] / 1e3
        mf = v.get("SQ_INSTS_MFMA", 0.0)
        tf = mf * MFMA_FLOPS / (us * 1e-6) / 1e12
        act = v.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (act * N_SIMD) if act else float("nan")
        clk = act / (us * 1e-6) / 1e9 if act else float("nan")
        lines.append(f"| {key} | {len(vals[key].get('SQ_INSTS_MFMA', []))} | {us:.1f} | {mf:.4g} | {tf:.1f} | "
                     f"{tf / MFMA_F16_PEAK_TFLOPS:.3f} | {busy:.3f} | {v.get('SQ_INSTS_VALU', 0.0):.4g} | "
                     f"{v.get('SQ_WAVES', 0.0):.4g} | {clk:.2f} |")
    if stall_dir:
        sv = _read_sq(stall_dir, SQ_STALL_COUNTERS)
        lines += ["", "Where the waves' cycles go, from a second counter pass of the same command:", "", "```",
                  f"rocprofv3 --pmc {' '.join(SQ_STALL_COUNTERS)} -d {stall_dir} -o pmc --output-format csv -- "
                  f"python3 bench.py {workload_ref(workload)[1]} --steps 5 --warmup 2 --no-cpu-baseline "
                  f"--no-extra", "```", "",
                  "Shares of SQ_WAVE_CYCLES (the summed lifetime of the kernel's waves): issuing any instruction, "
                  "issuing VALU instructions (MFMAs included), waiting at a wait or barrier (SQ_WAIT_ANY), and "
                  "ready but not issued (SQ_WAIT_INST_ANY: a dependency or a busy unit). LDS: instructions per "
                  "dispatch, and the LDS bank-conflict cycles over the LDS-active cycles.", "",
                  "| kernel | issue any | issue VALU | waiting | not issued | LDS instr | bank-conflict share |",
                  "|---|---|---|---|---|---|---|"]
        for key in [k for _, k in SQ_KEYS]:
            if key not in sv:
                continue
            v = {cn: stat(x) for cn, x in sv[key].items()}
            wc = v.get("SQ_WAVE_CYCLES", 0.0)
            lds = v.get("SQ_ACTIVE_INST_LDS", 0.0)
            if not wc:
                continue
            lines.append(f"| {key} | {v.get('SQ_ACTIVE_INST_ANY', 0.0) / wc:.3f} | "
                         f"{v.get('SQ_ACTIVE_INST_VALU', 0.0) / wc:.3f} | {v.get('SQ_WAIT_ANY', 0.0) / wc:.3f} | "
                         f"{v.get('SQ_WAIT_INST_ANY', 0.0) / wc:.3f} | {v.get('SQ_INSTS_LDS', 0.0):.4g} | "
                         f"{(v.get('SQ_LDS_BANK_CONFLICT', 0.0) / lds) if lds else 0.0:.3f} |")
    lines.append("")
    out = os.path.join(ROOT, "profiles", f"counters_{workload_ref(workload)[0]}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_trace(workload, trace_dir, top=30):
    """Kernel-time table (calls, mean, min, max, share) of a rocprofv3
    --kernel-trace --stats run of the default bench command (the workload,
    the prefill layer and the other three layers, set-up included) to
    profiles/kernels_<workload>.md."""
    import csv
    import glob
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(stats[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tag, wargs = workload_ref(workload)
    lines = [f"# Kernel time, {workload} (bench.py default command under rocprofv3)", "",
             "Commands (from the repository root, on one MI355X):", "", "```",
             f"cd /tmp && export TMPDIR=/tmp && cd - && rocprofv3 --kernel-trace --stats -d {trace_dir} -o kt "
             f"--output-format csv -- python3 bench.py --no-cpu-baseline",
             f"python3 bench.py {wargs} --summarize-trace {trace_dir}", "```", "",
             "Source `kt_kernel_stats.csv`: every kernel of the run (the decode layer, the prefill layer, the "
             "tiny, fine-grained and bit-plane layers, and set-up: quantization, LUTs, packing), the "
             f"{top} largest by total time. Durations in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        name = r["Name"][:110]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    lines.append("")
    with open(os.path.join(ROOT, "profiles", f"kernels_{tag}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def workload_ref(name):
    """(file-name tag, bench.py arguments) of a workload name: its short
    name, with --tokens when the token count is not the config's own."""
    import re
    from synth import configs
    m = re.search(r"_t(\d+)_", name)
    for short in ("decode", "prefill", "finegrained", "bitplane", "tiny"):
        base = configs.get(short)["name"]
        if base == name:
            return short, f"--workload {short}"
        if m and re.sub(r"_t\d+_", f"_t{m.group(1)}_", base) == name:
            return f"{short}_t{m.group(1)}", f"--workload {short} --tokens {m.group(1)}"
    return name, f"--workload {name}"


def summarize_pmc(workload, fetch_dir, write_dir, bench_log=None):
    """Per-launch HBM traffic (FETCH_SIZE, WRITE_SIZE passes, each scaled by
    what it reads for the calibration copy) of each kernel of the workload:
    stored in profiles/traffic_counters.json (with the kernel source hash)
    and written out as profiles/traffic_<workload>.md, beside the
    algorithmic bytes of the layer and of its gate/up launch when the
    profiled run's bench line (bench_log) is given."""
    fe = _read_pmc(fetch_dir, "FETCH_SIZE")
    wr = _read_pmc(write_dir, "WRITE_SIZE")
    # each counter is scaled by what it reads for the copy of CALIB_BYTES
    cf = CALIB_BYTES / (statistics.median(fe["calibration_copy"]) * 1024.0)
    cw = CALIB_BYTES / (statistics.median(wr["calibration_copy"]) * 1024.0)
    ent = dict(source_hash=kernel_source_hash(), fetch_scale=cf, write_scale=cw, kernels={})
    for key in sorted(set(fe) & set(wr)):
        f = statistics.mean(fe[key]) * 1024.0 * cf
        w = statistics.mean(wr[key]) * 1024.0 * cw
        ent["kernels"][key] = dict(launches=len(fe[key]), fetch_bytes=f, write_bytes=w,
                                   bytes=f + w)
    tr = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    tr[workload] = ent
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(tr, fh, indent=1, sort_keys=True)
    print(json.dumps({workload: ent}, indent=1))
    tag, wargs = workload_ref(workload)
    rx = "gateup_kernel|down_kernel|lowrank|route|combine|neg_kernel"
    steps, warmup = 20, 5
    if bench_log and os.path.exists(bench_log):
        # the step counts of the profiled run, from its bench line
        b0 = json.loads([l for l in open(bench_log) if l.startswith("{")][-1])
        steps, warmup = b0.get("steps", steps), b0.get("warmup", warmup)
    cmd = (f"python3 bench.py {wargs} --steps {steps} --warmup {warmup} --no-cpu-baseline --no-extra "
           f"--copy-calibration")
    lines = [f"# HBM traffic per launch, {workload}", "",
             "Two counter passes (one counter each) and their reduction to bytes per launch:", "", "```",
             f'rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "{rx}" -d {fetch_dir} -o pmc '
             f"--output-format csv -- {cmd}",
             f'rocprofv3 --pmc WRITE_SIZE --kernel-include-regex "{rx}" -d {write_dir} -o pmc '
             f"--output-format csv -- {cmd}",
             f"python3 bench.py {wargs} --summarize-pmc {fetch_dir} {write_dir}"
             + (f" {bench_log}" if bench_log else ""), "```", "",
             f"The calibration kernel is an int8 negation over 1 GiB (reads and writes 2^30 B once each). "
             f"Scale factors (bytes per counted byte): FETCH_SIZE x{cf:.4f}, WRITE_SIZE x{cw:.4f}. "
             f"Kernel sources hash `{ent['source_hash']}`.", "",
             "| kernel | launches | fetch MB | write MB | total MB |", "|---|---|---|---|---|"]
    for key, v in sorted(ent["kernels"].items()):
        lines.append(f"| {key} | {v['launches']} | {v['fetch_bytes'] / 1e6:.3f} | {v['write_bytes'] / 1e6:.3f} | "
                     f"{v['bytes'] / 1e6:.3f} |")
    if bench_log and os.path.exists(bench_log):
        line = [l for l in open(bench_log) if l.startswith("{")][-1]
        b = json.loads(line)
        lay = b.get("layer", {})
        lines += ["", f"Algorithmic bytes of the profiled call (the bench line of the FETCH pass): the layer "
                      f"{lay.get('alg_bytes', 0) / 1e6:.3f} MB; its gate/up launch (codes, metadata and U of "
                      f"the gate and up blocks of the active experts, x read, h written) "
                      f"{b['roofline']['bytes_per_launch'] / 1e6:.3f} MB."]
        gu = ent["kernels"].get("gateup_stream") or ent["kernels"].get("gateup_tiled")
        if gu:
            lines.append(f"Counter traffic of the gate/up launch over its algorithmic bytes: "
                         f"{gu['bytes'] / b['roofline']['bytes_per_launch']:.3f}.")
    lines.append("")
    with open(os.path.join(ROOT, "profiles", f"traffic_{tag}.md"), "w") as fh:
        fh.write("\n".join(lines))


def cpu_baseline(cfg, seed, sample_tokens, min_seconds=12.0):
    """The oracle as it stands on a bounded sample of the same workload:
    route all tokens, then the full expert FFN and combine for the sampled
    tokens (PTQ of the needed blocks done before timing), repeated until at
    least min_seconds have passed."""
    import numpy as np
    from oracle import forward
    from oracle.layer import OracleLayer
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1

    E, k = cfg["E"], cfg["k"]
    bits = gen.gen_bits(cfg, seed)

    def rows(e, blk, r):
        return gen.gen_weight_block(cfg, seed, e, blk) if r is None else gen.gen_weight_rows(cfg, seed, e, blk, r)

    fac = (lambda e, blk: gen.gen_factors(cfg, seed, e, blk)) if cfg["r"] else None
    sh = (lambda g, blk: gen.gen_shared_factors(cfg, seed, g, blk)) if cfg.get("rs") else None
    x = gen.gen_x(cfg, seed)
    logits = gen.gen_logits(cfg, seed)
    ids = forward.topk_ids(logits, k)
    tokens = list(range(sample_tokens))
    experts = sorted({int(e) for t in tokens for e in ids[t]})
    orc = OracleLayer(E, cfg["H"], cfg["I"], cfg["G"], cfg["fmt"], bits, rows, factors=fac,
                      shared=sh, share=cfg.get("share", 0), cache_blocks=3 * len(experts) + 3)
    for e in experts:                      # PTQ (data preparation) outside the timing
        for blk in range(3):
            orc.qblock(e, blk)
    reps, t0 = 0, time.perf_counter()
    while True:                            # repeat the sample until min_seconds have passed
        forward.moe_forward(orc, x, logits, k, cfg["n_comp"], tokens=np.array(tokens))
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return dict(value=reps * len(tokens) / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"{reps} x {len(tokens)} of {cfg['T']} tokens of the same layer: routing of all "
                       f"tokens, fp64 dequantization of the {len(experts)} experts they use, "
                       f"compensated SwiGLU FFN and combine ({dt:.1f} s)")


def workload_cfg(args):
    """The workload's config, with --tokens in place of its T (and in its name)."""
    import re
    from synth import configs
    cfg = configs.get(args.workload)
    if args.tokens > 0:
        cfg = dict(cfg, T=args.tokens, name=re.sub(r"_t\d+_", f"_t{args.tokens}_", cfg["name"]))
    return cfg


def main():
    args = parse()
    if args.summarize_sq:
        summarize_sq(workload_cfg(args)["name"], *args.summarize_sq)
        return
    if args.summarize_pmc:
        summarize_pmc(workload_cfg(args)["name"], *args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(workload_cfg(args)["name"], args.summarize_trace)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the expert layer is not "
              "sharded across GPUs", file=sys.stderr)
        sys.exit(2)
    import torch
    from synth import configs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = workload_cfg(args)
    t_setup = time.time()
    formats = {"main": cfg}
    copies = {"main": 3 if cfg["H"] * cfg["I"] * cfg["E"] > 1e8 else 2}
    extra_cfg = None
    if args.workload == "decode" and not args.no_extra:
        # the same Mixtral-shaped weights, int4, in the prefill regime
        extra_cfg = configs.get("prefill")
        formats["prefill"] = extra_cfg
        copies["prefill"] = 1
    layers = build_layers(cfg, args.seed, copies, formats)
    setup_s = time.time() - t_setup
    if args.copy_calibration:
        copy_calibration()

    ms, prof, alg = run_workload(cfg, layers["main"], args.seed, args.steps, args.warmup, args.path,
                                 graph=args.graph, split_k=args.split_k, fused=not args.no_fused)
    T = cfg["T"]
    tokens_s = T / (ms * 1e-3)

    kern = {n: dict(launches=c, avg_us=1e3 * t / max(c, 1)) for n, (c, t) in prof.items()}
    gu = kern.get("gateup_stream", {}).get("avg_us")
    achieved = alg["gateup_bytes"] / (gu * 1e-6) / 1e9 if gu else None
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get(cfg["name"], {})
        if ent.get("source_hash") == kernel_source_hash():
            traffic = ent.get("kernels", {}).get("gateup_stream", {}).get("bytes")
    # the dominant kernel (gate/up) by the bench contract, and beside it the
    # whole step (route + every FFN kernel) against the same peak
    step_gbs = alg["bytes"] / (ms * 1e-3) / 1e9
    roofline = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=(achieved / HBM_PEAK_GBS) if achieved else None, traffic=traffic,
                    kernel="gateup_stream", bytes_per_launch=alg["gateup_bytes"],
                    whole_step=dict(achieved=step_gbs, frac=step_gbs / HBM_PEAK_GBS, bytes=alg["bytes"],
                                    what="algorithmic bytes of the layer / step time (route + expert FFN)"))
    ffn_us = sum(v["avg_us"] for n, v in kern.items() if n != "route")
    out = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "T": T, "E": cfg["E"], "k": cfg["k"], "H": cfg["H"],
                   "I": cfg["I"], "fmt": cfg["fmt"], "bits": cfg["bits"], "G": cfg["G"],
                   "r": cfg["r"], "n_comp": cfg["n_comp"], "seed": args.seed,
                   "weight_copies": copies["main"], "parallelism": "none (1 GPU)",
                   "launch": "hip_graph" if args.graph else "stream"},
        "roofline": roofline,
        "layer": dict(alg_bytes=alg["bytes"], alg_flops=alg["flops"], active_experts=alg["active"],
                      expert_counts=alg["counts"],
                      hbm_frac_step=alg["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      hbm_frac_kernels=(alg["bytes"] / (ffn_us * 1e-6) / 1e9 / HBM_PEAK_GBS) if ffn_us else None),
        "kernels": kern,
        "step_ms_dist": alg["step_ms_dist"],
        "setup_s": setup_s,
    }
    if extra_cfg is not None:
        pms, pprof, palg = run_workload(extra_cfg, layers["prefill"], args.seed, max(10, args.steps // 10),
                                        max(5, args.warmup // 4), args.path, graph=args.graph,
                                        fused=not args.no_fused)
        pk = {n: dict(launches=c, avg_us=1e3 * t / max(c, 1)) for n, (c, t) in pprof.items()}
        out["prefill"] = dict(workload=extra_cfg["name"], ms_per_step=pms,
                              tokens_s=extra_cfg["T"] / (pms * 1e-3), alg_flops=palg["flops"],
                              tflops=palg["flops"] / (pms * 1e-3) / 1e12,
                              mfma_frac=palg["flops"] / (pms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                              expert_counts=palg["counts"], step_ms_dist=palg["step_ms_dist"], kernels=pk)
    del layers
    if args.workload == "decode" and not args.no_extra and not args.no_others:
        # the other three layers of the workload set, measured the same way
        # (cold weights: enough packed copies that the last-level cache
        # cannot hold them), as context for the decode line
        out["other_configs"] = {}
        for short, R in (("tiny", 2), ("finegrained", 5), ("bitplane", 4)):
            ocfg = configs.get(short)
            olayers = build_layers(ocfg, args.seed, {"main": R}, {"main": ocfg})["main"]
            oms, oprof, oalg = run_workload(ocfg, olayers, args.seed, max(20, args.steps // 4),
                                            max(5, args.warmup // 4), args.path, graph=args.graph,
                                            fused=not args.no_fused)
            ok = {n: dict(launches=c, avg_us=1e3 * t / max(c, 1)) for n, (c, t) in oprof.items()}
            out["other_configs"][short] = dict(
                workload=ocfg["name"], ms_per_step=oms, tokens_s=ocfg["T"] / (oms * 1e-3),
                alg_bytes=oalg["bytes"], alg_flops=oalg["flops"], active_experts=oalg["active"],
                hbm_frac=oalg["bytes"] / (oms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                mfma_frac=oalg["flops"] / (oms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                weight_copies=R, kernels=ok)
            if short == "bitplane":
                # the same bit-plane layer with many tokens per expert (4096
                # tokens, 256 pairs per expert on average): the default path
                # is then the tiled one
                pcfg = dict(ocfg, T=4096, name=ocfg["name"].replace("_t512_", "_t4096_"))
                pms, pprof, palg = run_workload(pcfg, olayers, args.seed, max(10, args.steps // 10),
                                                max(5, args.warmup // 4), args.path, graph=args.graph,
                                                fused=not args.no_fused)
                out["other_configs"]["bitplane_prefill"] = dict(
                    workload=pcfg["name"], ms_per_step=pms, tokens_s=pcfg["T"] / (pms * 1e-3),
                    alg_bytes=palg["bytes"], alg_flops=palg["flops"],
                    tflops=palg["flops"] / (pms * 1e-3) / 1e12,
                    mfma_frac=palg["flops"] / (pms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                    weight_copies=R,
                    kernels={n: dict(launches=c, avg_us=1e3 * t / max(c, 1)) for n, (c, t) in pprof.items()})
            del olayers
            torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_extra:
        out["hbm_context"] = hbm_context()
        out["route_scaling"] = route_scaling()
    if not args.no_cpu_baseline:
        # decode: the whole 16-token batch, repeated for about 12 s
        out["cpu_baseline"] = cpu_baseline(cfg, args.seed, min(cfg["T"], 16))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
