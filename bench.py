#!/usr/bin/env python3
"""Throughput of the VDA forward pass on one MI355X.

One step = one vda_forward call (statistics, symmetric Gauss-Jordan solve, chunk
composition, bidirectional boundary scan, fused readout) over the whole
workload, inputs already resident in HBM.  Default workload: the 768p-shaped one-GPU head share
(16 heads x 90 latent frames x 4032 tokens, d_k = d_v = 128, 512 text tokens,
bf16 features, fp32 state), synthetic seeded inputs.

Prints ONE JSON line: token-heads/s, the roofline of the dominant kernel
(timed with HIP events recorded by the library on the launch stream), the
MFMA fraction the metric asks for, the fp64 CPU oracle timed on a bounded
sample of the same workload on the host cores, (object "batched_rule") the
same inputs under SANA-WM's batched comparison rule with the boundary-state
norms of every rule, (object "decay") the same workload with channel-wise
decay gates through vda_forward_decay, (object "prep") the feature map on the
768p head share (k and v alone, with the query map left to the forward's
readout; with its query pass; and vda_prep then vda_forward both ways), and
(object "configs") the tiny, small, medium and stress
workloads, each with its own roofline and oracle baseline (the small ones
rotate through input copies that do not fit in the MALL together).  The text
seed follows --seed-mode (default 1: the text written at beta / 2).

  python bench.py [--steps K] [--warmup W] [--config 4] [--cpu-seconds S]
  python bench.py --summarize DIR [--config 4]   (profiles/ from rocprofv3 output)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "VDA fwd tokens/sec per head-layer on 1 MI355X; % MFMA peak"
HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5166e15      # MI355X dense bf16 MFMA, flop/s
PROFILES = os.path.join(ROOT, "profiles")
STAGES = ("stats", "solve", "compose", "scan", "readout")
CEILING_CALLS = 7          # torch.add launches of the stream-ceiling measurement (2 + 5)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg):
    """Algorithmic HBM bytes (and MFMA flops where the kernel is a contraction)
    per launch of each kernel: every input read once, every output written once.
    "stats" is the latent frames' kernel, "stats_text" the text frame's (fp32
    MFMA), which at bf16 with d_k = d_v = 128 runs inside the "stats" kernel (its
    work is then counted there and "stats_text" is zero); with decay the gates
    are read once by the composition and once by the split kernel (bf16,
    d_k = d_v = 128: one split image per frame) or the readout (other shapes),
    and the composition also writes the reverse maps; at bf16 with
    d_k = d_v = 128 without decay under the frame-wise rule the composition
    writes Mc and the scans' two operand images of it (one transition's size
    each) in place of Mc^T."""
    eb = 2 if cfg.dtype == "bf16" else 4
    th = cfg.units * cfg.frames * cfg.tokens        # token-heads
    tt = cfg.units * cfg.text_tokens
    dk, dv, n, u, F = cfg.d_k, cfg.d_v, cfg.n_chunks, cfg.units, cfg.frames
    mat, st = dk * dk * 4, dv * dk * 4               # one transition, one state (fp32)
    gates = u * F * dk * 4 if cfg.alpha_mu is not None else 0
    images = (cfg.dtype == "bf16" and dk == 128 and dv == 128 and cfg.alpha_mu is None
              and cfg.rule == 0)
    nmaps = 3 if cfg.alpha_mu is not None or images else 2  # Mc, Mc^T (+ Mr^T), or Mc + images
    # A is symmetric: under the frame-wise rule the kernel writes its blocks on
    # and below the diagonal (all the solve reads); the batched rules read all of A
    nkb = -(-dk // 32)
    a_frac = 1.0 if cfg.rule != 0 else nkb * (nkb + 1) / 2 / (nkb * nkb)
    stats_bytes = th * ((dk + dv) * eb + 4) + u * F * (a_frac * dk + dv) * dk * 4
    text_bytes = tt * ((dk + dv) * eb + 4) + u * (dk + dv) * dk * 4
    split = cfg.dtype == "bf16" and dk == 128 and dv == 128
    image = 2 * 128 * 136 * 2                        # one segment's split S~ (bf16 hi + lo)
    nimg = u * (F if cfg.alpha_mu is not None else n)  # segments: frames with decay, else chunks
    readout_bytes = (th * (dk + 2 * dv) * eb                           # q, gate read; out written
                     + (nimg * image if split else u * n * 2 * st + gates)  # S~ images, or states
                     + dv * 4)
    split_bytes = u * n * 2 * st + nimg * image + gates if split else 0  # P, R (gates) in; images
    solve_bytes = (a_frac + 1) * u * (F + 1) * mat                     # A in, M out
    compose_bytes = (u * (F + 1) * (mat + st) + gates                  # M, B (and gates) in
                     + u * n * (nmaps * mat + 2 * st)                   # chunk maps out
                     + u * 2 * st)                                      # the two seed copies
    scan_bytes = u * n * (2 * mat + 2 * st) + u * 2 * n * st            # chunk maps in; P, R out
    stats_flops, text_flops = 2 * th * (dk + dv) * dk, 2 * tt * (dk + dv) * dk
    if cfg.dtype == "bf16" and dk == 128 and dv == 128:  # one kernel
        stats_bytes, stats_flops, text_bytes, text_flops = (stats_bytes + text_bytes,
                                                            stats_flops + text_flops, 0, 0)
    return {"stats": (stats_bytes, stats_flops),
            "stats_text": (text_bytes, text_flops),
            "readout": (readout_bytes, 2 * th * dk * dv),
            "solve": (solve_bytes, None), "compose": (compose_bytes, None),
            "scan": (scan_bytes, None), "split": (split_bytes, None)}


def stage_alg(alg, stage):
    """(bytes, flops) of a timed stage: the statistics stage runs two kernels, the
    scan stage ends with the readout's state split."""
    if stage == "scan":
        return (alg["scan"][0] + alg["split"][0], None)
    if stage != "stats":
        return alg[stage]
    return (alg["stats"][0] + alg["stats_text"][0], alg["stats"][1] + alg["stats_text"][1])



KERNEL_SOURCES = {"stats": "k_stats.hip", "stats_text": "k_stats.hip", "readout": "k_readout.hip",
                  "split": "k_readout.hip", "solve": "k_solve.hip",
                  "compose": "k_scan.hip", "scan": "k_scan.hip"}


def source_digest(kernel):
    """sha256 over the kernel's source file and the device header it includes."""
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "vda_device.h"):
        with open(os.path.join(ROOT, "frame_wise_delta_gram_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


# occupancy, vector ALU and LDS counters of one pass (8 SQ + 1 GRBM counters)
XCDS = 8  # accelerator complex dies of an MI355X (one GRBM instance each)
SQ_COUNTERS = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU "
               "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE")
PROFILE_COMMANDS = {  # CFG: the workload id
    "FETCH_SIZE": "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --kernel-include-regex "
                  "'vda|add' -d DIR/FETCH_SIZE -o p --output-format csv -- python bench.py "
                  "--config CFG --steps 2 --warmup 1 --cpu-seconds 0 --decay-steps 0 "
                  "--batched-steps 0 --prep-steps 0 --variant-steps 0 --other-configs=",
    "WRITE_SIZE": "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --kernel-include-regex "
                  "'vda|add' -d DIR/WRITE_SIZE -o p --output-format csv -- python bench.py "
                  "--config CFG --steps 2 --warmup 1 --cpu-seconds 0 --decay-steps 0 "
                  "--batched-steps 0 --prep-steps 0 --variant-steps 0 --other-configs=",
    "MFMA": "timeout -s KILL 120 rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 "
            "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
            "--kernel-include-regex vda -d DIR/MFMA -o p --output-format csv -- python bench.py "
            "--config CFG --steps 2 --warmup 1 --cpu-seconds 0 --decay-steps 0 "
            "--batched-steps 0 --prep-steps 0 --variant-steps 0 --other-configs=",
    "OCC": "timeout -s KILL 120 rocprofv3 --pmc " + SQ_COUNTERS + " "
           "--kernel-include-regex vda -d DIR/OCC -o p --output-format csv -- python bench.py "
           "--config CFG --steps 2 --warmup 1 --cpu-seconds 0 --decay-steps 0 "
           "--batched-steps 0 --prep-steps 0 --variant-steps 0 --other-configs=",
    "stats": "rocprofv3 --kernel-trace --stats -d DIR/trace -o vda --output-format csv -- "
             "python bench.py --config CFG --steps 20 --warmup 50 --cpu-seconds 0 "
             "--decay-steps 0 --batched-steps 0 --prep-steps 0 --variant-steps 0 --other-configs=",
}
TRACE_WARMUP, TRACE_STEPS = 50, 20  # of the kernel-trace command above
KERNELS = ("stats_text", "stats", "solve", "compose", "scan", "split", "readout")  # launch order
PREP_COMMAND = ("rocprofv3 {pmc} -d DIR/{sub} -o p --output-format csv -- python bench.py "
                "--steps 1 --warmup 0 --cpu-seconds 0 --decay-steps 0 --batched-steps 0 "
                "--prep-steps 5 --variant-steps 0 --other-configs=")
# one launch each: the K and V sweeps alone (q = NULL), or followed by the Q pass
PREP_KERNELS = ("prep_kv", "prep")
KERNEL_NAMES = {"stats_bf16_kernel": "stats", "stats_f32_kernel": "stats",
                "stats_text_kernel": "stats_text",
                "readout_bf16_kernel": "readout", "readout_f32_kernel": "readout",
                "readout_c128_kernel": "readout", "split_states_kernel": "split",
                "solve_kernel": "solve", "batched_factor_kernel": "solve",
                "solve_chol_kernel": "solve",
                "compose_split_kernel": "compose",
                "compose_kernel": "compose", "scan_split_kernel": "scan", "scan_kernel": "scan",
                "scan_img_kernel": "scan"}


def short_kernel_name(full):
    import re
    m = re.search(r"vda::\(anonymous namespace\)::(\w+)", full)
    if m:
        if m.group(1) in ("prep_conv_kernel", "prep_mfma_kernel"):
            return "prep"
        return KERNEL_NAMES.get(m.group(1), m.group(1))
    return "copy" if "add" in full.lower() else None


def sq_table(path, order, kind=None):
    """Markdown lines of the SQ_COUNTERS pass at `path` (empty when absent):
    per kernel, occupancy, vector ALU activity and LDS figures per launch
    (kind(row) names a row's kernel; default: from its Kernel_Name)."""
    import collections
    import csv
    if not os.path.exists(path):
        return []
    ctr = collections.defaultdict(lambda: collections.defaultdict(float))
    kname = {}
    gui_rows = collections.Counter()
    with open(path) as fh:
        for r in csv.DictReader(fh):
            k = kind(r) if kind else short_kernel_name(r["Kernel_Name"])
            if k is None or k == "copy":
                continue
            i = int(r["Dispatch_Id"])
            kname[i] = k
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                gui_rows[i] += 1
                ctr[i]["GRBM_GUI_ACTIVE"] = max(ctr[i]["GRBM_GUI_ACTIVE"], float(r["Counter_Value"]))
            else:
                ctr[i][r["Counter_Name"]] += float(r["Counter_Value"])
    for i, n in gui_rows.items():
        if n == 1:  # one row: the sum over the XCDs' GRBM instances; per XCD = sum / 8
            ctr[i]["GRBM_GUI_ACTIVE"] /= XCDS
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for i, c in ctr.items():
        for name, val in c.items():
            agg[kname[i]][name].append(val)
    lines = ["", "## Occupancy, vector ALU and LDS per launch (`SQ_WAVE_CYCLES`, "
             "`SQ_ACTIVE_INST_VALU`, `SQ_LDS_BANK_CONFLICT`, ...)", "",
             "Occupancy = 400 x SQ_WAVE_CYCLES (quad-cycles) / GRBM_GUI_ACTIVE / 256 CUs / 32 "
             "wave slots per CU (rocprofv3's OccupancyPercent; GRBM_GUI_ACTIVE of one XCD, the "
             "per-dispatch value rocprofv3 writes being the sum over the 8 XCDs): the mean share of the wave "
             "slots holding a wave over the launch; mean waves per CU = that x 32. VALU active "
             "= SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (share of resident wave-cycles issuing "
             "vector ALU work). VALU instructions per wave = SQ_INSTS_VALU / SQ_WAVES. LDS "
             "conflict = SQ_LDS_BANK_CONFLICT cycles per LDS instruction; LDS wait = "
             "SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES.", "",
             "| kernel | waves | occupancy | mean waves per CU | VALU active | VALU instructions "
             "per wave | LDS instructions | LDS conflict cycles per instruction | LDS wait |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k in order:
        if k not in agg:
            continue
        m = {name: sum(v) / len(v) for name, v in agg[k].items()}
        gui = max(m.get("GRBM_GUI_ACTIVE", 0.0), 1.0)
        wc = max(m.get("SQ_WAVE_CYCLES", 0.0), 1.0)
        waves = max(m.get("SQ_WAVES", 0.0), 1.0)
        occ = 400.0 * wc / gui / 256 / 32
        lds = m.get("SQ_INSTS_LDS", 0.0)
        conf = m.get("SQ_LDS_BANK_CONFLICT", 0.0) / lds if lds else 0.0
        lines.append(f"| {k} | {waves:.0f} | {occ:.1f}% | {occ / 100 * 32:.1f} | "
                     f"{100 * m.get('SQ_ACTIVE_INST_VALU', 0.0) / wc:.1f}% | "
                     f"{m.get('SQ_INSTS_VALU', 0.0) / waves:.0f} | {lds:.4g} | {conf:.2f} | "
                     f"{100 * m.get('SQ_WAIT_INST_LDS', 0.0) / wc:.1f}% |")
    return lines


def summarize_prep(prep_dir):
    """profiles/prep_kernels_<workload>.md from a kernel trace and FETCH_SIZE /
    WRITE_SIZE passes of PREP_COMMAND (DIR = prep_dir)."""
    import collections
    import csv
    import workloads as W

    cfg = W.PREP_CONFIGS[3]
    base = W.CONFIGS[4]
    copy_bytes = base.units * base.frames * base.tokens * base.d_v * 2
    known = {"FETCH_SIZE": 2 * copy_bytes, "WRITE_SIZE": copy_bytes}
    eb = 2
    rows = cfg.batch * cfg.frames * cfg.tokens * cfg.heads
    # q (with the query pass), k, v read and written once; the K and V filters
    # (30 fp32 taps per channel)
    alg = {"prep": 2 * eb * rows * (2 * cfg.d_k + cfg.d_v) + cfg.heads * (cfg.d_k + cfg.d_v) * 120,
           "prep_kv": 2 * eb * rows * (cfg.d_k + cfg.d_v) + cfg.heads * (cfg.d_k + cfg.d_v) * 120}
    flops = {"prep": 60 * rows * (cfg.d_k + cfg.d_v), "prep_kv": 60 * rows * (cfg.d_k + cfg.d_v)}

    def prep_kind(name, grid, kv_grid):
        k = short_kernel_name(name)
        return ("prep_kv" if grid <= kv_grid else "prep") if k == "prep" else k

    def kv_grid_of(path, col):  # the K/V-only launches have the smallest prep grid
        with open(path) as fh:
            g = [int(r[col]) for r in csv.DictReader(fh)
                 if short_kernel_name(r["Kernel_Name"]) == "prep"]
        return min(g) if g else 0

    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(prep_dir, ctr, "p_counter_collection.csv")
        kvg = kv_grid_of(path, "Grid_Size")
        disp = collections.defaultdict(float)
        names = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                k = prep_kind(r["Kernel_Name"], int(r["Grid_Size"]), kvg)
                if k is None or r["Counter_Name"] != ctr:
                    continue
                disp[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
                names[int(r["Dispatch_Id"])] = k
        acc = collections.defaultdict(list)
        for i, v in sorted(disp.items()):
            acc[names[i]].append(v)
        # the calibration adds are the largest "add" dispatches (input generation adds
        # small tensors)
        acc["copy"] = sorted(acc["copy"])[-CEILING_CALLS:]
        per[ctr] = {k: sum(v) / len(v) for k, v in acc.items()}
    scale = {c: known[c] / (per[c]["copy"] * 1024.0) for c in per}
    durations = {}
    tpath = os.path.join(prep_dir, "trace", "p_kernel_trace.csv")
    kvg = kv_grid_of(tpath, "Grid_Size_X")
    ns = collections.defaultdict(list)
    with open(tpath) as fh:
        for r in csv.DictReader(fh):
            k = prep_kind(r["Kernel_Name"], int(r["Grid_Size_X"]), kvg)
            if k in PREP_KERNELS:
                ns[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    for k, v in ns.items():
        durations[k] = (len(v), sum(v) / len(v) / 1e3)
    cmds = [PREP_COMMAND.format(pmc="--kernel-trace --stats", sub="trace"),
            "timeout -s KILL 120 " + PREP_COMMAND.format(pmc="--pmc FETCH_SIZE", sub="FETCH_SIZE"),
            "timeout -s KILL 120 " + PREP_COMMAND.format(pmc="--pmc WRITE_SIZE", sub="WRITE_SIZE"),
            "timeout -s KILL 120 " + PREP_COMMAND.format(pmc="--pmc " + SQ_COUNTERS, sub="SQ"),
            "python bench.py --summarize-prep DIR"]
    lines = [f"# Feature-map kernels (vda_prep), {cfg.name} ({cfg.batch} x {cfg.heads} heads, "
             f"{cfg.frames} frames of {cfg.height} x {cfg.width} tokens, d_k = {cfg.d_k}, "
             f"d_v = {cfg.d_v}, bf16)", "",
             "Commands (from the repository root, on one MI355X; DIR = an output folder):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "| kernel | calls | average (us) | algorithmic GB/s | fp32 TFLOP/s (of "
              f"{VALU_FP32_PEAK / 1e12:.1f}) | HBM read (B) | HBM written (B) | total / algorithmic |",
              "|---|---|---|---|---|---|---|---|"]
    for k in PREP_KERNELS:
        if k not in durations:
            continue
        c, a = durations[k]
        rb = per["FETCH_SIZE"].get(k, 0.0) * 1024 * scale["FETCH_SIZE"]
        wb = per["WRITE_SIZE"].get(k, 0.0) * 1024 * scale["WRITE_SIZE"]
        lines.append(f"| {k} | {c} | {a:.1f} | {alg[k] / (a * 1e-6) / 1e9:.0f} | "
                     f"{flops[k] / (a * 1e-6) / 1e12:.1f} | {rb:.4g} | {wb:.4g} | "
                     f"{(rb + wb) / alg[k]:.3f} |")
    lines += ["", f"Counter scale factors (torch.add calibration in the same runs): FETCH x "
              f"{scale['FETCH_SIZE']:.3f}, WRITE x {scale['WRITE_SIZE']:.3f}."]
    sq_path = os.path.join(prep_dir, "SQ", "p_counter_collection.csv")
    if os.path.exists(sq_path):
        sq_kvg = kv_grid_of(sq_path, "Grid_Size")
        lines += sq_table(sq_path, PREP_KERNELS,
                          lambda r: prep_kind(r["Kernel_Name"], int(r["Grid_Size"]), sq_kvg))
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"prep_kernels_{cfg.name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize(prof_dir, cfg_id):
    """Write the profiles/ summaries from the rocprofv3 output of PROFILE_COMMANDS
    (DIR = prof_dir): kernel durations, and HBM bytes per launch from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for torch.add over the q and gate tensors (2 x bytes read, 1 x written)."""
    import collections
    import csv
    import workloads as W

    cfg = W.CONFIGS[cfg_id]
    eb = 2 if cfg.dtype == "bf16" else 4
    copy_bytes = cfg.units * cfg.frames * cfg.tokens * cfg.d_v * eb
    known = {"FETCH_SIZE": 2 * copy_bytes, "WRITE_SIZE": copy_bytes}
    alg = algorithmic(cfg)
    per = {}   # counter -> kernel -> mean KiB per dispatch
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        disp = collections.defaultdict(float)
        names = {}
        with open(os.path.join(prof_dir, ctr, "p_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                k = short_kernel_name(r["Kernel_Name"])
                if k is None or r["Counter_Name"] != ctr:
                    continue
                disp[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
                names[int(r["Dispatch_Id"])] = k
        acc = collections.defaultdict(list)
        for i, v in sorted(disp.items()):
            acc[names[i]].append(v)
        acc["copy"] = acc["copy"][-CEILING_CALLS:]  # earlier adds belong to input generation
        per[ctr] = {k: sum(v) / len(v) for k, v in acc.items()}
    scale = {c: known[c] / (per[c]["copy"] * 1024.0) for c in per}
    durations = {}
    with open(os.path.join(prof_dir, "trace", "vda_kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            k = short_kernel_name(r["Name"])
            if k and k != "copy":
                durations[k] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3)
    # the launches of the bench's timed steps: each kernel's calls after the
    # warm-up ones, in launch order
    launches = collections.defaultdict(list)
    with open(os.path.join(prof_dir, "trace", "vda_kernel_trace.csv")) as fh:
        for r in csv.DictReader(fh):
            k = short_kernel_name(r["Kernel_Name"])
            if k and k != "copy":
                launches[k].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    timed, serial = {}, {}
    for k, v in launches.items():
        v.sort()
        sel = v[TRACE_WARMUP:TRACE_WARMUP + TRACE_STEPS]
        if sel:
            timed[k] = sum(e - b for b, e in sel) / len(sel) / 1e3
        sel = v[TRACE_WARMUP + TRACE_STEPS:TRACE_WARMUP + 2 * TRACE_STEPS]
        if sel:
            serial[k] = sum(e - b for b, e in sel) / len(sel) / 1e3
    os.makedirs(PROFILES, exist_ok=True)
    order = [k for k in KERNELS if k in durations]
    head = (f"{cfg.name} workload ({cfg.units} heads x {cfg.frames} frames x {cfg.tokens} "
            f"tokens, d_k = {cfg.d_k}, d_v = {cfg.d_v}, {cfg.text_tokens} text tokens)")
    lines = [f"# VDA forward kernels, {head}", "",
             "Commands (from the repository root, on one MI355X; DIR = an output folder):", ""]
    cmd = {c: PROFILE_COMMANDS[c].replace("CFG", str(cfg_id)) for c in PROFILE_COMMANDS}
    lines += [f"    {cmd[c]}" for c in ("stats", "FETCH_SIZE", "WRITE_SIZE", "MFMA", "OCC")]
    lines += [f"    python bench.py --summarize DIR --config {cfg_id}", "",
              "## Kernel durations (`vda_kernel_stats.csv`, `vda_kernel_trace.csv`)", "",
              f"All calls: {TRACE_WARMUP} warm-up steps, {TRACE_STEPS} timed steps, "
              f"{TRACE_STEPS} per-stage breakdown steps (one launch of each kernel per "
              "step). Timed steps: vda_forward. Breakdown steps: vda_forward_timed, the "
              "same launches with the bench's stage events between them.", "",
              "| kernel | calls | average, all calls (us) | min (us) | max (us) | "
              "average, timed steps (us) | average, breakdown steps (us) | "
              "algorithmic GB/s (breakdown) |",
              "|---|---|---|---|---|---|---|---|"]
    for k in order:
        c, a, lo, hi = durations[k]
        tk = timed.get(k, a)
        sk = serial.get(k, a)
        lines.append(f"| {k} | {c} | {a:.1f} | {lo:.1f} | {hi:.1f} | {tk:.1f} | {sk:.1f} | "
                     f"{alg[k][0] / (sk * 1e-6) / 1e9:.0f} |")
    lines += ["", "Sum of the breakdown-step averages: "
              f"{sum(serial.get(k, durations[k][1]) for k in order):.1f} us per forward step."]
    mfma_path = os.path.join(prof_dir, "MFMA", "p_counter_collection.csv")
    if os.path.exists(mfma_path):
        # per dispatch: MOPS (x 512 flop), MFMA busy cycles summed over the SIMDs,
        # GPU-active cycles (the dispatch's duration in clocks)
        ctr = collections.defaultdict(lambda: collections.defaultdict(float))
        kname = {}
        with open(mfma_path) as fh:
            for r in csv.DictReader(fh):
                k = short_kernel_name(r["Kernel_Name"])
                if k is None or k == "copy":
                    continue
                i = int(r["Dispatch_Id"])
                kname[i] = k
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    ctr[i]["GRBM_GUI_ACTIVE"] = max(ctr[i]["GRBM_GUI_ACTIVE"],
                                                    float(r["Counter_Value"]))
                else:
                    ctr[i][r["Counter_Name"]] += float(r["Counter_Value"])
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for i, c in ctr.items():
            for name, val in c.items():
                agg[kname[i]][name].append(val)
        lines += ["", "## MFMA counters per launch (`SQ_INSTS_VALU_MFMA_MOPS_*`)", "",
                  "Executed MFMA flops = MOPS x 512 (hi/lo splits execute more than the algorithmic "
                  "flops); rates use the breakdown-step average duration; peaks: bf16 2516.6, fp32 matrix "
                  "157.3 TFLOP/s.", "",
                  "| kernel | bf16 flops executed | fp32 flops executed | algorithmic bf16 flops | "
                  "executed bf16 TFLOP/s (% of peak) | executed fp32 TFLOP/s (% of peak) |",
                  "|---|---|---|---|---|---|"]
        for k in order:
            if k not in agg:
                continue
            m = {name: sum(v) / len(v) for name, v in agg[k].items()}
            algf = alg[k][1] if alg[k][1] is not None else 0
            sec = serial.get(k, durations[k][1]) * 1e-6
            fb = m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) * 512
            ff = m.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0) * 512
            lines.append(f"| {k} | {fb:.4g} | {ff:.4g} | {algf:.4g} | "
                         f"{fb / sec / 1e12:.0f} ({100 * fb / sec / BF16_PEAK:.1f}%) | "
                         f"{ff / sec / 1e12:.1f} ({100 * ff / sec / 157.3e12:.1f}%) |")
    lines += sq_table(os.path.join(prof_dir, "OCC", "p_counter_collection.csv"), order)
    lines += ["", "## HBM traffic per launch (`FETCH_SIZE`, `WRITE_SIZE`)", "",
              f"Scale factors from torch.add over two {copy_bytes} B tensors into a third: "
              f"FETCH x {scale['FETCH_SIZE']:.3f}, WRITE x {scale['WRITE_SIZE']:.3f} "
              "(counter KiB x 1024 x factor = bytes).", "",
              "| kernel | FETCH (KiB) | WRITE (KiB) | read (B) | written (B) | total (B) | "
              "algorithmic (B) | total / algorithmic |", "|---|---|---|---|---|---|---|---|"]
    for k in order:
        f, w = per["FETCH_SIZE"].get(k), per["WRITE_SIZE"].get(k)
        if f is None or w is None:
            continue
        rb = f * 1024 * scale["FETCH_SIZE"]
        wb = w * 1024 * scale["WRITE_SIZE"]
        lines.append(f"| {k} | {f:.0f} | {w:.0f} | {rb:.4g} | {wb:.4g} | {rb + wb:.4g} | "
                     f"{alg[k][0]:.4g} | {(rb + wb) / alg[k][0]:.3f} |")
        rec = {"kernel": k, "workload": cfg.name, "source_sha256": source_digest(k),
               "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w,
               "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"],
               "read_bytes_per_launch": rb, "write_bytes_per_launch": wb,
               "hbm_bytes_per_launch": rb + wb, "algorithmic_bytes_per_launch": alg[k][0],
               "commands": [cmd["FETCH_SIZE"], cmd["WRITE_SIZE"],
                            f"python bench.py --summarize DIR --config {cfg_id}"]}
        with open(os.path.join(PROFILES, f"traffic_{k}_{cfg.name}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
    with open(os.path.join(PROFILES, f"vda_kernels_{cfg.name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(d, cfg, budget_s):
    """The fp64 oracle on whole units of the same inputs until ~budget_s of CPU
    time (passes over all units are repeated while the budget lasts, so that
    small workloads are timed over more than one pass)."""
    import numpy as np
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info

    feats = ("q", "k", "v", "gate", "text_k", "text_v")
    done = 0
    elapsed = 0.0
    passes = 0
    while elapsed < budget_s:
        for u in range(cfg.units):
            x = {}
            for name, t in d.items():
                a = W.tensor_to_host(t if name == "rms_weight" else t[u:u + 1])
                x[name] = W.to_f64(a, cfg.dtype) if name in feats else a.astype(np.float64)
            t0 = time.perf_counter()
            oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["gate"], x["text_k"],
                           x["text_v"], x["text_beta"], x["rms_weight"], chunk=cfg.chunk,
                           radius=cfg.radius, eps=cfg.rms_eps, alpha=x.get("alpha"),
                           seed_mode=SEED_MODE)
            elapsed += time.perf_counter() - t0
            done += 1
            if passes == 0:
                log(f"[bench] oracle unit {u}: {elapsed:.1f} s total")
            if elapsed >= budget_s:
                break
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    th = done * cfg.frames * cfg.tokens
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": th / elapsed, "unit": "token-heads/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{done} unit passes over {min(done, cfg.units)} of the {cfg.units} units "
                      f"of the same inputs (all {cfg.frames} frames x {cfg.tokens} tokens each), "
                      f"fp64 numpy, {elapsed:.2f} s"}


SEED_MODE = 1  # the text written into both states at beta / 2 (set from --seed-mode)
ARITH = {"solver": 0, "fp32_products": 0}  # descriptor options (set from --solver, --fp32-products)


def make_desc(cfg, **arith):
    import frame_wise_delta_gram_amd as vda
    a = dict(ARITH, **arith)
    return vda.make_desc(cfg.units, cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k, cfg.d_v,
                         cfg.chunk, cfg.radius, cfg.rms_eps, SEED_MODE,
                         vda.VDA_DTYPE_BF16 if cfg.dtype == "bf16" else vda.VDA_DTYPE_F32,
                         int(cfg.anchors), cfg.rule, a["fp32_products"],
                         a["solver"] if cfg.rule == 0 else 0)


def state_growth(cfg, d):
    """Largest Frobenius norm over all boundary states of all units, for each
    update rule on the same inputs (App. A.2: the batched rule's factor I - A
    expands once an eigenvalue of A passes 2)."""
    import dataclasses
    import torch
    import frame_wise_delta_gram_amd as vda
    res = {}
    n = cfg.n_chunks
    P = torch.empty((cfg.units, n + 1, cfg.d_v, cfg.d_k), device="cuda")
    R = torch.empty_like(P)
    for rule, name in ((0, "frame-wise (I + A)^-1"), (1, "batched I - A"),
                       (2, "batched I - A/U, keys / sqrt(U)")):
        desc = make_desc(dataclasses.replace(cfg, rule=rule))
        ws = torch.empty(max(vda.vda_workspace_bytes(desc), 1), dtype=torch.uint8,
                         device="cuda")
        vda.vda_debug_states(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                             d["text_beta"], P, R, ws)
        torch.cuda.synchronize()
        norms = torch.cat([torch.linalg.matrix_norm(P).flatten(),
                           torch.linalg.matrix_norm(R).flatten()])
        fin = torch.isfinite(norms)
        res[name] = {"max_state_norm": float(norms[fin].max()) if bool(fin.any()) else None,
                     "seed_norm": float(torch.linalg.matrix_norm(P[:, 0]).max()),
                     "non_finite_states": int((~fin).sum()), "states": int(norms.numel())}
        del ws
    return res


def time_steps(cfg, d, steps, warmup):
    """Run the forward pass on the current stream: `warmup` untimed steps, then
    `steps` timed steps of vda_forward (vda_forward_decay when d holds decay
    gates), then `steps` more steps of vda_forward_timed, the same launches with
    all six stage events between them, for the per-stage breakdown.  d is one input set, or a list of input sets that the steps take
    in turn (step i reads copy i mod len(d) and writes its own output: for
    workloads small enough to stay in the 256 MB MALL, so that every step
    streams its inputs from HBM).  Returns (seconds for the timed steps, dict of
    average ms: per stage from the breakdown pass, "timed_readout" and
    "timed_stats" the same two stages, and the median / minimum of the
    breakdown pass's per-step totals)."""
    import torch
    import frame_wise_delta_gram_amd as vda

    copies = d if isinstance(d, list) else [d]
    desc = make_desc(cfg)
    ws = torch.empty(max(vda.vda_workspace_bytes(desc), 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fws = []
    for c in copies:
        out = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), device="cuda",
                          dtype=c["q"].dtype)
        fws.append((desc, c["q"], c["k"], c["v"], c["beta"], c.get("alpha"), c["gate"],
                    c["text_k"], c["text_v"], c["text_beta"], c["rms_weight"], out, ws))

    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    events = []
    for _ in range(max(steps, 1)):
        row = []
        for _ in range(6):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            row.append(e.value)
        events.append(row)

    def elapsed_ms(row, a, b):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(row[a]),
                                   ctypes.c_void_p(row[b])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def forward(args):  # the untimed entry point (decay gates: vda_forward_decay)
        desc_, q, k, v, beta, alpha, gate, tk, tv, tb, w, out, ws_ = args
        if alpha is None:
            vda.vda_forward(desc_, q, k, v, beta, gate, tk, tv, tb, w, out, ws_, stream=stream)
        else:
            vda.vda_forward_decay(desc_, q, k, v, beta, alpha, gate, tk, tv, tb, w, out, ws_,
                                  stream=stream)

    log(f"[bench] {cfg.name}: warmup {warmup}")
    for i in range(warmup):
        forward(fws[i % len(fws)])
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for i in range(steps):
        forward(fws[i % len(fws)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    avg = {}

    log(f"[bench] {cfg.name}: per-stage breakdown over {steps} more steps")
    for i in range(steps):
        vda.vda_forward_timed(*fws[i % len(fws)], events[i], stream=stream)
    torch.cuda.synchronize()
    stage_ms = {s: [elapsed_ms(events[i], j, j + 1) for i in range(steps)]
                for j, s in enumerate(STAGES)}
    for row in events:
        for e in row:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    per_step = sorted(sum(stage_ms[s][i] for s in STAGES) for i in range(steps))
    avg.update({s: sum(v) / len(v) for s, v in stage_ms.items()})
    avg["timed_stats"] = avg["stats"]
    avg["timed_readout"] = avg["readout"]
    avg["step_events_median"] = per_step[len(per_step) // 2]
    avg["step_events_min"] = per_step[0]
    return elapsed, avg


def split_steps(avg_ms):
    """(per-stage averages, {median, min} of the per-step event totals)."""
    stages = {s: avg_ms[s] for s in STAGES}
    return stages, {"median": avg_ms["step_events_median"], "min": avg_ms["step_events_min"]}


def roofline_of(cfg, avg_ms):
    """Roofline of the dominant HBM-bound kernel (statistics or readout), with
    its average launch duration from the breakdown pass's stage events (one
    launch per stage)."""
    alg = algorithmic(cfg)
    dominant = max(("stats", "readout"), key=lambda s: avg_ms["timed_" + s])
    ms = avg_ms["timed_" + dominant]
    bytes_ = stage_alg(alg, dominant)[0]
    achieved = bytes_ / (ms * 1e-3)
    return {"bound": "hbm", "kernel": dominant, "achieved": achieved / 1e9,
            "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": achieved / HBM_PEAK,
            "traffic": measured_traffic(dominant, cfg.name),
            "algorithmic_bytes_per_launch": bytes_, "avg_launch_ms": ms}


MALL_BYTES = 256 << 20  # MI355X Infinity Cache


def input_copies(cfg):
    """Input sets the steps of ``cfg`` rotate through: enough that the steps'
    inputs and outputs together exceed four times the MALL (at most 64), so
    that no step finds its inputs cached; one set for the large workloads."""
    eb = 2 if cfg.dtype == "bf16" else 4
    per = cfg.token_heads * ((2 * cfg.d_k + 3 * cfg.d_v) * eb + 4)
    return max(1, min(64, -(-4 * MALL_BYTES // max(per, 1))))


def bench_config(cfg_id, steps, warmup, cpu_seconds):
    """One more workload (the tiny, small, medium and stress configs): its own
    throughput, per-stage breakdown, the roofline of its dominant kernel, the
    HBM fraction of the whole op, and the fp64 oracle on a bounded sample of
    its inputs."""
    import torch
    import workloads as W
    cfg = W.CONFIGS[cfg_id]
    n = input_copies(cfg)
    log(f"[bench] generating {n} input set(s) of {cfg.name} on the device")
    copies = [W.device_inputs(cfg, seed=i) for i in range(n)]
    torch.cuda.synchronize()
    elapsed, avg_ms = time_steps(cfg, copies, steps, warmup)
    alg = algorithmic(cfg)
    ms_step = elapsed * 1e3 / steps
    total_bytes = stage_alg(alg, "stats")[0] + alg["readout"][0]
    res = {"workload": cfg.name, "units": cfg.units, "frames": cfg.frames,
           "tokens_per_frame": cfg.tokens, "d_k": cfg.d_k, "d_v": cfg.d_v,
           "text_tokens": cfg.text_tokens, "dtype": cfg.dtype, "steps": steps,
           "input_sets": n, "ms_per_step": ms_step,
           "value": cfg.token_heads * steps / elapsed, "unit": "token-heads/s",
           "roofline": roofline_of(cfg, avg_ms),
           "hbm_frac_whole_op": total_bytes / (ms_step * 1e-3) / HBM_PEAK,
           "hbm_floor_ms": total_bytes / HBM_PEAK * 1e3,
           "stage_ms": split_steps(avg_ms)[0], "step_ms_from_events": split_steps(avg_ms)[1]}
    if cpu_seconds > 0:
        log(f"[bench] CPU oracle baseline, {cfg.name}")
        res["cpu_baseline"] = cpu_baseline(copies[0], cfg, cpu_seconds)
    del copies
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4,
                    help="workload id (4 = 768p-bf16, 6 = the same with decay gates)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU budget of the oracle baseline (0 disables it)")
    ap.add_argument("--decay-steps", type=int, default=None,
                    help="steps of the decay measurement that follows the 768p-bf16 one "
                         "(default: --steps; 0 disables it)")
    ap.add_argument("--batched-steps", type=int, default=None,
                    help="steps of the batched comparison rule measurement on the 768p-bf16 "
                         "inputs (default: --steps; 0 disables it)")
    ap.add_argument("--prep-steps", type=int, default=None,
                    help="steps of the feature-map (vda_prep) measurement on the 768p head share "
                         "(default: --steps; 0 disables it)")
    ap.add_argument("--seed-mode", type=int, default=1, choices=(0, 1),
                    help="text seed: 1 = the text written into both states at beta / 2 (the "
                         "workload's statement, default), 0 = half the text state S_T / 2")
    ap.add_argument("--solver", type=int, default=0, choices=(0, 1),
                    help="transition solver: 0 = block sweep (default), 1 = blocked Cholesky")
    ap.add_argument("--fp32-products", type=int, default=0, choices=(0, 1),
                    help="bf16 features: 1 = composition and scan with fp32 MFMA products "
                         "(default 0: split-bf16 products)")
    ap.add_argument("--variant-steps", type=int, default=None,
                    help="steps of the solver / product variants timed on the headline "
                         "workload (default: --steps; 0 disables them)")
    ap.add_argument("--other-configs", default="1,2,3,5",
                    help="workload ids timed after the headline one, each with its own "
                         "roofline and oracle baseline (empty: none)")
    ap.add_argument("--summarize-prep", metavar="DIR",
                    help="write the feature-map profile summary from rocprofv3 output under DIR")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 output under DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.config)
        return
    if args.summarize_prep:
        summarize_prep(args.summarize_prep)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the VDA forward shards by head with no "
              "communication inside the op, and this benchmark times a single MI355X. "
              "Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    global SEED_MODE
    SEED_MODE = args.seed_mode
    ARITH.update(solver=args.solver, fp32_products=args.fp32_products)
    import torch
    import frame_wise_delta_gram_amd as vda
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    vda.load_library()
    cfg = W.CONFIGS[args.config]
    log(f"[bench] generating {cfg.name} inputs on the device")
    d = W.device_inputs(cfg)
    torch.cuda.synchronize()
    elapsed, avg_ms = time_steps(cfg, d, args.steps, args.warmup)

    # context: what a plain library kernel with the readout's traffic mix (two
    # reads + one write of the same tensors) reaches on this GPU
    ceil_out = torch.empty_like(d["q"])
    for _ in range(2):
        torch.add(d["q"], d["gate"], out=ceil_out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch.add(d["q"], d["gate"], out=ceil_out)
    e1.record()
    torch.cuda.synchronize()
    add_ms = e0.elapsed_time(e1) / 5
    add_bytes = 3 * d["q"].numel() * d["q"].element_size()
    del ceil_out

    th = cfg.token_heads
    ms_per_step = elapsed * 1e3 / args.steps
    value = th * args.steps / elapsed
    alg = algorithmic(cfg)
    stats_flops = stage_alg(alg, "stats")[1]
    mfma = {
        "whole_op": (stats_flops + alg["readout"][1]) / (ms_per_step * 1e-3) / BF16_PEAK,
        "stats": stats_flops / (avg_ms["timed_stats"] * 1e-3) / BF16_PEAK,
        "readout": alg["readout"][1] / (avg_ms["timed_readout"] * 1e-3) / BF16_PEAK,
    }
    hbm_whole = ((stage_alg(alg, "stats")[0] + alg["readout"][0]) / (ms_per_step * 1e-3)
                 / HBM_PEAK)
    # the MFMA fraction a contraction can reach when its operands stream from HBM
    # at the full 8 TB/s: arithmetic intensity x HBM peak / MFMA peak
    def ceiling(flops, bytes_):
        return min(1.0, flops / bytes_ * HBM_PEAK / BF16_PEAK)
    mfma_ceiling = {
        "whole_op": ceiling(stats_flops + alg["readout"][1],
                            stage_alg(alg, "stats")[0] + alg["readout"][0]),
        "stats": ceiling(stats_flops, stage_alg(alg, "stats")[0]),
        "readout": ceiling(alg["readout"][1], alg["readout"][0]),
    }
    line = {
        "metric": METRIC, "value": value, "unit": "token-heads/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "units": cfg.units, "frames": cfg.frames,
                   "tokens_per_frame": cfg.tokens, "d_k": cfg.d_k, "d_v": cfg.d_v,
                   "text_tokens": cfg.text_tokens, "chunk": cfg.chunk, "radius": cfg.radius,
                   "decay": cfg.alpha_mu is not None, "state": "fp32",
                   "seed_mode": SEED_MODE, "solver": ["sweep", "cholesky"][args.solver],
                   "products": ["split-bf16", "fp32"][args.fp32_products or cfg.dtype == "f32"],
                   "parallelism": "single GPU"},
        "roofline": roofline_of(cfg, avg_ms),
        "mfma_frac": mfma,
        "mfma_ceiling_at_hbm_peak": mfma_ceiling,
        "mfma_frac_of_ceiling": {k: mfma[k] / mfma_ceiling[k] for k in mfma},
        "hbm_frac_whole_op": hbm_whole,
        "stage_ms": split_steps(avg_ms)[0],
        "step_ms_from_events": split_steps(avg_ms)[1],
        "stream_ceiling": {"kernel": "torch.add over the q and gate tensors (2 reads + 1 write)",
                           "GB/s": add_bytes / (add_ms * 1e-3) / 1e9, "ms": add_ms},
    }
    rl = line["roofline"]
    line["stream_ceiling"]["dominant_kernel_frac"] = (rl["achieved"] * 1e9
                                                      / (add_bytes / (add_ms * 1e-3)))
    if args.cpu_seconds > 0:
        log("[bench] CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(d, cfg, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    line["batched_rule"] = None
    if args.config == 4 and args.batched_steps != 0:
        import dataclasses
        bcfg = dataclasses.replace(cfg, rule=2)
        bsteps = args.steps if args.batched_steps is None else args.batched_steps
        el, ms = time_steps(bcfg, d, bsteps, args.warmup)
        bvalue = th * bsteps / el
        line["batched_rule"] = {
            "workload": cfg.name, "rule": "SANA-WM frozen-state batched update with frame-size "
            "key scaling (rule 2)", "steps": bsteps, "ms_per_step": el * 1e3 / bsteps,
            "value": bvalue, "unit": "token-heads/s", "relative_to_vda": bvalue / value,
            "stage_ms": split_steps(ms)[0], "state_growth": state_growth(cfg, d)}
    line["variants"] = None
    vsteps = args.steps if args.variant_steps is None else args.variant_steps
    if vsteps > 0 and args.config == 4:
        line["variants"] = {}
        base = dict(ARITH)
        for name, arith in (("cholesky_solver", dict(solver=1)),
                            ("sweep_solver", dict(solver=0)),
                            ("fp32_products", dict(fp32_products=1)),
                            ("split_bf16_products", dict(fp32_products=0))):
            ARITH.update(base, **arith)
            log(f"[bench] variant {name}")
            el, ms = time_steps(cfg, d, vsteps, args.warmup)
            st = split_steps(ms)[0]
            line["variants"][name] = {
                "descriptor": dict(ARITH), "steps": vsteps, "ms_per_step": el * 1e3 / vsteps,
                "value": th * vsteps / el, "unit": "token-heads/s", "stage_ms": st}
        ARITH.update(base)
    decay_steps = args.steps if args.decay_steps is None else args.decay_steps
    line["decay"] = None
    del d
    if decay_steps > 0 and args.config == 4:
        dcfg = W.CONFIGS[6]
        log(f"[bench] generating {dcfg.name} inputs on the device")
        dd = W.device_inputs(dcfg)
        torch.cuda.synchronize()
        el, ms = time_steps(dcfg, dd, decay_steps, args.warmup)
        dvalue = dcfg.token_heads * decay_steps / el
        line["decay"] = {
            "workload": dcfg.name, "entry_point": "vda_forward_decay", "steps": decay_steps,
            "ms_per_step": el * 1e3 / decay_steps, "value": dvalue, "unit": "token-heads/s",
            "alpha": f"sigmoid(N({dcfg.alpha_mu}, 1)) per (unit, frame, key channel), fp32",
            "relative_to_plain": dvalue / value, "stage_ms": split_steps(ms)[0],
            "step_ms_from_events": split_steps(ms)[1], "roofline": roofline_of(dcfg, ms)}
        del dd
    prep_steps = args.steps if args.prep_steps is None else args.prep_steps
    line["prep"] = None
    if prep_steps > 0 and args.config == 4:
        line["prep"] = bench_prep(W.PREP_CONFIGS[3], prep_steps, args.warmup)
    line["configs"] = {}
    for cid in [int(x) for x in args.other_configs.split(",") if x.strip()]:
        if cid != args.config:
            r = bench_config(cid, args.steps, args.warmup, min(args.cpu_seconds, 3.0))
            line["configs"][r["workload"]] = r
    print(json.dumps(line), flush=True)


VALU_FP32_PEAK = 256 * 4 * 16 * 2 * 2.4e9  # unpacked fp32 FMA: CUs x SIMDs x lanes x 2 flop x clock


def prep_algorithmic(cfg, query_pass=True):
    """Bytes (q, k, v read once, q', k', v' written once, filters; without the
    query pass k and v only) and fp32 flops (30 multiply-adds per convolved
    element of k and v) of one vda_prep call."""
    eb = 2 if cfg.dtype == "bf16" else 4
    rows = cfg.batch * cfg.frames * cfg.tokens * cfg.heads
    elems = rows * ((2 if query_pass else 1) * cfg.d_k + cfg.d_v)
    filt = cfg.heads * (cfg.d_k + cfg.d_v) * 30 * 4
    return 2 * elems * eb + filt, 2 * 30 * rows * (cfg.d_k + cfg.d_v)


def _time_calls(fn, steps, warmup, stream):
    """Average ms of fn() over `steps` calls after `warmup`, by events on stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _prep_line(cfg, ms, query_pass):
    bytes_, flops = prep_algorithmic(cfg, query_pass)
    return {"ms_per_call": ms, "token_heads_per_s": cfg.units * cfg.frames * cfg.tokens / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved": flops / (ms * 1e-3) / 1e12,
                         "peak": VALU_FP32_PEAK / 1e12, "unit": "TFLOP/s",
                         "frac": flops / (ms * 1e-3) / VALU_FP32_PEAK,
                         "hbm_GB/s": bytes_ / (ms * 1e-3) / 1e9,
                         "hbm_frac": bytes_ / (ms * 1e-3) / HBM_PEAK,
                         "algorithmic_bytes": bytes_, "flops": flops}}


def bench_prep(cfg, steps, warmup):
    """The feature map on ``cfg`` (inputs resident): vda_prep on k and v alone
    (the query map left to the forward's readout) and with its query pass, each
    with its ALU and HBM fractions; then the linear branch from projection
    outputs both ways, vda_prep then vda_forward on the 768p share: the query
    pass's q' in the unit layout, or the raw projection q normalised inside the
    readout (q_heads = heads, q_l2_eps = the feature map's eps)."""
    import torch
    import frame_wise_delta_gram_amd as vda
    import workloads as W
    log(f"[bench] generating {cfg.name} inputs on the device")
    d = W.device_prep_inputs(cfg)
    desc = vda.make_prep_desc(cfg.batch, cfg.heads, cfg.frames, cfg.height, cfg.width, cfg.d_k,
                              cfg.d_v, cfg.eps, vda.VDA_DTYPE_BF16)
    N, F, U = cfg.units, cfg.frames, cfg.tokens
    qo = torch.empty((N, F, U, cfg.d_k), dtype=torch.bfloat16, device="cuda")
    ko = torch.empty_like(qo)
    vo = torch.empty((N, F, U, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    w = (d["wk_s"], d["wk_t"], d["wv_s"], d["wv_t"])

    def prep_qkv():
        vda.vda_prep(desc, d["q"], d["k"], d["v"], *w, qo, ko, vo, stream=stream)

    def prep_kv():
        vda.vda_prep(desc, None, d["k"], d["v"], *w, None, ko, vo, stream=stream)

    log(f"[bench] {cfg.name}: timing {steps} calls, k and v only, then with the query pass")
    ms_kv = _time_calls(prep_kv, steps, warmup, stream)
    ms_qkv = _time_calls(prep_qkv, steps, warmup, stream)
    res = {"workload": cfg.name, "entry_point": "vda_prep", "steps": steps}
    res.update(_prep_line(cfg, ms_kv, False))
    res["scope"] = ("k and v (q = q_out = NULL; the query map runs in the forward's readout, "
                    "q_heads / q_l2_eps)")
    res["with_query_pass"] = _prep_line(cfg, ms_qkv, True)
    fc = W.CONFIGS[4]
    if (fc.units, fc.frames, fc.tokens, fc.d_k, fc.d_v) == (N, F, U, cfg.d_k, cfg.d_v):
        log(f"[bench] {cfg.name}: vda_prep then vda_forward, both ways")
        fi = W.device_inputs(fc)
        del fi["q"], fi["k"], fi["v"]
        fdesc = make_desc(fc)
        qdesc = make_desc(fc)
        qdesc.q_heads, qdesc.q_l2_eps = cfg.heads, cfg.eps
        ws = torch.empty(vda.vda_workspace_bytes(fdesc), dtype=torch.uint8, device="cuda")
        out = torch.empty((N, F, U, fc.d_v), dtype=torch.bfloat16, device="cuda")
        q_proj = d["q"].view(cfg.batch, F, U, cfg.heads, cfg.d_k)
        rest = (fi["beta"], fi["gate"], fi["text_k"], fi["text_v"], fi["text_beta"],
                fi["rms_weight"], out, ws)

        def pipe_unit_q():
            prep_qkv()
            vda.vda_forward(fdesc, qo, ko, vo, *rest, stream=stream)

        def pipe_query_map():
            prep_kv()
            vda.vda_forward(qdesc, q_proj, ko, vo, *rest, stream=stream)

        ms_a = _time_calls(pipe_unit_q, steps, warmup, stream)
        ms_b = _time_calls(pipe_query_map, steps, warmup, stream)
        res["prep_then_forward"] = {
            "forward_workload": fc.name,
            "query_pass_then_unit_layout_q_ms": ms_a,
            "query_map_in_readout_ms": ms_b,
            "speedup": ms_a / ms_b}
        del fi, ws, out
    return res


if __name__ == "__main__":
    main()
