#!/usr/bin/env python3
"""Benchmark of the D-Quant hot path on one MI355X.

Workload (default): Llama-3.1-8B-shaped layer at its maximum batch -- batch
128, 32 query / 8 kv heads, head_dim 128, 8K-token prompt, 34-byte containers
(2.25 bits/value with the fp16 norm), keys 8 levels, values 6, bf16 K/V with 4
outlier channels per head.  Synthetic data (synth/), no model weights.

Untimed setup: draw K/V, encode the whole prompt into the compressed pools
(timed separately for encode vectors/s).  One timed step = one decode step,
one call of dq_attn_decode_append: the new token's K and V of every
sequence encoded into the pools and attention of every sequence over its
grown context (the call runs the encodes inside the attention launch at
small batch, as a short launch of their own before it at this one).
`value` = compressed KV bytes (containers + fp16 norms) read by attention
per step / time per step, over the timed steps with one event pair around
them all.  The same steps then run again with HIP events around each call's
split-K kernel, on its stream, for the roofline entry (re-encoding a step's
token into its slot writes the same bytes).  Then the steps as two launches
(dq_encode_kv, then dq_attn_decode), and both forms at batch 1 and 4,
eagerly and as HIP-graph replays.

    python bench.py [--steps 16] [--warmup 12] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
COUNTERS = os.path.join(ROOT, "profiles", "attn_splitk_llama31_8b_b128_8k_counters.json")
ATTN_SOURCES = ["kv_cache_entropy_amd/csrc/attention.hip", "kv_cache_entropy_amd/csrc/decode_common.h",
                "kv_cache_entropy_amd/csrc/dq_internal.h", "kv_cache_entropy_amd/csrc/encode_wave.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for p in ATTN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(bytes_per_launch_alg):
    """HBM bytes per attention launch from committed rocprofv3 counters, or
    None when they were taken on a different kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha256_16") != attn_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


# The profiles under profiles/ come from these commands (run from the repo
# root on the GPU machine, one after the other), then
# `python bench.py --summarize-profiles prof_out` on any host.
PROF = "prof_out"
# instruction mix and pipe activity (8 SQ counters and one GRBM counter: one
# rocprofv3 pass)
SQ_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_ACTIVE_INST_VALU",
               "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
PROFILE_CMDS = {
    "trace": ("R=$PWD && mkdir -p $R/" + PROF + " && cd /tmp && export TMPDIR=/tmp && timeout -k 10 900 "
              "rocprofv3 --kernel-trace --stats --output-format csv -d $R/" + PROF + "/trace -o run -- "
              "python3 $R/bench.py > $R/" + PROF + "/trace_bench.json"),
    "fetch": ("R=$PWD && mkdir -p $R/" + PROF + " && cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 "
              "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'attn_splitk|copyBuffer' --output-format csv "
              "-d $R/" + PROF + "/fetch -o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline "
              "--no-compare --no-others --copy-calibration > $R/" + PROF + "/fetch_bench.json"),
    "write": ("R=$PWD && mkdir -p $R/" + PROF + " && cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 "
              "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex 'attn_splitk|copyBuffer' --output-format csv "
              "-d $R/" + PROF + "/write -o run -- python3 $R/bench.py --steps 3 --warmup 1 --no-cpu-baseline "
              "--no-compare --no-others --copy-calibration > $R/" + PROF + "/write_bench.json"),
    "sq": ("R=$PWD && mkdir -p $R/" + PROF + " && cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 "
           "rocprofv3 --pmc " + " ".join(SQ_COUNTERS) + " --kernel-include-regex 'attn_splitk|encode_fast_kernel|encode_rest_kernel' "
           "--output-format csv -d $R/" + PROF + "/sq -o run -- python3 $R/bench.py --steps 3 --warmup 1 "
           "--no-cpu-baseline --no-compare --no-rd --no-paged --no-prefill --no-others > $R/" + PROF
           + "/sq_bench.json"),
    # the LDS gather ceiling of a decode step's table reads (kv_cache_entropy_amd/build.py builds it)
    "lds_gather": ("R=$PWD && mkdir -p $R/" + PROF + " && timeout -k 10 120 "
                   "$R/kv_cache_entropy_amd/_build/lds_gather_probe > $R/" + PROF + "/lds_gather.txt"),
    # the 64K-context workload alone (its split-K launches, MALL evicted before each)
    "trace_c4": ("R=$PWD && mkdir -p $R/" + PROF + " && cd /tmp && export TMPDIR=/tmp && timeout -k 10 600 "
                 "rocprofv3 --kernel-trace --stats --output-format csv -d $R/" + PROF + "/trace_c4 -o run -- "
                 "python3 $R/bench.py --others-only longctx_b4_64k_c29 > $R/" + PROF + "/trace_c4_bench.json"),
}


# Clocks leave their idle state only after tens of milliseconds of sustained
# load: on one box the split-K kernel ran 886-918 us for its first launches
# after a 34 ms idle gap and settled at 775-785 us after ~30 of them.  Each
# timed section is therefore preceded by this much untimed repetition of its
# own work (same inputs, same bytes written).
SETTLE_MS = 100.0


def settle_clocks(run_once, min_ms=SETTLE_MS):
    """Repeats run_once (GPU work, idempotent) until about min_ms of it has
    run; returns the repetitions.  Nothing here is timed."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < 2 or (time.perf_counter() - t0) * 1e3 < min_ms:
        run_once()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()  # keep the host at most a few launches ahead
    torch.cuda.synchronize()
    return n


def _csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(root, name)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _bench_line(path):
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def summarize_profiles(d):
    """Writes the committed summaries from the rocprofv3 CSV output of
    PROFILE_CMDS: the kernel-trace statistics of the default bench command,
    and HBM bytes per split-K launch from FETCH_SIZE / WRITE_SIZE, each
    scaled by what the same counter reads for the 1 GiB device copy that
    --copy-calibration runs (rocprofv3 reports both in KiB per dispatch)."""
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    wl = "llama31_8b_b128_8k"
    src = attn_source_hash()

    # ---- kernel trace
    stats = _csv(_find(os.path.join(d, "trace"), "kernel_stats.csv"))
    live = _bench_line(os.path.join(d, "trace_bench.json"))
    if live.get("attn_source_sha256_16") != src:
        raise SystemExit("trace run was made on a different attention source")
    rows = []
    for r in stats:
        name = r["Name"]
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()
        rows.append((float(r["TotalDurationNs"]), short, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(reverse=True)
    lines = [f"# Kernel trace: decode step, {wl}", "",
             "Batch 128, 32 q / 8 kv heads, 8K context, K 8 levels / V 6 levels in 34-byte containers; "
             "the default bench command (prefill encode, 12 warm-up and 16 timed decode steps, oracle timing "
             "on the host).", "",
             "Command (from the repository root):", "", "```", PROFILE_CMDS["trace"], "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for tot, short, calls, avg, mn, mx, pct in rows[:12]:
        lines.append(f"| `{short}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.2f} |")
    rl = live["roofline"]
    # per-dispatch durations of the split-K kernels by launch shape: the bench
    # also runs them at batch 1 and 4 (the small-batch comparison), so the
    # figure that must agree with the bench line is the one at its grid
    disp, seqd = {}, {}
    for r in _csv(_find(os.path.join(d, "trace"), "kernel_trace.csv")):
        n = r["Kernel_Name"]
        if "attn_splitk_kernel" not in n:
            continue
        key = (n[n.index("attn_splitk_kernel"):n.index(">") + 1], int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        disp.setdefault(key, []).append(dur)
        seqd.setdefault(key, []).append((int(r["Start_Timestamp"]), dur))
    lines += ["", "Split-K kernels per launch shape (rocprofv3 kernel trace, one record per dispatch):", "",
              "| kernel | blocks | launches | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    for (kname, blocks), v in sorted(disp.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        lines.append(f"| `{kname}` | {blocks} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    # the decode step's split-K variant: the one launched most at the bench's
    # shape (dq_attn_decode_append runs the attention without the encode loop
    # when its items fill every round of waves, as at batch 128).  The bench
    # runs its timed steps twice, the second time with HIP events around
    # each split-K launch: those are its launches number warmup + steps ..
    # warmup + 2 steps - 1 at that shape (the two-launch and paged
    # comparisons and the other workloads follow)
    head = sorted(disp.items(), key=lambda kv: (kv[0][1], len(kv[1])))
    kname = head[-1][0][0] if head else "attn_splitk_kernel"
    if head:
        (kname, blocks), _ = head[-1]
        seq = sorted(seqd[(kname, blocks)])
        ns = live["steps"]
        w0 = live["warmup"] + ns
        v = [dur for _, dur in seq[w0:w0 + ns]]
        lines += ["", f"`{kname}` (the decode step's split-K kernel) at the bench's shape "
                  f"({blocks} blocks), the bench's {ns} event-timed steps (its launches {w0} .. {w0 + ns - 1} "
                  f"at that shape): rocprofv3 average {sum(v) / len(v):.1f} us (min {min(v):.1f}, max "
                  f"{max(v):.1f}); the same run's bench line measured {rl['avg_launch_ms'] * 1e3:.1f} us with "
                  f"HIP events around the kernel over those steps, {rl['achieved']:.1f} GB/s of compressed "
                  f"bytes = {rl['frac']:.2%} of 8 TB/s."]
    lines += ["", "Bench line of this run:", "", "```", json.dumps(live), "```"]
    with open(os.path.join(out_dir, f"all_kernels_{wl}_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # ---- HBM counters (of that kernel); kept as they are when this run has none
    if os.path.isdir(os.path.join(d, "fetch")) and os.path.isdir(os.path.join(d, "write")):
        def per_kernel(kind, counter):
            rows = _csv(_find(os.path.join(d, kind), "counter_collection.csv"))
            rows = [r for r in rows if r["Counter_Name"] == counter]
            copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
            cal = max(copies, key=lambda r: float(r["Counter_Value"]))
            att = [float(r["Counter_Value"]) for r in rows if kname in r["Kernel_Name"]]
            bl = _bench_line(os.path.join(d, f"{kind}_bench.json"))
            if bl.get("attn_source_sha256_16") != src:
                raise SystemExit(f"{kind} run was made on a different attention source")
            return float(cal["Counter_Value"]), att
        f_cal, f_att = per_kernel("fetch", "FETCH_SIZE")
        w_cal, w_att = per_kernel("write", "WRITE_SIZE")
        gib_kib = float(1 << 20)
        f_scale, w_scale = gib_kib / f_cal, gib_kib / w_cal
        fetch_b = sum(f_att) / len(f_att) * 1024 * f_scale
        write_b = sum(w_att) / len(w_att) * 1024 * w_scale
        alg = rl["alg_bytes_per_launch"]
        rec = {"kernel": kname, "workload": wl, "source_sha256_16": src,
               "fetch_kib_per_launch_raw": sum(f_att) / len(f_att), "write_kib_per_launch_raw": sum(w_att) / len(w_att),
               "launches": [len(f_att), len(w_att)],
               "copy_1gib_fetch_kib": f_cal, "copy_1gib_write_kib": w_cal,
               "fetch_scale": f_scale, "write_scale": w_scale,
               "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
               "traffic_bytes_per_launch": fetch_b + write_b,
               "alg_bytes_per_launch": alg, "traffic_over_alg": (fetch_b + write_b) / alg,
               "commands": [PROFILE_CMDS["fetch"], PROFILE_CMDS["write"]]}
        with open(os.path.join(out_dir, f"attn_splitk_{wl}_counters.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        md = [f"# HBM counters: {kname}, {wl}", "",
              "Commands (from the repository root), one counter per run:", "", "```",
              PROFILE_CMDS["fetch"], PROFILE_CMDS["write"], "```", "",
              "| | FETCH_SIZE | WRITE_SIZE |", "|---|---:|---:|",
              f"| 1 GiB device copy (KiB) | {f_cal:.0f} | {w_cal:.0f} |",
              f"| scale to bytes moved | {f_scale:.3f} | {w_scale:.3f} |",
              f"| split-K kernel, raw KiB per launch | {rec['fetch_kib_per_launch_raw']:.0f} | "
              f"{rec['write_kib_per_launch_raw']:.0f} |",
              f"| split-K kernel, scaled MB per launch | {fetch_b / 1e6:.1f} | {write_b / 1e6:.1f} |", "",
              f"Algorithmic bytes per launch (containers + fp16 norms of every context token, K and V): "
              f"{alg / 1e6:.1f} MB.  Measured traffic {(fetch_b + write_b) / 1e6:.1f} MB = "
              f"{rec['traffic_over_alg']:.3f} x algorithmic; the writes are the split-K partial results and the "
              f"appended tokens' containers.", ""]
        with open(os.path.join(out_dir, f"attn_splitk_{wl}_counters.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        print(f"wrote profiles for source {src}: traffic {(fetch_b + write_b) / 1e6:.1f} MB per launch")
    if os.path.isdir(os.path.join(d, "sq")):
        summarize_sq(d, kname, wl, src)
    if os.path.isdir(os.path.join(d, "trace_c4")):
        summarize_trace_workload(d, "trace_c4", "longctx_b4_64k_c29", src)
    if os.path.exists(os.path.join(d, "lds_gather.txt")):
        summarize_lds_gather(d)


def summarize_lds_gather(d):
    """The gather microbenchmark's table, with its command."""
    with open(os.path.join(d, "lds_gather.txt")) as f:
        table = f.read().strip()
    md = ["# LDS gather ceiling (MI355X)", "",
          "Dependent random table reads shaped like a decode step (state -> slot -> entry -> state), "
          "one block per CU; `kv_cache_entropy_amd/csrc/probes/lds_gather.hip`, built by "
          "`python -m kv_cache_entropy_amd.build`.", "",
          "Command (from the repository root):", "", "```", PROFILE_CMDS["lds_gather"], "```", "", table, ""]
    with open(os.path.join(ROOT, "profiles", "lds_gather_ceiling.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("wrote the LDS gather summary")


def summarize_trace_workload(d, sub, name, src):
    """Kernel trace of one of the other workloads (`--others-only NAME`):
    its split-K launches against the bench's own HIP-event figure."""
    live = _bench_line(os.path.join(d, f"{sub}_bench.json"))
    if live.get("attn_source_sha256_16") != src:
        raise SystemExit(f"{sub} run was made on a different attention source")
    wrec = live["workloads"][name]
    stats = _csv(_find(os.path.join(d, sub), "kernel_stats.csv"))
    rows = sorted(((float(r["TotalDurationNs"]), r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
                    .replace("void ", "").strip(), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])) for r in stats),
                  reverse=True)
    lines = [f"# Kernel trace: decode attention, {name}", "",
             f"Batch {wrec['batch']}, {wrec['q_heads']} q / {wrec['kv_heads']} kv heads, context "
             f"{wrec['context'][1]}, containers {wrec['container_bytes'][0]}/{wrec['container_bytes'][1]} bytes, "
             f"{wrec['kv_distribution']} data; each timed launch preceded by a 512 MB write that evicts the MALL.",
             "", "Command (from the repository root):", "", "```", PROFILE_CMDS[sub], "```", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for tot, short, calls, avg, mn, mx, pct_ in rows[:10]:
        lines.append(f"| `{short}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct_:.2f} |")
    durs = {}
    for r in _csv(_find(os.path.join(d, sub), "kernel_trace.csv")):
        n = r["Kernel_Name"]
        if "attn_splitk_kernel" in n:
            k = n[n.index("attn_splitk_kernel"):n.index(">") + 1]
            durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, v in sorted(durs.items()):
        lines += ["", f"`{k}`: {len(v)} launches, rocprofv3 median {sorted(v)[len(v) // 2]:.1f} us (min "
                  f"{min(v):.1f}, max {max(v):.1f}); the bench's median of its timed launches (HIP events) was "
                  f"{wrec['split_ms'] * 1e3:.1f} us: {wrec['split_gbps']:.1f} GB/s of compressed bytes = "
                  f"{wrec['hbm_frac']:.2%} of 8 TB/s."]
    lines += ["", "Bench output of this run:", "", "```", json.dumps(wrec), "```"]
    with open(os.path.join(ROOT, "profiles", f"attn_splitk_{name}_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote the {name} trace summary")


def summarize_sq(d, kname, wl, src):
    """Pipe activity of the split-K kernel and the prompt encode from the SQ
    counter pass.  Normalisation: 256 CUs, 1024 SIMDs; GRBM_GUI_ACTIVE sums
    the 8 XCDs' busy cycles, so GRBM_GUI_ACTIVE / 8 is the dispatch's length
    in cycles; a wave64 VALU instruction occupies its 16-lane SIMD 4 cycles."""
    rows = _csv(_find(os.path.join(d, "sq"), "counter_collection.csv"))
    bl = _bench_line(os.path.join(d, "sq_bench.json"))
    if bl.get("attn_source_sha256_16") != src:
        raise SystemExit("sq run was made on a different attention source")
    disp = {}
    for r in rows:
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]))
        disp.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])

    def table(sel):
        n = len(sel)
        avg = {c: sum(v[c] for v in sel) / n for c in SQ_COUNTERS}
        cyc = avg["GRBM_GUI_ACTIVE"] / 8
        return avg, {"dispatches": n, "cycles": cyc,
                     "valu_busy": avg["SQ_ACTIVE_INST_VALU"] * 4 / 1024 / cyc,
                     "lds_active": avg["SQ_LDS_IDX_ACTIVE"] / 256 / cyc,
                     "bank_conflict_share": avg["SQ_LDS_BANK_CONFLICT"] / max(avg["SQ_LDS_IDX_ACTIVE"], 1.0)}

    cmd = PROFILE_CMDS["sq"]
    # split-K at the bench's grid
    att = [(k, v) for k, v in disp.items() if kname in k[1]]
    grid = max(k[2] for k, _ in att)
    avg, der = table([v for k, v in att if k[2] == grid])
    syms = bl["roofline"]["alg_bytes_per_launch"] / (bl["config"]["container_bytes"][0] + 2 +
                                                     bl["config"]["container_bytes"][1] + 2) * 256
    md = [f"# Pipe activity: {kname}, {wl}", "", "Command (from the repository root):", "", "```", cmd, "```", "",
          f"Dispatches of `{kname}` at the bench's grid ({grid // 768} blocks): {der['dispatches']}, averaged.", "",
          "| counter | per dispatch |", "|---|---:|"]
    md += [f"| {c} | {avg[c]:.4g} |" for c in SQ_COUNTERS]
    md += ["", f"Decoded symbols per dispatch (K and V, 128 per container): {syms:.4g}.", "",
           "| derived | value |", "|---|---:|",
           f"| dispatch length, cycles (GRBM_GUI_ACTIVE / 8 XCDs) | {der['cycles']:.4g} |",
           f"| VALU busy (SQ_ACTIVE_INST_VALU x 4 / 1024 SIMDs / cycles) | {der['valu_busy']:.1%} |",
           f"| LDS pipe active (SQ_LDS_IDX_ACTIVE / 256 CUs / cycles) | {der['lds_active']:.1%} |",
           f"| bank-conflict cycles, share of LDS active | {der['bank_conflict_share']:.1%} |",
           f"| VALU lane-ops per decoded symbol (SQ_INSTS_VALU x 64 / symbols) | "
           f"{avg['SQ_INSTS_VALU'] * 64 / syms:.2f} |",
           f"| LDS instructions per symbol step (SQ_INSTS_LDS x 64 / symbols) | "
           f"{avg['SQ_INSTS_LDS'] * 64 / syms:.2f} |", ""]
    with open(os.path.join(ROOT, "profiles", f"attn_splitk_{wl}_sq_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    # prompt encode: the first four encode dispatches are K (first pass,
    # second pass), then V, of the whole prompt
    enc = sorted((k, v) for k, v in disp.items() if "encode_fast_kernel" in k[1] or "encode_rest_kernel" in k[1])[:4]
    names = [("first pass" if "encode_fast_kernel" in k[1] else "second pass") for k, _ in enc]
    if names != ["first pass", "second pass"] * 2:
        raise SystemExit(f"unexpected encode dispatch order: {names}")
    nvec = bl["config"]["batch"] * bl["config"]["context"][1] * bl["config"]["kv_heads"]
    md = ["# Pipe activity: prompt encode (encode_fast_kernel, then encode_rest_kernel), " + wl, "",
          "Command (from the repository root):", "", "```", cmd, "```", "",
          f"The prompt's K, then V: {nvec} vectors each (8 kv heads x {nvec // 8} tokens), one vector per lane; "
          "the first pass runs round 0 of the drift search for every vector, the second the full search "
          "for the few it leaves.", "",
          "| counter | K first | K second | V first | V second |", "|---|---:|---:|---:|---:|"]
    md += [f"| {c} | " + " | ".join(f"{v[c]:.4g}" for _, v in enc) + " |" for c in SQ_COUNTERS]
    edr = [table([v])[1] for _, v in enc]
    md += ["", "| derived | K | V |", "|---|---:|---:|"]
    cyc = [edr[0]["cycles"] + edr[1]["cycles"], edr[2]["cycles"] + edr[3]["cycles"]]
    busy = [(enc[0][1]["SQ_ACTIVE_INST_VALU"] + enc[1][1]["SQ_ACTIVE_INST_VALU"]) * 4 / 1024 / cyc[0],
            (enc[2][1]["SQ_ACTIVE_INST_VALU"] + enc[3][1]["SQ_ACTIVE_INST_VALU"]) * 4 / 1024 / cyc[1]]
    ops = [(enc[0][1]["SQ_INSTS_VALU"] + enc[1][1]["SQ_INSTS_VALU"]) * 64 / nvec,
           (enc[2][1]["SQ_INSTS_VALU"] + enc[3][1]["SQ_INSTS_VALU"]) * 64 / nvec]
    md += [f"| both passes, cycles | {cyc[0]:.4g} | {cyc[1]:.4g} |",
           f"| second pass, share of the cycles | {edr[1]['cycles'] / cyc[0]:.1%} | {edr[3]['cycles'] / cyc[1]:.1%} |",
           f"| VALU busy | {busy[0]:.1%} | {busy[1]:.1%} |",
           f"| VALU lane-ops per vector | {ops[0]:.0f} | {ops[1]:.0f} |", ""]
    with open(os.path.join(ROOT, "profiles", f"encode_{wl}_sq_counters.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(f"wrote SQ counter summaries: split-K VALU {der['valu_busy']:.1%}, LDS {der['lds_active']:.1%}")


def pct(xs):
    """10th, 50th and 90th percentile of a list of times (nearest rank)."""
    v = sorted(xs)
    return [round(v[min(len(v) - 1, int(q * len(v)))], 4) for q in (0.1, 0.5, 0.9)]


def cpu_baseline(w, ck, cv, kc, kn, vc, vn, q, starts, ctx, seconds):
    """The oracle, as it stands, on a bounded sample: decode attention for the
    first n sequences (n grown until ~`seconds` of CPU work), on the host
    cores this process may use."""
    import numpy as np
    import oracle
    import synth
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    ock = oracle.Codec(8, ck.C, seed=ck.seed, hkv=ck.kv_heads, step64=ck.step64)
    ocv = oracle.Codec(6, cv.C, seed=cv.seed, hkv=cv.kv_heads, step64=cv.step64)
    qb = synth.bf16_bits(q)
    done_bytes, done_tokens, elapsed, n = 0, 0, 0.0, 0
    per_tok = w.hkv * (ck.C + 2 + cv.C + 2)
    while elapsed < seconds and n < w.batch:
        b = n
        lo, hi = int(starts[b]), int(starts[b]) + int(ctx[b])
        kcs = np.ascontiguousarray(kc[:, lo:hi].cpu().numpy())
        vcs = np.ascontiguousarray(vc[:, lo:hi].cpu().numpy())
        kns = synth.bf16_bits(kn[:, lo:hi])
        vns = synth.bf16_bits(vn[:, lo:hi])
        t0 = time.perf_counter()
        oracle.attention(ock, ocv, qb[b:b + 1], kcs, kns, vcs, vns, np.array([0]),
                         np.array([hi - lo], np.int32), nthreads=threads)
        elapsed += time.perf_counter() - t0
        done_bytes += (hi - lo) * per_tok
        done_tokens += hi - lo
        n += 1
    # oracle encode on one sequence's K vectors
    xk = synth.kv_tensor(w.kind, min(2048, int(ctx[0])), w.hkv, seed=w.seed + 10)
    t0 = time.perf_counter()
    oracle.encode(ock, synth.bf16_bits(xk), nthreads=threads)
    enc_s = time.perf_counter() - t0
    return {"value": done_bytes / elapsed / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 decode attention of {n} of {w.batch} sequences "
                      f"({done_tokens} context tokens x {w.hkv} kv heads, {w.hq} q heads) "
                      f"in {elapsed:.1f} s; encode of {xk.shape[0] * w.hkv} K vectors",
            "context_tokens_per_s": done_tokens / elapsed,
            "encode_vectors_per_s": xk.shape[0] * w.hkv / enc_s}


OTHER_WORKLOADS = ["tiny_1seq_1k", "qwen3_8b_b16_8k", "longctx_b4_64k_c29", "ragged_32seq_4k_128k"]
MALL_FLUSH_BYTES = 512 << 20  # twice the 256 MB MALL: written between timed launches


def oracle_attention_rate(w, ck, cv, kc, kn, vc, vn, q, starts, ctx, seconds):
    """The oracle's fp64 decode attention on a bounded sample of a workload:
    whole sequences in order until ~`seconds` of CPU work (at least one, cut
    to its first 16384 tokens if longer), on the host cores this process may
    use.  Returns (context tokens/s, threads, sample text)."""
    import numpy as np
    import oracle
    import synth
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    ock = oracle.Codec(ck.levels, ck.C, seed=ck.seed, hkv=ck.kv_heads, step64=ck.step64)
    ocv = oracle.Codec(cv.levels, cv.C, seed=cv.seed, hkv=cv.kv_heads, step64=cv.step64)
    qb = synth.bf16_bits(q)
    tokens, elapsed, n = 0, 0.0, 0
    while (elapsed < seconds or n == 0) and n < len(ctx):
        lo = int(starts[n])
        L = min(int(ctx[n]), 16384)
        kcs = np.ascontiguousarray(kc[:, lo:lo + L].cpu().numpy())
        vcs = np.ascontiguousarray(vc[:, lo:lo + L].cpu().numpy())
        kns, vns = synth.bf16_bits(kn[:, lo:lo + L]), synth.bf16_bits(vn[:, lo:lo + L])
        t0 = time.perf_counter()
        oracle.attention(ock, ocv, qb[n:n + 1], kcs, kns, vcs, vns, np.array([0]), np.array([L], np.int32),
                         nthreads=threads)
        elapsed += time.perf_counter() - t0
        tokens += L
        n += 1
    return tokens / elapsed, threads, (f"fp64 decode attention of {n} sequence(s), {tokens} context tokens "
                                       f"x {w.hkv} kv heads, {w.hq} q heads, in {elapsed:.1f} s")


def measure_workload(name, steps, warmup, dev, flush, oracle_seconds, copy_gbps=None):
    """Decode attention (dq_attn_decode) over one workload's prompt, each timed
    launch preceded by a write of a 512 MB buffer so that no part of the
    compressed cache is still in the 256 MB MALL; the split-K kernel is timed
    with HIP events on its stream.  The ragged workload also times its
    8192-token chunk encode per sequence; the tiny one is a latency figure."""
    import numpy as np
    import torch

    import kv_cache_entropy_amd as dq
    import synth
    w = synth.workloads()[name]
    B, Hq, Hkv = w.batch, w.hq, w.hkv
    ctx = np.array(w.ctx, np.int64)
    cap = ctx + w.append_tokens + 1
    starts = np.concatenate([[0], np.cumsum(cap)[:-1]])
    ck = dq.Codec(w.levels_k, w.container_k, seed=w.seed, kv_heads=Hkv)
    cv = dq.Codec(w.levels_v, w.container_v, seed=w.seed + 1, kv_heads=Hkv)
    S = int(cap.sum())
    kc, kn = dq.alloc_pool(ck, S, dev)
    vc, vn = dq.alloc_pool(cv, S, dev)
    T = int(ctx.sum())
    slots = torch.from_numpy(np.concatenate([np.arange(a, a + L) for a, L in zip(starts, ctx)])).to(dev)
    for cont, norm, codec, sd in ((kc, kn, ck, 10), (vc, vn, cv, 11)):
        x = synth.kv_tensor(w.kind, T, Hkv, seed=w.seed + sd, device=dev)
        dq.encode(codec, x, slots, cont, norm)
        del x
    del slots
    q = synth.q_tensor(B, Hq, seed=w.seed + 100, device=dev)
    ss = torch.from_numpy(starts).to(dev)
    sl = torch.from_numpy(ctx.astype(np.int32)).to(dev)
    max_len = int(ctx.max())
    # sized for one more token: the tiny workload also times a step with append
    ws = torch.empty(dq.attn_workspace_bytes(B, Hq, Hkv, max_len + 1), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    alg = T * Hkv * (ck.C + 2 + cv.C + 2)
    def flushed_call():
        flush.zero_()
        dq.attn_decode(ck, cv, q, kc, kn, vc, vn, ss, sl, max_len, out=out, workspace=ws)
    settle_clocks(flushed_call)
    for _ in range(warmup):
        flushed_call()
    torch.cuda.synchronize()
    # back to back (no host wait between launches, so the clocks stay up);
    # the flush before each launch runs on the same stream
    evs = []
    for _ in range(steps):
        flush.zero_()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        dq.attn_decode(ck, cv, q, kc, kn, vc, vn, ss, sl, max_len, out=out, workspace=ws,
                       split_events=(ev[1], ev[2]))
        ev[3].record()
        evs.append(ev)
    torch.cuda.synchronize()
    call = [ev[0].elapsed_time(ev[3]) for ev in evs]
    split = [ev[1].elapsed_time(ev[2]) for ev in evs]
    call_ms, split_ms = float(np.median(call)), float(np.median(split))
    achieved = alg / (split_ms / 1e3) / 1e9
    rec = {"batch": B, "q_heads": Hq, "kv_heads": Hkv, "context": [int(ctx.min()), int(ctx.max())],
           "context_tokens": T, "container_bytes": [ck.C, cv.C], "kv_distribution": w.kind,
           "alg_bytes_per_launch": alg, "attn_call_ms": round(call_ms, 4), "split_ms": round(split_ms, 4),
           "split_ms_p10_p50_p90": pct(split), "call_gbps": round(alg / (call_ms / 1e3) / 1e9, 2),
           "split_gbps": round(achieved, 2), "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4),
           "context_tokens_per_s": round(T / (call_ms / 1e3), 1), "timing": "median of "
           f"{steps} launches, each after a {MALL_FLUSH_BYTES >> 20} MB write that evicts the MALL"}
    if copy_gbps:
        rec["frac_of_copy"] = round(achieved / copy_gbps, 4)
    if name == "tiny_1seq_1k":
        # latency: the decode step with append in one call, no flush needed
        k_new = synth.kv_tensor(w.kind, B, Hkv, seed=w.seed + 20, device=dev)
        v_new = synth.kv_tensor(w.kind, B, Hkv, seed=w.seed + 21, device=dev)
        sl1 = sl + 1
        for _ in range(warmup):
            dq.attn_decode_append(ck, cv, q, k_new, v_new, kc, kn, vc, vn, ss, sl1, max_len + 1, out=out,
                                  workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            dq.attn_decode_append(ck, cv, q, k_new, v_new, kc, kn, vc, vn, ss, sl1, max_len + 1, out=out,
                                  workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        rec["append_step_us"] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
        rec["attn_call_us"] = round(call_ms * 1e3, 2)
    if w.append_tokens:
        # the prefill chunk: append_tokens new tokens per sequence, K and V
        n_app = w.append_tokens
        aslots = torch.from_numpy(np.concatenate([np.arange(a + L, a + L + n_app)
                                                  for a, L in zip(starts, ctx)])).to(dev)
        xk = synth.kv_tensor(w.kind, B * n_app, Hkv, seed=w.seed + 30, device=dev)
        xv = synth.kv_tensor(w.kind, B * n_app, Hkv, seed=w.seed + 31, device=dev)
        dq.encode_kv(ck, cv, xk, xv, aslots, kc, kn, vc, vn)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dq.encode_kv(ck, cv, xk, xv, aslots, kc, kn, vc, vn)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ems = float(np.median(times))
        rec["append_encode"] = {"tokens_per_seq": n_app, "vectors": 2 * B * n_app * Hkv, "ms": round(ems, 3),
                                "vectors_per_s": round(2 * B * n_app * Hkv / (ems / 1e3), 1)}
        del xk, xv, aslots
    if oracle_seconds > 0:
        rate, thr, sample = oracle_attention_rate(w, ck, cv, kc, kn, vc, vn, q, starts, ctx, oracle_seconds)
        rec["cpu_oracle"] = {"context_tokens_per_s": round(rate, 1), "cores": thr, "kind": "oracle",
                             "sample": sample}
    log(f"[bench] {name}: attention {call_ms:.4f} ms per call (split-K {split_ms:.4f} ms = "
        f"{achieved:.1f} GB/s = {achieved / HBM_PEAK_GBPS:.2%} of HBM), "
        f"{rec['context_tokens_per_s'] / 1e9:.3f} G context-tokens/s"
        + (f"; oracle {rec['cpu_oracle']['context_tokens_per_s']:.0f} context-tokens/s" if "cpu_oracle" in rec else "")
        + (f"; chunk encode {rec['append_encode']['vectors_per_s'] / 1e9:.2f} G vectors/s"
           if "append_encode" in rec else "")
        + (f"; append step {rec['append_step_us']} us" if "append_step_us" in rec else ""))
    del kc, kn, vc, vn, ws, out, q
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--workload", default="llama31_8b_b128_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-pool attention timing")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the two-launch and small-batch timings of the decode step")
    ap.add_argument("--no-rd", action="store_true", help="skip the rate-distortion drift-order encode")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill attention timing")
    ap.add_argument("--splitk-waves", type=int, default=None,
                    help="resident waves per CU of the split-K kernel (occupancy study; default: the library's)")
    ap.add_argument("--knob", action="append", default=[], metavar="NAME=VALUE",
                    help="force a library path (dq_set_knob) for a study, e.g. slot_table=0")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the decode-attention timings of the other workloads")
    ap.add_argument("--others-only", metavar="NAME", nargs="*",
                    help="time only these other workloads (all four if none named) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter scale for rocprofv3)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ from the rocprofv3 output of PROFILE_CMDS (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_entropy_amd as dq
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.splitk_waves:
        dq.set_knob("splitk_waves", args.splitk_waves)
    for kv in args.knob:
        name, value = kv.split("=")
        dq.set_knob(name, int(value))
    if args.others_only is not None:
        flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        res = {n: measure_workload(n, args.steps, args.warmup, dev, flush, 0.0)
               for n in (args.others_only or OTHER_WORKLOADS)}
        print(json.dumps({"workloads": res, "attn_source_sha256_16": attn_source_hash()}), flush=True)
        return
    w = synth.workloads()[args.workload]
    B, Hq, Hkv = w.batch, w.hq, w.hkv
    ctx = np.array(w.ctx, np.int64)
    nsteps = args.warmup + args.steps
    cap = ctx + nsteps + w.append_tokens
    starts = np.concatenate([[0], np.cumsum(cap)[:-1]])
    S_total = int(cap.sum())
    ck = dq.Codec(w.levels_k, w.container_k, seed=w.seed, kv_heads=Hkv)
    cv = dq.Codec(w.levels_v, w.container_v, seed=w.seed + 1, kv_heads=Hkv)
    kc, kn = dq.alloc_pool(ck, S_total, dev)
    vc, vn = dq.alloc_pool(cv, S_total, dev)
    log(f"[bench] workload {w.name}: B={B} Hq={Hq} Hkv={Hkv} ctx={int(ctx.min())}..{int(ctx.max())} "
        f"pool {S_total} slots, containers {ck.C}/{cv.C} B")

    # ---- prefill encode (untimed for the step; timed on its own)
    T_pre = int(ctx.sum())
    slots_pre = torch.from_numpy(np.concatenate([np.arange(s, s + L) for s, L in zip(starts, ctx)])).to(dev)
    K = synth.kv_tensor(w.kind, T_pre, Hkv, seed=w.seed + 10, device=dev)
    V = synth.kv_tensor(w.kind, T_pre, Hkv, seed=w.seed + 11, device=dev)
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # untimed repetitions first (they also load the kernels); the same bytes each time
    settle_clocks(lambda: (dq.encode(ck, K, slots_pre, kc, kn), dq.encode(cv, V, slots_pre, vc, vn)))
    stk, stv = dq.new_stats(dev), dq.new_stats(dev)
    torch.cuda.synchronize()
    e_a.record()
    dq.encode(ck, K, slots_pre, kc, kn, stk)
    dq.encode(cv, V, slots_pre, vc, vn, stv)
    e_b.record()
    torch.cuda.synchronize()
    prefill_ms = e_a.elapsed_time(e_b)
    prefill_vps = 2 * T_pre * Hkv / (prefill_ms / 1e3)
    sk, sv = dq.stats_dict(stk), dq.stats_dict(stv)
    drift_k = sk["drifted_symbols"] / (128.0 * sk["vectors"])
    drift_v = sv["drifted_symbols"] / (128.0 * sv["vectors"])
    # algorithmic bytes of the encode: the bf16 vector in, its container and
    # fp16 norm out
    enc_gbps = T_pre * Hkv * (2 * 256 + ck.C + 2 + cv.C + 2) / (prefill_ms / 1e3) / 1e9
    log(f"[bench] prefill encode {2 * T_pre * Hkv} vectors in {prefill_ms:.2f} ms "
        f"({prefill_vps / 1e9:.2f} G vectors/s, {enc_gbps:.0f} GB/s = {enc_gbps / HBM_PEAK_GBPS:.1%} of HBM); "
        f"drift K {drift_k:.3%} V {drift_v:.3%}")

    # the same prompt with the rate-distortion drift order (separate pools)
    rd = None
    if not args.no_rd:
        ck_rd = dq.Codec(w.levels_k, w.container_k, seed=w.seed, kv_heads=Hkv, drift_order=1)
        cv_rd = dq.Codec(w.levels_v, w.container_v, seed=w.seed + 1, kv_heads=Hkv, drift_order=1)
        rk_c, rk_n = dq.alloc_pool(ck_rd, S_total, dev)
        rv_c, rv_n = dq.alloc_pool(cv_rd, S_total, dev)
        srk, srv = dq.new_stats(dev), dq.new_stats(dev)
        torch.cuda.synchronize()
        e_a.record()
        dq.encode(ck_rd, K, slots_pre, rk_c, rk_n, srk)
        dq.encode(cv_rd, V, slots_pre, rv_c, rv_n, srv)
        e_b.record()
        torch.cuda.synchronize()
        rd_ms = e_a.elapsed_time(e_b)
        a_k, a_v = dq.stats_dict(srk), dq.stats_dict(srv)
        rd = {"encode_vectors_per_s": round(2 * T_pre * Hkv / (rd_ms / 1e3), 1),
              "drift_rate": {"k": round(a_k["drifted_symbols"] / (128.0 * a_k["vectors"]), 5),
                             "v": round(a_v["drifted_symbols"] / (128.0 * a_v["vectors"]), 5)},
              "kernel": "encode_fast_kernel + encode_rest_kernel"}
        log(f"[bench] rate-distortion drift order: prefill encode {rd_ms:.1f} ms "
            f"({rd['encode_vectors_per_s'] / 1e9:.3f} G vectors/s); drift K {rd['drift_rate']['k']:.3%} "
            f"V {rd['drift_rate']['v']:.3%}")
        del rk_c, rk_n, rv_c, rv_n
    del K, V

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()
        del a, b2

    # ---- decode steps: inputs drawn up front
    Kn = synth.kv_tensor(w.kind, nsteps * B, Hkv, seed=w.seed + 20, device=dev).view(nsteps, B, Hkv, 128)
    Vn = synth.kv_tensor(w.kind, nsteps * B, Hkv, seed=w.seed + 21, device=dev).view(nsteps, B, Hkv, 128)
    qs = [synth.q_tensor(B, Hq, seed=w.seed + 100 + s, device=dev) for s in range(nsteps)]
    st_t = torch.from_numpy(starts).to(dev)
    slots_s = [(st_t + torch.from_numpy(ctx).to(dev) + s).contiguous() for s in range(nsteps)]
    lens_s = [torch.from_numpy(ctx + s + 1).to(torch.int32).to(dev) for s in range(nsteps)]
    max_len = int(ctx.max()) + nsteps
    ws = torch.empty(dq.attn_workspace_bytes(B, Hq, Hkv, max_len), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    per_tok = Hkv * (ck.C + 2 + cv.C + 2)
    bytes_s = [int((ctx + s + 1).sum()) * per_tok for s in range(nsteps)]

    nq = 3 if max(ck.C, cv.C) <= 47 else (5 if max(ck.C, cv.C) <= 79 else 9)  # the kernel's tile pieces

    def step(s, ev=None):
        # one decode step, one call: the new token's K/V encoded into the
        # pools and attention over the grown contexts (dq_attn_decode_append)
        if ev is not None:
            ev[0].record()
        dq.attn_decode_append(ck, cv, qs[s], Kn[s], Vn[s], kc, kn, vc, vn, st_t, lens_s[s], max_len, out=out,
                              workspace=ws, split_events=None if ev is None else (ev[1], ev[2]))
        if ev is not None:
            ev[3].record()

    # clocks first (untimed repetitions of the first step: the same token
    # re-encoded into the same slots), then the warm-up steps
    settle_clocks(lambda: step(0))
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    # the timed steps: one event pair around all of them, nothing recorded
    # in between (an event between two kernels is a gap of its own)
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_a.record()
    for k in range(args.steps):
        step(args.warmup + k)
    ev_b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_s = max(wall, ev_a.elapsed_time(ev_b) / 1e3)
    # the same steps again (re-encoding a step's tokens into the same slots
    # writes the same bytes), now with events per step: [step start, split-K
    # start, split-K done, step done], for the kernel's own time; all on the
    # current stream, which is the one every library launch goes to
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(args.warmup + k, evs[k])
    torch.cuda.synchronize()
    att_ms = [evs[k][0].elapsed_time(evs[k][3]) for k in range(args.steps)]
    timed_bytes = sum(bytes_s[args.warmup:])
    ms_per_step = total_s * 1e3 / args.steps
    value = timed_bytes / total_s / 1e9
    split_ms = [evs[k][1].elapsed_time(evs[k][2]) for k in range(args.steps)]
    att_avg_ms = sum(att_ms) / len(att_ms)
    split_avg_ms = sum(split_ms) / len(split_ms)
    alg_bytes = timed_bytes / args.steps
    achieved = alg_bytes / (split_avg_ms / 1e3) / 1e9
    ctx_tokens = sum(int((ctx + args.warmup + k + 1).sum()) for k in range(args.steps))
    # a plain device copy on this GPU: what HBM sustains for a read + write
    # stream, for the kernel's fraction of it
    cpy_a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cpy_b = torch.empty_like(cpy_a)
    cpy_b.copy_(cpy_a)
    torch.cuda.synchronize()
    e_a.record()
    for _ in range(5):
        cpy_b.copy_(cpy_a)
    e_b.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * (1 << 30) / (e_a.elapsed_time(e_b) / 1e3) / 1e9
    del cpy_a, cpy_b
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (one dq_attn_decode_append call; split-K "
        f"kernel {split_avg_ms:.3f} ms), {value:.1f} GB/s step, split-K kernel "
        f"{achieved:.1f} GB/s = {achieved / HBM_PEAK_GBPS:.1%} of HBM peak, {achieved / copy_gbps:.1%} of a "
        f"device copy's {copy_gbps:.0f} GB/s")

    # the same steps as two launches (dq_encode_kv, then dq_attn_decode);
    # re-encoding the same tokens into the same slots writes the same bytes.
    # Then both forms at small batch (the first sequences), eagerly and as
    # HIP-graph replays.
    two = small = None
    if not args.no_compare:
        tev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]

        def step2(s, ev=None):
            if ev is not None:
                ev[0].record()
            dq.encode_kv(ck, cv, Kn[s], Vn[s], slots_s[s], kc, kn, vc, vn)
            if ev is not None:
                ev[1].record()
            dq.attn_decode(ck, cv, qs[s], kc, kn, vc, vn, st_t, lens_s[s], max_len, out=out, workspace=ws,
                           split_events=None if ev is None else (ev[3], ev[4]))
            if ev is not None:
                ev[2].record()
        for s in range(args.warmup):
            step2(s)
        torch.cuda.synchronize()
        for k in range(args.steps):
            step2(args.warmup + k, tev[k])
        torch.cuda.synchronize()
        t_step = tev[0][0].elapsed_time(tev[-1][2]) / args.steps
        t_enc = float(np.mean([e[0].elapsed_time(e[1]) for e in tev]))
        t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in tev]))
        t_split = float(np.mean([e[3].elapsed_time(e[4]) for e in tev]))
        two = {"ms_per_step": round(t_step, 4), "gbps": round(alg_bytes / (t_step / 1e3) / 1e9, 2),
               "append_encode_ms": round(t_enc, 4), "attn_call_ms": round(t_att, 4),
               "split_ms": round(t_split, 4), "split_gbps": round(alg_bytes / (t_split / 1e3) / 1e9, 2),
               "kernel": f"attn_splitk_kernel<{nq}, false>"}
        log(f"[bench] as dq_encode_kv then dq_attn_decode: {t_step:.3f} ms/step (append encode {t_enc:.3f} ms, attention {t_att:.3f} "
            f"ms of which split-K {t_split:.3f} ms = {two['split_gbps']:.1f} GB/s)")

        def small_ms(nb, fused_call, graph=False):
            qb = [qs[s][:nb].contiguous() for s in range(nsteps)]
            kb = [Kn[s][:nb] for s in range(nsteps)]
            vb = [Vn[s][:nb] for s in range(nsteps)]
            lb = [lens_s[s][:nb].contiguous() for s in range(nsteps)]
            sb = [slots_s[s][:nb].contiguous() for s in range(nsteps)]
            stb = st_t[:nb].contiguous()
            mlb = int(ctx[:nb].max()) + nsteps
            wsb = torch.empty(dq.attn_workspace_bytes(nb, Hq, Hkv, mlb), dtype=torch.uint8, device=dev)
            ob = torch.empty((nb, Hq, 128), dtype=torch.float32, device=dev)

            def one(s):
                if fused_call:
                    dq.attn_decode_append(ck, cv, qb[s], kb[s], vb[s], kc, kn, vc, vn, stb, lb[s], mlb, out=ob,
                                          workspace=wsb)
                else:
                    dq.encode_kv(ck, cv, kb[s], vb[s], sb[s], kc, kn, vc, vn)
                    dq.attn_decode(ck, cv, qb[s], kc, kn, vc, vn, stb, lb[s], mlb, out=ob, workspace=wsb)
            for s in range(args.warmup):
                one(s)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if graph:
                # one step captured once (HIP graph) and replayed: the launches
                # cost no host time; the step re-encodes the same token
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    one(args.warmup)
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    one(args.warmup)
                g.replay()
                torch.cuda.synchronize()
                e0.record()
                for k in range(args.steps):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / args.steps
            e0.record()
            for k in range(args.steps):
                one(args.warmup + k)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        small = {}
        for nb in (1, 4):
            small[str(nb)] = {"append_call_ms": round(small_ms(nb, True), 4),
                              "encode_then_attn_ms": round(small_ms(nb, False), 4),
                              "append_call_graph_ms": round(small_ms(nb, True, graph=True), 4),
                              "encode_then_attn_graph_ms": round(small_ms(nb, False, graph=True), 4)}
        log(f"[bench] batch 1: {small['1']['append_call_ms']:.4f} ms per step as one dq_attn_decode_append call vs "
            f"{small['1']['encode_then_attn_ms']:.4f} as encode then attention (graph replay {small['1']['append_call_graph_ms']:.4f} vs "
            f"{small['1']['encode_then_attn_graph_ms']:.4f}); batch 4: {small['4']['append_call_ms']:.4f} vs "
            f"{small['4']['encode_then_attn_ms']:.4f} (graph replay {small['4']['append_call_graph_ms']:.4f} vs "
            f"{small['4']['encode_then_attn_graph_ms']:.4f})")

    # the same caches re-laid as shuffled 64-token pages (page-table pool)
    paged = None
    if not args.no_paged:
        P = dq.PAGE_TOKENS
        npg = int((cap.max() + P - 1) // P)
        gen = torch.Generator(device="cpu").manual_seed(w.seed + 50)
        phys = torch.randperm(B * npg, generator=gen).to(dev).view(B, npg)
        src = torch.from_numpy(starts).to(dev)[:, None] + torch.arange(npg, device=dev)[None, :] * P
        pools = []
        for cont, norm in ((kc, kn), (vc, vn)):
            cont2 = torch.zeros((Hkv, dq.pool_slots(B * npg * P), cont.shape[2]), dtype=torch.uint8, device=dev)
            norm2 = torch.zeros((Hkv, cont2.shape[1]), dtype=torch.float16, device=dev)
            for j in range(P):
                s_idx = (src + j).clamp(max=cont.shape[1] - 1).flatten()
                d_idx = (phys * P + j).flatten()
                cont2[:, d_idx] = cont[:, s_idx]
                norm2[:, d_idx] = norm[:, s_idx]
            pools += [cont2, norm2]
        pages = phys.to(torch.int32).contiguous()
        outp = torch.empty_like(out)
        for s in range(args.warmup):
            dq.attn_decode_paged(ck, cv, qs[s], *pools, pages, lens_s[s], max_len, out=outp, workspace=ws)
        torch.cuda.synchronize()
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for k in range(args.steps):
            s = args.warmup + k
            pev[k][0].record()
            dq.attn_decode_paged(ck, cv, qs[s], *pools, pages, lens_s[s], max_len, out=outp, workspace=ws)
            pev[k][1].record()
        torch.cuda.synchronize()
        paged_ms = sum(e[0].elapsed_time(e[1]) for e in pev) / args.steps
        paged = {"attn_call_ms": round(paged_ms, 4), "gbps": round(alg_bytes / (paged_ms / 1e3) / 1e9, 2),
                 "page_tokens": P, "layout": "pages shuffled over the pool"}
        contig = f"vs contiguous {two['attn_call_ms']:.3f} ms" if two else ""
        log(f"[bench] paged pool: attention call {paged_ms:.3f} ms ({paged['gbps']:.1f} GB/s) {contig}")
        del pools

    # chunked prefill over the same caches: the first 16 sequences, their
    # last 512 cached tokens taken as the chunk (8K-token prompts)
    prefill = None
    if not args.no_prefill:
        nb, tq = min(16, B), 512
        lens_p = lens_s[-1][:nb].contiguous()
        qp = synth.kv_tensor("iid", nb * tq, Hq, seed=w.seed + 60, device=dev).view(nb, tq, Hq, 128).contiguous()
        max_p = int(lens_p.max())
        wsp = torch.empty(dq.attn_prefill_workspace_bytes(nb, tq, Hq, Hkv, max_p), dtype=torch.uint8, device=dev)
        outp = torch.empty((nb, tq, Hq, 128), dtype=torch.float32, device=dev)
        ss_p = st_t[:nb].contiguous()
        settle_clocks(lambda: dq.attn_prefill(ck, cv, qp, kc, kn, vc, vn, ss_p, lens_p, max_p, out=outp,
                                              workspace=wsp))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        reps = 3
        for _ in range(reps):
            dq.attn_prefill(ck, cv, qp, kc, kn, vc, vn, ss_p, lens_p, max_p, out=outp, workspace=wsp)
        e1.record()
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / reps
        group = Hq // Hkv
        # compressed bytes the kernel reads: each item of query blocks reads its
        # causal prefix once (8 blocks of 16 rows per item for containers of up
        # to 35 bytes, one block otherwise)
        tb = (16 // group) * (8 if max(ck.C, cv.C) <= 35 else 1)
        lens_np = lens_p.cpu().numpy().astype(np.int64)
        read = 0
        for L in lens_np:
            for qb in range((tq + tb - 1) // tb):
                read += (L - tq + min(tq, (qb + 1) * tb)) * Hkv * (ck.C + 2 + cv.C + 2)
        # the method's flops, counted once: every query row against its
        # causal prefix, QK and PV, 2 flops per multiply-add, all Hq heads
        flops = 0
        for L in lens_np:
            vis = np.arange(L - tq + 1, L + 1, dtype=np.int64)  # keys each query row sees
            flops += int(vis.sum()) * Hq * 128 * 2 * 2
        syms = read // (ck.C + 2 + cv.C + 2) * 256  # K and V symbols the kernel decodes
        tflops = flops / (pms / 1e3) / 1e12
        prefill = {"batch": nb, "chunk_tokens": tq, "context": int(lens_np.max()), "call_ms": round(pms, 3),
                   "query_tokens_per_s": round(nb * tq / (pms / 1e3), 1),
                   "kv_bytes_read_gbps": round(read / (pms / 1e3) / 1e9, 1), "rows_per_item": tb * group,
                   "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0,
                                "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                                "flops_per_call": flops, "dtype": "fp16 (hi/lo pairs: 2 MFMAs per product)",
                                "kernel": "attn_prefill_shared_kernel" if max(ck.C, cv.C) <= 35
                                else "attn_prefill_kernel"},
                   "decoded_symbols_per_s": round(syms / (pms / 1e3), 1)}
        log(f"[bench] chunked prefill: {nb} x {tq} queries over {prefill['context']} tokens in {pms:.2f} ms "
            f"({prefill['query_tokens_per_s'] / 1e3:.1f} K query tokens/s, {prefill['kv_bytes_read_gbps']} GB/s read, "
            f"{tflops:.1f} TFLOP/s = {tflops / 2500.0:.2%} of fp16 MFMA peak, "
            f"{syms / (pms / 1e3) / 1e9:.1f} G symbols/s decoded)")
        del qp, wsp, outp

    # the other workloads: decode attention over each prompt, the MALL
    # evicted before every timed launch, with the oracle on a bounded sample
    others = None
    if not args.no_others:
        del ws
        torch.cuda.empty_cache()
        flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        others = {n: measure_workload(n, max(args.steps, 10), 3, dev, flush,
                                      0.0 if args.no_cpu_baseline else 2.0, copy_gbps)
                  for n in OTHER_WORKLOADS}
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores")
        cpu = cpu_baseline(w, ck, cv, kc, kn, vc, vn, qs[0], starts, ctx, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']:.4f} GB/s on {cpu['cores']} threads")

    rec = {
        "metric": "dq_attn_decode compressed-KV GB/s (decode step incl. append encode)",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_ms": SETTLE_MS,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": 128,
                   "context": [int(ctx.min()), int(ctx.max())], "container_bytes": [ck.C, cv.C],
                   "levels": [ck.levels, cv.levels], "kv_distribution": w.kind},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(alg_bytes), "kernel": "attn_splitk_kernel",
                     "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": round(split_avg_ms, 4),
                     "launch_ms_p10_p50_p90": pct(split_ms), "copy_gbps": round(copy_gbps, 1),
                     "frac_of_copy": round(achieved / copy_gbps, 4)},
        "step_ms_p10_p50_p90": pct(att_ms),
        "attn_source_sha256_16": attn_source_hash(),
        "step_call": "dq_attn_decode_append",
        "step_call_ms": round(att_avg_ms, 4),
        "encode_then_attn_step": two,
        "small_batch_step": small,
        "paged_attn": paged,
        "rd_drift_order": rd,
        "prefill_attn": prefill,
        "workloads": others,
        "cpu_baseline": cpu,
        "attn_context_tokens_per_s": round(ctx_tokens / (sum(att_ms) / 1e3), 1),
        "prefill_encode_vectors_per_s": round(prefill_vps, 1),
        "prefill_encode_roofline": {"bound": "valu", "alg_gbps": round(enc_gbps, 1),
                                    "hbm_frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
                                    "alg_bytes_per_vector": [256 + ck.C + 2, 256 + cv.C + 2]},
        "drift_rate": {"k": round(drift_k, 5), "v": round(drift_v, 5)},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
