"""Summaries of rocprofv3 output for the committed profiles.

Usage (from the repository root, after the profiling runs):

  python bench_tools.py stats <rocprof-dir> <out.md> --cmd "<command>" --title "<title>"
      kernel table (calls, average / min / max duration, share of GPU time) from
      <rocprof-dir>/run_kernel_trace.csv (rocprofv3 --kernel-trace --stats --output-format csv -o run);
      --split-at <kernel> makes one table of the dispatches before that kernel's first one and one
      of the rest

  python bench_tools.py traffic --fetch <dir> --write <dir> --workload <name> \\
      --out <traffic.json> [--md <out.md>] [--cmd-fetch "<command>"] [--cmd-write "<command>"]
      HBM traffic of one moe_expert_mlp call from two counter runs of ``bench.py --copy-calibration``:
      rocprofv3 --pmc TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum (reads, summed
      by request size), then --pmc WRITE_SIZE (writes); --output-format csv -o run.  The copy of a known
      number of bytes is reported as the check of both.

  python bench_tools.py reqsize <rocprof-dir> <out.md> --cmd "<command>"
      read requests by size per kernel (the same three counters and TCC_BUBBLE_sum), and what
      FETCH_SIZE's expression counts from them.

  python bench_tools.py waves --dirs <d1> <d2> <d3> --kernels <k...> --cmds "<c1>" "<c2>" "<c3>" \\
      --out <out.md> --title "<title>"
      wave-state, LDS and L2 counters of the named kernels from the three WAVE_PASSES runs.

  python bench_tools.py library <out.md> --cmd "<command>"
      (on a GPU) times the vendor library (torch.matmul, hipBLASLt) on dense bf16 GEMMs of the
      grouped GEMMs' shapes, for context.

  python bench_tools.py mfma --pmc <dir> --stats <dir> --out <out.md> --cmd-pmc "<command>" \
      --cmd-stats "<command>" --title "<title>"
      MFMA utilisation per kernel from one counter run (rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
      SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 GRBM_GUI_ACTIVE) and the kernel
      durations of a trace run of the same command: busy share of the MFMA units, MFMA FLOP per
      dispatch (MOPS x 512), the rate they give over the traced duration, and the clock the
      active-cycle counter implies.

The traffic record carries a hash of the sources of the workload's expert-MLP
kernels; bench.py reports it only while those are unchanged.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.join(ROOT, "grouped_gemm_router_amd")
COPY_BYTES = 1 << 30                    # bytes moved by bench.py --copy-calibration per copy
COPY_KERNEL = "copyBuffer"              # the HIP runtime's device-to-device copy kernel
MLP_KERNELS = {                         # kernels of one moe_expert_mlp call, per workload kind
    "bf16": ("k_fwd_gateup", "k_fwd_down"),
    "decode": ("k_decode_gateup", "k_decode_down"),
    "mxfp8": ("k_mx_quantize", "k_mx_gateup", "k_mx_down"),
}


# library sources the kernels of one moe_expert_mlp call are built from, per workload kind
# (the host code and shared headers for all; the backward and routing sources for none)
_COMMON_SOURCES = ("api.cpp", "common.h", "kernels.h", "grouped_gemm.h")
MLP_SOURCES = {
    "bf16": _COMMON_SOURCES + ("gemm_rows.h", "gemm_bf16.hip"),
    "decode": _COMMON_SOURCES + ("gemm_rows.h", "decode.hip"),
    "mxfp8": _COMMON_SOURCES + ("gemm_rows.h", "mx_gemm.hip", "elementwise.hip"),
}


def source_hash(workload: str) -> str:
    """sha256 over the sources of the workload's moe_expert_mlp kernels (and the header)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    files = [os.path.join(ROOT, "include", "moe.h")]
    files += [os.path.join(csrc, f) for f in sorted(MLP_SOURCES[_kind(workload)])]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _short(name: str) -> str:
    return name.split("(")[0].replace("moe::", "")


def _trace_table(rows: list) -> list:
    """markdown rows (calls, avg / min / max duration, share of the section's GPU time) per kernel
    of kernel-trace rows, longest total first."""
    dur = collections.defaultdict(list)
    for r in rows:
        dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in dur.values()) or 1.0
    lines = ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for name, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        n = name.replace("|", "/")
        if len(n) > 90:
            n = n[:87] + "..."
        lines.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} "
                     f"| {100 * sum(v) / total:.2f} |")
    return lines


def stats_md(src: str, out: str, cmd: str, title: str, note: str = "", split_at: str = "") -> None:
    """Kernel table of one trace run.  With split_at (part of a kernel's name), the dispatches that
    start before that kernel's first dispatch and the rest get a table each (bench.py's default
    run measures its own workload first and then the other configurations)."""
    trace = list(csv.DictReader(open(os.path.join(src, "run_kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    agent = list(csv.DictReader(open(os.path.join(src, "run_agent_info.csv"))))
    gpus = [a for a in agent if a.get("Agent_Type", "").upper() == "GPU"]
    dev = gpus[0].get("Name", "?") if gpus else "?"
    lines = [f"# {title}", "", "Command (repository root, one MI355X):", "", "```", cmd, "```", "",
             f"Device: {dev}.  Per-kernel durations from the kernel trace (`run_kernel_trace.csv`).", ""]
    if note:
        lines += [note, ""]
    if split_at:
        first = next((i for i, r in enumerate(trace) if split_at in r["Kernel_Name"]), len(trace))
        lines += [f"Dispatches before the first `{split_at}`:", ""] + _trace_table(trace[:first])
        if first < len(trace):
            lines += ["", f"From the first `{split_at}` on:", ""] + _trace_table(trace[first:])
    else:
        lines += _trace_table(trace)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def _per_dispatch(src: str, counter: str) -> dict:
    """kernel short name -> list of (dispatch id, counter value summed over instances / XCDs)."""
    acc = collections.defaultdict(float)
    name_of = {}
    for r in csv.DictReader(open(os.path.join(src, "run_counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        acc[d] += float(r["Counter_Value"])
        name_of[d] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for d in sorted(acc):
        out[_short(name_of[d])].append((d, acc[d]))
    return out


def _kind(workload: str) -> str:
    if workload.startswith("decode") or workload == "tiny":
        return "decode"
    if "mxfp8" in workload:
        return "mxfp8"
    return "bf16"


# Read traffic: the TCC->EA read requests counted by size.  On gfx950 almost every read request
# is 128 bytes and TCC_BUBBLE (which FETCH_SIZE's expression takes as the 128-byte count) reads 0,
# so FETCH_SIZE counts them as 64 bytes, half the bytes; the sizes summed give the bytes directly.
READ_COUNTERS = ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")
READ_BYTES = (32, 64, 128)


def read_bytes(src: str) -> dict:
    """kernel short name -> list of (dispatch id, bytes read from memory) of a run with READ_COUNTERS."""
    per = [_per_dispatch(src, c) for c in READ_COUNTERS]
    out = collections.defaultdict(list)
    for name, vals in per[-1].items():
        for i, (d, _) in enumerate(vals):
            out[name].append((d, sum(b * dict(p.get(name, [])).get(d, 0.0) for p, b in zip(per, READ_BYTES))))
    return out


def write_bytes(src: str) -> dict:
    """kernel short name -> list of (dispatch id, bytes written) of a run with WRITE_SIZE (KiB)."""
    return {k: [(d, v * 1024.0) for d, v in vals] for k, vals in _per_dispatch(src, "WRITE_SIZE").items()}


def traffic(fetch_dir: str, write_dir: str, workload: str) -> dict:
    """Bytes read (request sizes) and written (WRITE_SIZE) by one moe_expert_mlp call; the copy of
    COPY_BYTES bytes (bench.py --copy-calibration) is reported as the check of both counters."""
    res = {"workload": workload, "source_sha": source_hash(workload), "copy_bytes": COPY_BYTES}
    for what, per in (("read", read_bytes(fetch_dir)), ("write", write_bytes(write_dir))):
        copy = sorted(v for k, vals in per.items() if COPY_KERNEL in k for _, v in vals)
        if not copy:
            raise SystemExit(f"no {COPY_KERNEL} dispatch: run bench.py with --copy-calibration")
        kernels = MLP_KERNELS[_kind(workload)]
        main = [k for k in kernels if k != "k_mx_quantize"][0]      # one dispatch per call
        calls = per.get(main, [])
        if not calls:
            raise SystemExit(f"no {main} dispatch")
        first = calls[0][0]
        call = 0.0
        detail = {}
        for k in kernels:
            # per-call dispatches only (weight quantisation at load time comes before the first call;
            # a call's input quantisation is the dispatch just before its first GEMM)
            vals = [v for d, v in per.get(k, []) if d >= first - 1]
            if not vals:
                continue
            b = sum(vals) / len(calls)
            detail[k] = round(b)
            call += b
        res[what] = {"copy_bytes_counted": round(copy[len(copy) // 2]), "calls": len(calls),
                     "per_kernel_bytes": detail, "call_bytes": round(call)}
    res["traffic_bytes"] = res["read"]["call_bytes"] + res["write"]["call_bytes"]
    return res


def traffic_md(t: dict, out: str, cmd_fetch: str, cmd_write: str) -> None:
    lines = [f"# HBM traffic of one moe_expert_mlp call, workload {t['workload']}", "",
             "Commands (repository root, one MI355X; reads and writes in separate counter runs):", "", "```",
             cmd_fetch, cmd_write, "```", "",
             "Reads are the TCC->EA read requests summed by size (32, 64 and 128 bytes); writes are WRITE_SIZE. "
             f"Check: the device-to-device copy of {t['copy_bytes']} bytes (`--copy-calibration`) counts as the "
             "bytes in the table (no scale factor is applied).", "",
             "| direction | copy counted (bytes) | per kernel (bytes per launch) | per call (bytes) |",
             "|---|---:|---|---:|"]
    for c in ("read", "write"):
        d = t[c]
        per = ", ".join(f"{k}: {v / 1e6:.1f} MB" for k, v in d["per_kernel_bytes"].items())
        lines.append(f"| {c} | {d['copy_bytes_counted']} | {per} | {d['call_bytes'] / 1e6:.1f} MB |")
    lines += ["", f"Total per call: {t['traffic_bytes'] / 1e6:.1f} MB.  Expert-MLP source sha256: `{t['source_sha']}`."]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def reqsize_md(src: str, out: str, cmd: str) -> None:
    """Per kernel: read requests by size, the bytes they give, and what FETCH_SIZE's expression would
    count from the same requests (TCC_BUBBLE added)."""
    per = {c: _per_dispatch(src, c) for c in READ_COUNTERS + ("TCC_BUBBLE_sum",)}
    med = lambda vals: sorted(v for _, v in vals)[len(vals) // 2] if vals else 0.0
    lines = ["# Read request sizes of the prefill workload's kernels (the FETCH_SIZE factor of 2)", "",
             "Command (repository root, one MI355X):", "", "```", cmd, "```", "",
             "Median per dispatch.  Bytes = 32 x 32B + 64 x 64B + 128 x 128B requests.  FETCH_SIZE's "
             "expression, (TCC_BUBBLE x 128 + (RDREQ - TCC_BUBBLE - RDREQ_32B) x 64 + RDREQ_32B x 32) / 1024 KiB, "
             "takes TCC_BUBBLE as the 128-byte count; on this part TCC_BUBBLE reads 0 where 128-byte requests are "
             "issued, so FETCH_SIZE counts them as 64 bytes.", "",
             "| kernel | 32B | 64B | 128B | TCC_BUBBLE | bytes (sizes) | FETCH_SIZE x 1024 |", "|---|---:|---:|---:|---:|---:|---:|"]
    for name in sorted(per[READ_COUNTERS[-1]]):
        n = [med(per[c].get(name, [])) for c in READ_COUNTERS]
        bub = med(per["TCC_BUBBLE_sum"].get(name, []))
        b = sum(x * y for x, y in zip(n, READ_BYTES))
        fetch = bub * 128 + (sum(n) - bub - n[0]) * 64 + n[0] * 32
        lines.append(f"| `{name[:48]}` | {n[0]:.0f} | {n[1]:.0f} | {n[2]:.0f} | {bub:.0f} | {b / 1e6:.1f} MB | "
                     f"{fetch / 1e6:.1f} MB |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


SIMD_NUM = 256 * 4                      # MI355X: 256 compute units x 4 SIMDs
NUM_XCD = 8
PEAK_TFLOPS = {"BF16": 2516.6, "F8": 5033.2}


def _per_dispatch_multi(src: str):
    """dispatch id -> (kernel short name, {counter: value}).  rocprofv3's csv holds one row per
    dispatch and counter, summed over all instances: GRBM_GUI_ACTIVE is then the active cycles of
    the 8 XCDs added up, so the per-XCD count (what the MfmaUtil metric's max-reduction takes) is
    that value / 8."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(os.path.join(src, "run_counter_collection.csv"))):
        d = int(r["Dispatch_Id"])
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        names[d] = _short(r["Kernel_Name"])
        vals[d][c] += v
    for v in vals.values():
        if "GRBM_GUI_ACTIVE" in v:
            v["GRBM_GUI_ACTIVE"] /= NUM_XCD
    return {d: (names[d], vals[d]) for d in vals}


def mfma_md(pmc_dir: str, stats_dir: str, out: str, cmd_pmc: str, cmd_stats: str, title: str) -> None:
    per = _per_dispatch_multi(pmc_dir)
    dur = {_short(r["Name"]): float(r["AverageNs"]) for r in
           csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv")))}
    agg = collections.defaultdict(lambda: collections.defaultdict(float))
    cnt = collections.Counter()
    for name, v in per.values():
        mops = v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + v.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        if mops <= 0:
            continue
        cnt[name] += 1
        for c, x in v.items():
            agg[name][c] += x
    lines = [f"# {title}", "", "Commands (repository root, one MI355X):", "", "```", cmd_pmc, cmd_stats, "```", "",
             "Per kernel, averaged over its dispatches:", "",
             "- MFMA busy = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (active cycles per XCD x 1024 SIMDs), the "
             "utilisation rocprofv3's MfmaUtil metric defines (active cycles per XCD = GRBM_GUI_ACTIVE summed "
             "over the 8 XCDs / 8);",
             "- MFMA FLOP = SQ_INSTS_VALU_MFMA_MOPS_{BF16,F8} x 512 per dispatch, over the kernel's average traced "
             "duration (second command) = the counted MFMA rate, as a share of the dtype's dense peak;",
             "- clock = active cycles per XCD / traced duration;",
             "- % of clock peak = the counted rate against the dense peak scaled to that clock (nominal 2.4 GHz).", "",
             "| kernel | dispatches | MFMA busy | MFMA GFLOP per dispatch | avg us (trace) | counted TFLOP/s | "
             "% of peak | clock GHz | % of clock peak |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for name in sorted(agg, key=lambda n: -agg[n]["SQ_VALU_MFMA_BUSY_CYCLES"]):
        n = cnt[name]
        a = {c: x / n for c, x in agg[name].items()}
        gui = a.get("GRBM_GUI_ACTIVE", 0.0)
        busy = 100.0 * a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * SIMD_NUM) if gui else float("nan")
        bf, f8 = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0), a.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0)
        flop = (bf + f8) * 512
        dtype = "F8" if f8 > bf else "BF16"
        ns = dur.get(name)
        rate = flop / ns / 1e3 if ns else float("nan")          # FLOP/ns = GFLOP/s -> TFLOP/s
        clock = gui / ns if ns else float("nan")
        lines.append(f"| `{name}` | {n} | {busy:.1f}% | {flop / 1e9:.2f} | {ns / 1e3 if ns else float('nan'):.1f} "
                     f"| {rate:.0f} | {100 * rate / PEAK_TFLOPS[dtype]:.1f}% ({dtype}) | {clock:.2f} "
                     f"| {100 * rate / (PEAK_TFLOPS[dtype] * clock / 2.4):.1f}% |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# Dense bf16 GEMMs of the same shapes as the grouped GEMMs, run by the vendor library (torch.matmul
# on ROCm: hipBLASLt), for context: (label, batch, M, N, K).  A batch of equal experts stands in
# for the grouped GEMM (the prefill workload's routing puts 4096 rows on each of 8 experts).
LIBRARY_SHAPES = (
    ("prefill gate/up: 8 experts x [4096 x 2048] x [2048 x 1024]", 8, 4096, 1024, 2048),
    ("prefill down: 8 experts x [4096 x 512] x [512 x 2048]", 8, 4096, 2048, 512),
    ("prefill gate/up rows as one GEMM: [32768 x 2048] x [2048 x 1024]", 1, 32768, 1024, 2048),
    ("training gate/up: 128 experts x [512 x 4096] x [4096 x 2048]", 128, 512, 2048, 4096),
    ("square 8192", 1, 8192, 8192, 8192),
)


def library_md(out: str, cmd: str, iters: int = 50) -> None:
    """Times torch.matmul (hipBLASLt) on LIBRARY_SHAPES with device events; writes a table."""
    import torch
    torch.manual_seed(0)
    dev = torch.device("cuda")
    lines = ["# The vendor GEMM library on the grouped GEMMs' shapes (bf16, one MI355X)", "",
             "Command (repository root):", "", "```", cmd, "```", "",
             f"torch.matmul on bf16 operands (hipBLASLt), fp32 accumulation, {iters} back-to-back calls timed with "
             "device events after 5 warm-up calls; contiguous operands.  % of peak against the dense bf16 peak "
             f"{PEAK_TFLOPS['BF16']} TFLOP/s.", "",
             "| shape | us per call | TFLOP/s | % of bf16 peak |", "|---|---:|---:|---:|"]
    for label, b, m, n, k in LIBRARY_SHAPES:
        a = torch.randn(b, m, k, device=dev, dtype=torch.bfloat16)
        w = torch.randn(b, k, n, device=dev, dtype=torch.bfloat16).contiguous()
        for _ in range(5):
            torch.matmul(a, w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            torch.matmul(a, w)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        tf = 2.0 * b * m * n * k / ms / 1e9
        lines.append(f"| {label} | {ms * 1e3:.1f} | {tf:.0f} | {100 * tf / PEAK_TFLOPS['BF16']:.1f}% |")
        print(lines[-1], flush=True)
        del a, w
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


# Wave-state and LDS counters (two rocprofv3 passes of eight SQ counters each; a third pass with
# the L2 hit and miss counts).  SQ_WAVE_CYCLES and the SQ_WAIT_* / SQ_ACTIVE_* counters count in
# the same unit, so their ratios compare like with like.
WAVE_PASSES = (
    ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_VALU"),
    ("SQ_BUSY_CYCLES", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
     "SQ_INST_CYCLES_VMEM_RD", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_MISC", "GRBM_GUI_ACTIVE"),
    ("TCC_HIT_sum", "TCC_MISS_sum"),
)


def waves_md(dirs: list, kernels: list, out: str, cmds: list, title: str) -> None:
    """Per-dispatch means of the WAVE_PASSES counters for the named kernels (short names)."""
    vals = collections.defaultdict(dict)
    for d in dirs:
        per = _per_dispatch_multi(d)
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        cnt = collections.Counter()
        for name, v in per.values():
            if name not in kernels:
                continue
            cnt[name] += 1
            for c, x in v.items():
                acc[name][c] += x
        for name in acc:
            for c, x in acc[name].items():
                vals[name][c] = x / cnt[name]
    lines = [f"# {title}", "", "Commands (repository root, one MI355X; one counter pass each):", "", "```", *cmds, "```",
             "", "Values per dispatch (mean over the kernel's dispatches; counters summed over the device as "
             "`run_counter_collection.csv` reports them).  Percentages of the first rows are shares of SQ_WAVE_CYCLES.",
             "", "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |", "|---|" + "---:|" * len(kernels)]

    def row(label, f):
        cells = []
        for k in kernels:
            try:
                cells.append(f(vals[k]))
            except (KeyError, ZeroDivisionError):
                cells.append("n/a")
        lines.append(f"| {label} | " + " | ".join(cells) + " |")

    row("SQ_WAVE_CYCLES", lambda v: f"{v['SQ_WAVE_CYCLES']:,.0f}")
    for c, label in (("SQ_WAIT_ANY", "SQ_WAIT_ANY (waiting on s_waitcnt / barriers)"),
                     ("SQ_WAIT_INST_ANY", "SQ_WAIT_INST_ANY (waiting for an issue slot)"),
                     ("SQ_WAIT_INST_LDS", "SQ_WAIT_INST_LDS"),
                     ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_ANY"),
                     ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_VALU (MFMA included)"),
                     ("SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_LDS"),
                     ("SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_VMEM")):
        row(label, lambda v, c=c: f"{v[c]:,.0f} ({100 * v[c] / v['SQ_WAVE_CYCLES']:.1f}%)")
    row("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (active cycles per XCD x 1024 SIMDs)",
        lambda v: f"{100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (v['GRBM_GUI_ACTIVE'] * SIMD_NUM):.1f}%")
    row("SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE",
        lambda v: f"{100 * v['SQ_LDS_BANK_CONFLICT'] / v['SQ_LDS_IDX_ACTIVE']:.1f}%")
    row("SQ_LDS_IDX_ACTIVE / SQ_BUSY_CYCLES", lambda v: f"{v['SQ_LDS_IDX_ACTIVE'] / v['SQ_BUSY_CYCLES']:.2f}")
    row("SQ_LDS_DATA_FIFO_FULL", lambda v: f"{v['SQ_LDS_DATA_FIFO_FULL']:,.0f}")
    row("SQ_LDS_CMD_FIFO_FULL", lambda v: f"{v['SQ_LDS_CMD_FIFO_FULL']:,.0f}")
    row("L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS)",
        lambda v: f"{100 * v['TCC_HIT_sum'] / (v['TCC_HIT_sum'] + v['TCC_MISS_sum']):.1f}%")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("src")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--split-at", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--md")
    t.add_argument("--cmd-fetch", default="")
    t.add_argument("--cmd-write", default="")
    q = sub.add_parser("reqsize")
    q.add_argument("src")
    q.add_argument("out")
    q.add_argument("--cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--cmd-pmc", default="")
    m.add_argument("--cmd-stats", default="")
    m.add_argument("--title", required=True)
    w = sub.add_parser("waves")
    w.add_argument("--dirs", nargs="+", required=True)
    w.add_argument("--kernels", nargs="+", required=True)
    w.add_argument("--cmds", nargs="+", required=True)
    w.add_argument("--out", required=True)
    w.add_argument("--title", required=True)
    lib = sub.add_parser("library")
    lib.add_argument("out")
    lib.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.action == "waves":
        waves_md(a.dirs, a.kernels, a.out, a.cmds, a.title)
    elif a.action == "library":
        library_md(a.out, a.cmd)
    elif a.action == "mfma":
        mfma_md(a.pmc, a.stats, a.out, a.cmd_pmc, a.cmd_stats, a.title)
    elif a.action == "stats":
        stats_md(a.src, a.out, a.cmd, a.title, a.note, a.split_at)
    elif a.action == "reqsize":
        reqsize_md(a.src, a.out, a.cmd)
    else:
        res = traffic(a.fetch, a.write, a.workload)
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1)
        if a.md:
            traffic_md(res, a.md, a.cmd_fetch, a.cmd_write)
    return 0


if __name__ == "__main__":
    sys.exit(main())
