"""Summaries of rocprofv3 output for profiles/ (markdown, a few KB each).

Reads the CSV files rocprofv3 writes (``--output-format csv``) and prints a
markdown summary; with ``--out`` it writes it to that file.  Kernel names
are shortened to a label: the library's GEMM kernel is named by its element
type, tile and stage (Gram, polynomial, update), read from its template
arguments.

  trace    <dir>                     --kernel-trace --stats: calls, average and
                                     total duration per kernel, per optimizer step
  mfma     <dir> --trace <dir>       --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
                                     SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE:
                                     executed MFMA flops, busy fraction, clock
  traffic  <fetch dir> <write dir>   --pmc FETCH_SIZE and --pmc WRITE_SIZE, each
                                     scaled by what the counter reads for the 1 GiB
                                     calibration copy in the same run
  counters <dir> [<dir> ...]         several --pmc passes of memory-pipeline counters:
                                     L2 latency and hit rate, address translation,
                                     texture-addresser and LDS activity

The optimizer steps in a run are counted as the dispatches of the momentum
kernel (one per step).  ``--command`` records the commands that produced the
input; ``--title`` names the summary.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
from collections import OrderedDict, defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ROOT, "matrix_aware_optimizer_step_amd", "csrc")
PEAK_BF16_TFLOPS = 2500.0
SIMDS = 1024            # 256 CUs x 4 SIMDs
XCDS = 8
# one dispatch per optimizer step: the momentum kernel of the packed pair, or of the separate calls
STEP_KERNELS = ("momentum_pack_kernel", "momentum_grouped_kernel")
EPI = {0: "Gram A=XX^T", 1: "poly B=bA+cAA", 2: "update X=aX+BX", 3: "update, last step (caller output)"}


def sha256(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def label(name: str) -> str:
    """Short label of a kernel name as rocprofv3 prints it."""
    m = re.search(r"ns_gemm_kernel<([^>]*)>", name)
    if m:
        args = [a.strip() for a in m.group(1).split(",")]
        dt = "bf16" if args[0] in ("unsigned short", "ushort", "uint16_t") else "fp32"
        bm = int(args[1])
        epi = int(args[4])
        bn = int(args[12]) if len(args) > 12 else bm
        qn = int(args[13]) if len(args) > 13 else 0
        ap = int(args[14]) if len(args) > 14 else 0
        stage = EPI.get(epi, f"epi {epi}")
        if epi == 3 and ap:
            stage = "update, last step (applies the update to W)"
        if epi in (2, 3):
            stage += ", X k-major" if qn else ", X^T operand"
        return f"ns_gemm_kernel {dt} {bm}x{bn} [{stage}]"
    base = name.replace("(anonymous namespace)", "anon")
    base = re.sub(r"\(.*$", "", base)          # drop the argument list
    base = re.sub(r"<.*$", "", base)           # and template arguments
    base = base.split("::")[-1].replace("void ", "").strip()
    return base


LIBRARY_KERNELS = ("ns_gemm", "gram_reduce", "momentum", "pack", "apply", "finalize", "sumsq", "copy_out", "adamw", "sgemm", "qr_",
                   "rot_adam", "eye", "gather_kernel", "sign_copy", "ns_")


def find(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    return files


def rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def col(r, *names):
    for n in names:
        if n in r:
            return r[n]
    raise KeyError(f"none of {names} in {list(r)}")


def trace_table(d):
    """label -> [durations in ns], from the kernel trace; and the step count."""
    durs = defaultdict(list)
    for p in find(d, "kernel_trace.csv"):
        for r in rows(p):
            n = col(r, "Kernel_Name", "KernelName", "Name")
            t = int(col(r, "End_Timestamp", "EndNs")) - int(col(r, "Start_Timestamp", "BeginNs"))
            durs[label(n)].append(t)
    steps = sum(len(durs.get(k, [])) for k in STEP_KERNELS)
    return durs, steps


def counters(d):
    """dispatch id -> {"label", "start", "end", counter name -> value}."""
    out = OrderedDict()
    for p in find(d, "counter_collection.csv"):
        for r in rows(p):
            key = (p, col(r, "Dispatch_Id", "Dispatch-Id", "Index"))
            e = out.setdefault(key, {"label": label(col(r, "Kernel_Name", "KernelName", "Name"))})
            try:
                e["start"] = int(col(r, "Start_Timestamp", "Begin_Timestamp"))
                e["end"] = int(col(r, "End_Timestamp"))
            except KeyError:
                pass
            e[col(r, "Counter_Name")] = float(col(r, "Counter_Value"))
    return list(out.values())


def header(title, commands, note=None):
    lines = [f"# {title}", "", "Commands (on the MI355X box from /tmp with TMPDIR=/tmp; $R = the repository root there):",
             "", "```"]
    lines += commands
    lines += ["```", ""]
    if note:
        lines += [note, ""]
    lines.append(f"ns_gemm.hip sha256 at the time of the run: `{sha256(os.path.join(SRC, 'ns_gemm.hip'))}`")
    lines.append("")
    return lines


def cmd_trace(a):
    durs, steps = trace_table(a.dirs[0])
    lines = header(a.title, a.command, f"The trace covers {steps} optimizer steps (the dispatches of "
                                       f"{' or '.join(STEP_KERNELS)}); kernels that are not the library's (input generation) are "
                                       f"omitted.")
    lines += ["| kernel | calls | avg us | total ms | ms per step |", "|---|---:|---:|---:|---:|"]
    ours = {k: v for k, v in durs.items() if k.startswith(LIBRARY_KERNELS)}
    ns_total = 0.0
    for k, v in sorted(ours.items(), key=lambda kv: -sum(kv[1])):
        tot = sum(v) / 1e6
        per = tot / steps if steps else float("nan")
        lines.append(f"| {k} | {len(v)} | {statistics.mean(v) / 1e3:.1f} | {tot:.2f} | {per:.3f} |")
        if k.startswith(("ns_gemm", "gram_reduce", "pack", "ns_")):
            ns_total += per
    lines += ["", f"Newton-Schulz kernels (every ns_gemm launch and the operand packing) per step: {ns_total:.3f} ms.",
              ""]
    return lines


def cmd_mfma(a):
    disp = counters(a.dirs[0])
    tdurs, _ = trace_table(a.trace) if a.trace else ({}, 0)
    steps = sum(1 for e in disp if e["label"] in STEP_KERNELS)
    fam = OrderedDict()
    for e in disp:
        if not e["label"].startswith("ns_gemm"):
            continue
        fam.setdefault(e["label"], []).append(e)
    note = ("Per launch family, averaged over its dispatches: executed bf16 MFMA flops = "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x "
            f"{SIMDS} SIMDs) (GRBM_GUI_ACTIVE is summed over the {XCDS} XCDs); clock = GRBM_GUI_ACTIVE/8 / the "
            "dispatch's duration in this run (not given for dispatches under 50 us, where the counter's window and the "
            "timestamps disagree); executed TFLOP/s = executed flops / the average duration of the "
            "same family in the kernel trace of the same command without counters. Executed flops include work "
            "beyond the algorithmic count (full diagonal tiles of the symmetric products, padding).")
    lines = header(a.title, a.command, note)
    lines += ["| kernel | dispatches | executed GFLOP / launch | trace avg us | executed TFLOP/s | % of 2.5 PFLOP/s "
              "| MFMA busy % | clock GHz |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    tot_flops = tot_time = tot_busy = tot_active = 0.0
    for k, es in fam.items():
        fl = statistics.mean(e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for e in es)
        act = [e["GRBM_GUI_ACTIVE"] / XCDS for e in es]
        busy = statistics.mean(e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) for e in es)
        long_ = [e for e in es if "end" in e and e["end"] - e["start"] >= 50_000]
        clk = statistics.mean(e["GRBM_GUI_ACTIVE"] / XCDS / (e["end"] - e["start"]) for e in long_) if long_ else None
        tavg = statistics.mean(tdurs[k]) / 1e3 if k in tdurs else float("nan")
        tf = fl / (tavg * 1e-6) / 1e12 if k in tdurs else float("nan")
        lines.append(f"| {k} | {len(es)} | {fl / 1e9:.1f} | {tavg:.1f} | {tf:.0f} | {100 * tf / PEAK_BF16_TFLOPS:.1f} "
                     f"| {100 * busy:.1f} | {'-' if clk is None else f'{clk:.2f}'} |")
        per_step = len(es) / steps if steps else 0
        tot_flops += fl * per_step
        tot_time += (tavg if k in tdurs else 0.0) * per_step
        tot_busy += sum(e["SQ_VALU_MFMA_BUSY_CYCLES"] for e in es) / (steps or 1)
        tot_active += sum(e["GRBM_GUI_ACTIVE"] / XCDS * SIMDS for e in es) / (steps or 1)
    if tot_time > 0:
        lines += ["", f"Per optimizer step, all Newton-Schulz GEMM launches: {tot_flops / 1e12:.2f} TFLOP executed in "
                      f"{tot_time / 1e3:.3f} ms of kernel time ({tot_flops / (tot_time * 1e-6) / 1e12:.0f} TFLOP/s "
                      f"executed); MFMA busy {100 * tot_busy / tot_active:.1f} % of the GPU-active SIMD cycles.", ""]
    return lines


def cmd_traffic(a):
    fetch, write = counters(a.dirs[0]), counters(a.dirs[1])
    cal_f = [e["FETCH_SIZE"] for e in fetch if "copyBuffer" in e["label"] or "copy" in e["label"].lower()]
    cal_w = [e["WRITE_SIZE"] for e in write if "copyBuffer" in e["label"] or "copy" in e["label"].lower()]
    if not cal_f or not cal_w:
        sys.exit("no calibration copy kernel in the counter output (run the benchmark with --copy-calibration)")
    gib_kb = 1 << 20
    fs, ws = gib_kb / max(cal_f), gib_kb / max(cal_w)
    steps = sum(1 for e in fetch if e["label"] in STEP_KERNELS)
    note = (f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {max(cal_f):.0f} KB and WRITE_SIZE = "
            f"{max(cal_w):.0f} KB against {gib_kb} KB moved each way; the factors applied below are {fs:.3f} (fetch) "
            f"and {ws:.3f} (write).")
    lines = header(a.title, a.command, note)
    lines += ["| kernel | launches | fetch GB/launch (scaled) | write GB/launch (scaled) |", "|---|---:|---:|---:|"]
    fam_f, fam_w = defaultdict(list), defaultdict(list)
    for e in fetch:
        fam_f[e["label"]].append(e["FETCH_SIZE"] * 1024 * fs)
    for e in write:
        fam_w[e["label"]].append(e["WRITE_SIZE"] * 1024 * ws)
    ns_bytes = 0.0
    launches = 0
    for k in sorted(fam_f):
        if not k.startswith(LIBRARY_KERNELS):
            continue
        f = statistics.mean(fam_f[k])
        w = statistics.mean(fam_w[k]) if fam_w.get(k) else float("nan")
        lines.append(f"| {k} | {len(fam_f[k])} | {f / 1e9:.3f} | {w / 1e9:.3f} |")
        if k.startswith("ns_gemm"):
            ns_bytes += (sum(fam_f[k]) + sum(fam_w.get(k, []))) / (steps or 1)
            launches += len(fam_f[k]) / (steps or 1)
    rec = {"workload": a.workload, "kernel_source_sha256": sha256(os.path.join(SRC, "ns_gemm.hip")),
           "ns_gemm_bytes_per_step": ns_bytes, "fetch_scale": fs, "write_scale": ws}
    lines += ["", f"Newton-Schulz GEMM launches per step: {launches:.0f}; HBM bytes per step of those launches "
                  f"(fetch + write, scaled): {ns_bytes / 1e9:.3f} GB.", "", "traffic-record: " + json.dumps(rec), ""]
    return lines


# derived quantities of the memory-pipeline counters: (name, numerator, denominator, scale)
DERIVED = [("L2 read latency, cycles per request", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", 1),
           ("L2 write latency, cycles per request", "TCP_TCC_WRITE_REQ_LATENCY_sum", "TCP_TCC_WRITE_REQ_sum", 1),
           ("L2 hit rate %", "TCC_HIT_sum", ("TCC_HIT_sum", "TCC_MISS_sum"), 100),
           ("address translation miss rate %", "TCP_UTCL1_TRANSLATION_MISS_sum",
            ("TCP_UTCL1_TRANSLATION_MISS_sum", "TCP_UTCL1_TRANSLATION_HIT_sum"), 100),
           ("TA busy % (average TA over one XCD's active cycles)", "TA_BUSY_avr", "GRBM_GUI_ACTIVE/8", 100),
           ("LDS bank conflicts % of LDS-active cycles", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", 100),
           ("waves waiting on LDS instructions % of wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", 100),
           ("waves waiting (s_waitcnt, barriers) % of wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", 100),
           ("waves with an instruction ready but not issued % of wave cycles", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES",
            100)]


def cmd_counters(a):
    """Several --pmc passes of the same command: per launch family the mean
    of every counter over its dispatches, and the derived quantities."""
    fams = OrderedDict()
    for d in a.dirs:
        for e in counters(d):
            if not e["label"].startswith(LIBRARY_KERNELS):
                continue
            f = fams.setdefault(e["label"], {})
            for c, v in e.items():
                if c not in ("label", "start", "end"):
                    f.setdefault(c, []).append(v)
    note = ("Means over each launch family's dispatches, one --pmc pass per line of the commands (a counter "
            "taken in several passes is averaged over all of them); counters ending in _sum are summed over "
            "the GPU's instances, _avr averaged over them; GRBM_GUI_ACTIVE is summed over the 8 XCDs.")
    lines = header(a.title, a.command, note)
    names = [n for n, *_ in DERIVED]
    lines += ["| kernel | " + " | ".join(names) + " |", "|---|" + "---:|" * len(names)]

    def val(f, key):
        if key == "GRBM_GUI_ACTIVE/8":
            return statistics.mean(f["GRBM_GUI_ACTIVE"]) / XCDS if "GRBM_GUI_ACTIVE" in f else None
        if isinstance(key, tuple):
            parts = [val(f, k) for k in key]
            return None if None in parts else sum(parts)
        return statistics.mean(f[key]) if key in f else None

    for k, f in fams.items():
        cells = []
        for _, num, den, sc in DERIVED:
            n, d = val(f, num), val(f, den)
            cells.append("-" if n is None or not d else f"{sc * n / d:.1f}")
        lines.append(f"| {k} | " + " | ".join(cells) + " |")
    lines.append("")
    return lines


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kind", choices=["trace", "mfma", "traffic", "counters"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--trace", help="kernel-trace directory of the same command (mfma)")
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", action="append", default=[], help="a command that produced the input (repeatable)")
    ap.add_argument("--workload", default="", help="workload name for the traffic record")
    ap.add_argument("--out")
    a = ap.parse_args()
    lines = {"trace": cmd_trace, "mfma": cmd_mfma, "traffic": cmd_traffic, "counters": cmd_counters}[a.kind](a)
    text = "\n".join(lines)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
