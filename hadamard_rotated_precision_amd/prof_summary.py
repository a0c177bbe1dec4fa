"""Summaries of rocprofv3 CSV output for the profiles/ folder.

  python -m hadamard_rotated_precision_amd.prof_summary stats DIR OUT.md --cmd "..."
      per-kernel table from DIR/*kernel_stats.csv (calls, average and total duration).

  python -m hadamard_rotated_precision_amd.prof_summary counters DIR OUT.md --cmd "..." [--ratio A/B]
      any --pmc counters per kernel, averaged over its dispatches.

  python -m hadamard_rotated_precision_amd.prof_summary mfma DIR OUT.md --cmd "..."
      matrix-core counters per kernel (int8 MFMA ops, MFMA busy cycles, busy fraction).

  python -m hadamard_rotated_precision_amd.prof_summary traffic FETCH_DIR WRITE_DIR \
      --copy-bytes B --workload NAME --json OUT.json --md OUT.md --cmd "..."
      HBM bytes per GEMM launch, and of the prologue kernels per step, from two --pmc runs
      (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch). Each counter is scaled by what it reads for the plain device copies of B
      bytes the same run made (read B, write B), so the figure is in bytes of the copy's
      own accounting.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, "csrc", "hq_gemm.hip")
# the rotate -> quantize prologue: its kernels and the host code that picks them
PROLOGUE_SOURCES = [os.path.join(HERE, "csrc", f) for f in ("hq_prologue.hip", "hq_api.cpp")]
PROLOGUE_KERNELS = ("right_mma_kernel", "left_mma_kernel", "both_mma_kernel", "both_pipe_kernel",
                    "both_narrow_kernel", "both_single_kernel", "right_fast_kernel", "right_kernel",
                    "left_fast_kernel", "left_kernel", "both_kernel")


def prologue_source_hash():
    h = hashlib.sha256()
    for path in PROLOGUE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _is_prologue(key):
    return key.split("<")[0] in PROLOGUE_KERNELS


def _one(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise SystemExit("no file matches %s" % pattern)
    return files[0]


def short_name(name):
    name = re.sub(r"\(hq::\w+\)$", "", name)
    name = name.replace("void ", "").replace("hq::", "")
    return name[:100]


def cmd_stats(args):
    path = _one(os.path.join(args.dir, "**", "*kernel_stats.csv")) if not args.dir.endswith(".csv") \
        else args.dir
    rows = list(csv.DictReader(open(path)))
    out = ["# Kernel durations: %s" % args.title, "",
           "Command (from the repository root, rocprofv3 run in /tmp):", "",
           "```", args.cmd, "```", "",
           "| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append("| `%s` | %s | %.2f | %.1f | %.1f |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e3, float(r["Percentage"])))
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def _counter_rows(d, counter):
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    res = []
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        res.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    res.sort()
    return res


def _is_copy(name):
    n = name.lower()
    return "copy" in n and "hq::" not in n


def cmd_traffic(args):
    fetch = _counter_rows(args.fetch_dir, "FETCH_SIZE")
    write = _counter_rows(args.write_dir, "WRITE_SIZE")
    cf = [v for _, n, v in fetch if _is_copy(n)]
    cw = [v for _, n, v in write if _is_copy(n)]
    if not cf or not cw:
        raise SystemExit("no copy dispatches found for the calibration")
    # the largest copies are the calibration copies of --copy-bytes
    cf = sorted(cf)[-3:]
    cw = sorted(cw)[-3:]
    f_scale = (sum(cf) / len(cf)) * 1024.0 / args.copy_bytes
    w_scale = (sum(cw) / len(cw)) * 1024.0 / args.copy_bytes

    def per_kernel(rows, scale):
        acc = {}
        for _, n, v in rows:
            if "hq::" not in n:
                continue
            key = short_name(n)
            acc.setdefault(key, []).append(v * 1024.0 / scale)
        return acc

    kf = per_kernel(fetch, f_scale)
    kw = per_kernel(write, w_scale)
    gemm_f = [v for k, vs in kf.items() if "gemm_i8_kernel" in k for v in vs]
    gemm_w = [v for k, vs in kw.items() if "gemm_i8_kernel" in k for v in vs]
    if not gemm_f or not gemm_w:
        raise SystemExit("no GEMM dispatches found")
    fpl = sum(gemm_f) / len(gemm_f)
    wpl = sum(gemm_w) / len(gemm_w)
    # prologue bytes per step: every prologue dispatch of the run over the number of steps
    steps = len(gemm_f) / args.gemms_per_step
    pro_f = sum(v for k, vs in kf.items() if _is_prologue(k) for v in vs) / steps
    pro_w = sum(v for k, vs in kw.items() if _is_prologue(k) for v in vs) / steps
    with open(GEMM_SOURCE, "rb") as f:
        src_hash = hashlib.sha256(f.read()).hexdigest()[:16]
    doc = {"workload": args.workload, "gemm_source_sha256_16": src_hash,
           "bytes_per_launch": round(fpl + wpl), "fetch_bytes_per_launch": round(fpl),
           "write_bytes_per_launch": round(wpl), "gemm_launches_counted": len(gemm_f),
           "prologue_source_sha256_16": prologue_source_hash(),
           "prologue_bytes_per_step": round(pro_f + pro_w),
           "prologue_fetch_bytes_per_step": round(pro_f),
           "prologue_write_bytes_per_step": round(pro_w),
           "calibration": {"copy_bytes": args.copy_bytes,
                           "fetch_kib_per_copy": sum(cf) / len(cf),
                           "write_kib_per_copy": sum(cw) / len(cw),
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "command": args.cmd}
    json.dump(doc, open(args.json, "w"), indent=1)
    out = ["# Counted memory traffic per launch: %s" % args.workload, "",
           "Two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch). Each counter",
           "is divided by what it reads for a plain device copy of %d bytes in the same run" % args.copy_bytes,
           "(fetch scale %.4f, write scale %.4f counted bytes per copied byte)." % (f_scale, w_scale),
           "These counters count bytes between the L2s and the memory fabric, hits in the 256 MB",
           "MALL included: an upper bound on the HBM bytes, not the HBM bytes themselves.", "",
           "Commands (from the repository root, rocprofv3 run in /tmp):", "", "```", args.cmd, "```", "",
           "| kernel | dispatches | read MB / launch | written MB / launch |", "|---|---:|---:|---:|"]
    for k in sorted(set(kf) | set(kw)):
        f = kf.get(k, [0.0])
        w = kw.get(k, [0.0])
        out.append("| `%s` | %d | %.2f | %.2f |" % (k, len(f), sum(f) / len(f) / 1e6, sum(w) / len(w) / 1e6))
    out += ["", "GEMM average per launch: read %.2f MB, written %.2f MB, total %.2f MB "
            "(source hash %s)." % (fpl / 1e6, wpl / 1e6, (fpl + wpl) / 1e6, src_hash),
            "", "Prologue (rotate -> quantize kernels) per step: read %.2f MB, written %.2f MB, "
            "total %.2f MB (source hash %s)." % (pro_f / 1e6, pro_w / 1e6, (pro_f + pro_w) / 1e6,
                                                 prologue_source_hash())]
    open(args.md, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_mfma(args):
    """Matrix-core counters per kernel: int8 MFMA ops (SQ_INSTS_VALU_MFMA_MOPS_I8 x 512),
    MFMA busy cycles, and the busy fraction of all SIMDs over the kernel's active cycles."""
    path = _one(os.path.join(args.dir, "**", "*counter_collection.csv"))
    acc = {}
    for r in csv.DictReader(open(path)):
        if "hq::" not in r["Kernel_Name"]:
            continue
        acc.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    out = ["# Matrix-core counters: %s" % args.title, "",
           "One rocprofv3 --pmc run; values are per dispatch, averaged over the dispatches of each",
           "kernel. GRBM_GUI_ACTIVE comes summed over the %d XCDs (per XCD it matches the kernel's" % args.xcds,
           "duration times the clock), so MFMA busy %% = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE /",
           "%d x %d SIMDs). int8 ops = SQ_INSTS_VALU_MFMA_MOPS_I8 x 512." % (args.xcds, args.simds), "",
           "Command (from the repository root, rocprofv3 run in /tmp):", "", "```", args.cmd, "```", "",
           "| kernel | dispatches | int8 MFMA ops | MFMA busy cycles | active cycles per XCD | MFMA busy % |",
           "|---|---:|---:|---:|---:|---:|"]
    for k in sorted(acc):
        c = acc[k]
        avg = {n: sum(v) / len(v) for n, v in c.items()}
        n = len(next(iter(c.values())))
        gui = avg.get("GRBM_GUI_ACTIVE", 0.0) / args.xcds
        busy = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        ops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0) * 512
        util = 100.0 * busy / (gui * args.simds) if gui > 0 else 0.0
        out.append("| `%s` | %d | %.4g | %.4g | %.4g | %.1f |" % (k, n, ops, busy, gui, util))
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_counters(args):
    """Any --pmc counters per kernel: the value per dispatch (as rocprofv3 reports it for the
    device), averaged over the dispatches of each kernel; --ratio A/B adds a column A / B."""
    path = _one(os.path.join(args.dir, "**", "*counter_collection.csv"))
    acc = {}
    for r in csv.DictReader(open(path)):
        if "hq::" not in r["Kernel_Name"]:
            continue
        acc.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    names = sorted({n for c in acc.values() for n in c})
    ratios = [tuple(x.split("/")) for x in args.ratio]
    out = ["# Counters: %s" % args.title, "", args.note, "",
           "Command (from the repository root, rocprofv3 run in /tmp):", "", "```", args.cmd, "```", "",
           "| kernel | " + " | ".join(names + ["%s / %s" % r for r in ratios]) + " |",
           "|---|" + "---:|" * (len(names) + len(ratios))]
    for k in sorted(acc):
        avg = {n: sum(v) / len(v) for n, v in acc[k].items()}
        cells = ["%.4g" % avg.get(n, 0.0) for n in names]
        for a, b in ratios:
            cells.append("%.1f %%" % (100.0 * avg.get(a, 0.0) / avg[b]) if avg.get(b) else "-")
        out.append("| `%s` | %s |" % (k, " | ".join(cells)))
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--json", required=True)
    t.add_argument("--md", required=True)
    t.add_argument("--cmd", required=True)
    cc = sub.add_parser("counters")
    cc.add_argument("dir")
    cc.add_argument("out")
    cc.add_argument("--cmd", required=True)
    cc.add_argument("--title", default="")
    cc.add_argument("--note", default="")
    cc.add_argument("--ratio", action="append", default=[])
    mm = sub.add_parser("mfma")
    mm.add_argument("dir")
    mm.add_argument("out")
    mm.add_argument("--cmd", required=True)
    mm.add_argument("--title", default="")
    mm.add_argument("--xcds", type=int, default=8)
    mm.add_argument("--simds", type=int, default=1024)
    t.add_argument("--gemms-per-step", type=int, default=3,
                   help="GEMM launches per step of the workload (fwd + dX + dW = 3)")
    args = ap.parse_args(argv)
    if args.what == "stats":
        cmd_stats(args)
    elif args.what == "mfma":
        cmd_mfma(args)
    elif args.what == "counters":
        cmd_counters(args)
    else:
        cmd_traffic(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
