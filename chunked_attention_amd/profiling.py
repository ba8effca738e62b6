"""Summaries of rocprofv3 CSV output for the profiles/ folder.

    python -m chunked_attention_amd.profiling stats DIR --cmd "..." --out FILE.md
        kernel statistics (--kernel-trace --stats --output-format csv run in DIR)
    python -m chunked_attention_amd.profiling counters DIR [DIR ...] --cmd "..." [--cmd ...] \\
        --flops F --out FILE.md
        SQ / TCC / GRBM counters of the attention kernel (one --pmc run per
        DIR), per dispatch, with the MFMA-busy fraction and its algorithmic part
    python -m chunked_attention_amd.profiling traffic --fetch DIR --write DIR \\
        --calib-mib M --cmd-fetch "..." --cmd-write "..." --out FILE.json --md FILE.md
        HBM bytes per launch of the attention kernel from two counter runs
        (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
        the same counter's reading for a plain elementwise kernel that reads
        and writes M MiB once.

Only the last `--steady` dispatches of the attention kernel are used: the
earlier ones run while the window fills and attend fewer keys.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the sources the bf16 attention kernel is compiled from
KERNEL_SOURCES = [os.path.join(ROOT, "chunked_attention_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "attn_common.hpp", "device_common.hpp",
                            "kvc_internal.hpp")] + [os.path.join(ROOT, "include", "kvc.h")]


def kernel_code_digest() -> str:
    """sha256 of the attention kernel's sources with comments and whitespace
    removed: it changes when the code changes, not when a comment does."""
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        txt = open(path, encoding="utf-8").read()
        txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
        txt = re.sub(r"//[^\n]*", " ", txt)
        h.update(" ".join(txt.split()).encode())
    return h.hexdigest()
ATTN = "attn_fwd_bf16"
ATTN8 = "attn_fwd_fp8"
CALIB = "neg_kernel"


def _one(dirname: str, pattern: str) -> str:
    hits = sorted(glob.glob(os.path.join(dirname, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {dirname}")
    return hits[-1]


def short_name(name: str) -> str:
    for key in (ATTN, ATTN8, "cache_write", "cache_amax", "cache_quant", "edit_mask_kernel",
                "fill_u32", CALIB):
        if key in name:
            if key in (ATTN, ATTN8):
                i = name.find(key + "<")
                return name[i:name.find(">", i) + 1] if i >= 0 else key
            return key
    return name[:60]


def steady_attention(dirname: str, steady: int):
    """(kernel, mean us, calls) of the last `steady` attention dispatches in the
    kernel trace: the timed steady-state calls of a bench run."""
    path = _one(dirname, "*kernel_trace.csv")
    rows = [r for r in csv.DictReader(open(path))
            if ATTN in r["Kernel_Name"] or ATTN8 in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-steady:]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in last]
    return short_name(last[-1]["Kernel_Name"]), statistics.mean(durs), len(durs)


def steady_mean_us(dirname: str, kernel: str, steady: int) -> float:
    """mean duration (us) of the last `steady` dispatches of `kernel` in a
    kernel trace"""
    path = _one(dirname, "*kernel_trace.csv")
    rows = [r for r in csv.DictReader(open(path)) if _is(kernel, r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    last = rows[-steady:]
    if not last:
        raise SystemExit(f"no {kernel} dispatches in {path}")
    return statistics.mean((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                           for r in last)


def stats_md(dirname: str, cmd: str, steady: int = 0) -> str:
    path = _one(dirname, "*kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", "",
           "```", cmd, "```", "",
           "| kernel | calls | total us | average us | min us | max us | % time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        ns = lambda k: float(r[k]) / 1e3
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {ns('TotalDurationNs'):.1f} | "
                   f"{ns('AverageNs'):.2f} | {ns('MinNs'):.2f} | {ns('MaxNs'):.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    out.append("")
    if steady:
        k, mean_us, n = steady_attention(dirname, steady)
        out += [f"Steady state (the last {n} calls of {k}, the bench's timed steps, from the "
                f"kernel trace): mean {mean_us:.2f} us per call.", ""]
    return "\n".join(out)


def _counter(dirname: str, counter: str):
    path = _one(dirname, "*counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        did = int(r["Dispatch_Id"])
        per.setdefault(did, [r["Kernel_Name"], 0.0])
        per[did][1] += float(r["Counter_Value"])
    return [per[d] for d in sorted(per)]


def _dispatches(dirname: str):
    """{dispatch id: (kernel name, duration ns, {counter: value summed over instances})}"""
    path = _one(dirname, "*counter_collection.csv")
    per = {}
    for r in csv.DictReader(open(path)):
        did = int(r["Dispatch_Id"])
        if did not in per:
            per[did] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {})
        c = per[did][2]
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


# gfx950: 256 CUs in 8 XCDs, 4 SIMDs per CU; a 32x32x16 bf16 MFMA keeps its
# SIMD's matrix pipe busy 32 cycles for 32768 FLOPs
CUS, XCDS, SIMDS = 256, 8, 4
BF16_FLOPS_PER_SIMD_CYCLE = 1024


# dense fp8 (E4M3) MFMAs do twice the FLOPs per SIMD-cycle of bf16 ones
FLOPS_PER_SIMD_CYCLE = {ATTN: BF16_FLOPS_PER_SIMD_CYCLE, ATTN8: 2 * BF16_FLOPS_PER_SIMD_CYCLE}


def counters_md(dirs, cmds, steady: int, flops: float, workload: str, kernel: str = ATTN) -> str:
    vals, durs = {}, []
    for d in dirs:
        attn = [v for _, v in sorted(_dispatches(d).items())
                if kernel in v[0] and not (kernel == ATTN and ATTN8 in v[0])][-steady:]
        if not attn:
            raise SystemExit(f"no {kernel} dispatches in {d}")
        durs += [dur for _, dur, _ in attn]
        for name in attn[0][2]:
            vals[name] = statistics.mean(c[name] for _, _, c in attn)
    dur_s = statistics.mean(durs) * 1e-9
    out = [f"# Counters of {kernel} (rocprofv3 --pmc)", "",
           f"Workload: {workload}.  Each counter summed over its hardware instances and "
           f"averaged over the last {steady} {kernel} dispatches of its run; one run per "
           f"counter set.", "", "Commands (from the repository root):", "", "```", *cmds,
           "```", "", "| counter | per dispatch |", "|---|---|"]
    out += [f"| {k} | {v:,.0f} |" for k, v in sorted(vals.items())]
    out += ["", f"Mean dispatch time in these runs: {dur_s * 1e6:.1f} us.", ""]
    derived = []
    if "GRBM_GUI_ACTIVE" in vals:
        cycles = vals["GRBM_GUI_ACTIVE"] / XCDS
        derived.append(f"- GPU cycles per dispatch: GRBM_GUI_ACTIVE / {XCDS} XCDs = "
                       f"{cycles:,.0f}, i.e. a {cycles / dur_s / 1e9:.2f} GHz clock over the "
                       f"dispatch time.")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            simd_cycles = cycles * CUS * SIMDS
            busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"]
            derived.append(f"- Matrix pipes busy: SQ_VALU_MFMA_BUSY_CYCLES / ({CUS} CUs x "
                           f"{SIMDS} SIMDs x cycles) = {100 * busy / simd_cycles:.1f}%.")
            if flops:
                per = FLOPS_PER_SIMD_CYCLE.get(kernel, BF16_FLOPS_PER_SIMD_CYCLE)
                need = flops / per
                derived.append(f"- The algorithmic {flops / 1e9:.2f} GFLOP need {need:,.0f} "
                               f"busy SIMD-cycles at {per} FLOP each: "
                               f"{100 * need / busy:.1f}% of the busy cycles (the rest: "
                               f"padded tiles and rows).")
    if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_INSTS_LDS"):
        derived.append(f"- LDS bank-conflict cycles per LDS instruction: "
                       f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_INSTS_LDS']:.3f}.")
    if "TCC_HIT_sum" in vals and "TCC_MISS_sum" in vals:
        h, m = vals["TCC_HIT_sum"], vals["TCC_MISS_sum"]
        derived.append(f"- L2 hit rate: {100 * h / (h + m):.1f}%.")
    if derived:
        out += ["Derived:", ""] + derived + [""]
    return "\n".join(out)


def _is(kernel: str, name: str) -> bool:
    return kernel in name and not (kernel == ATTN and ATTN8 in name)


def traffic(fetch_dir, write_dir, calib_mib, steady, kernel: str = ATTN):
    calib_bytes = calib_mib << 20
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter(d, counter)
        attn = [v for n, v in rows if _is(kernel, n)][-steady:]
        cal = [v for n, v in rows if CALIB in n]
        if not attn or not cal:
            raise SystemExit(f"{counter}: no {kernel} or calibration dispatches in {d}")
        kib_attn = statistics.mean(attn)
        kib_cal = statistics.median(cal)
        factor = calib_bytes / (kib_cal * 1024.0)
        res[counter] = {"attn_kib_per_dispatch": kib_attn, "attn_dispatches": len(attn),
                        "calib_kib_per_dispatch": kib_cal, "calib_bytes": calib_bytes,
                        "scale": factor, "attn_bytes": kib_attn * 1024.0 * factor}
    total = res["FETCH_SIZE"]["attn_bytes"] + res["WRITE_SIZE"]["attn_bytes"]
    return res, total


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--cmd", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--steady", type=int, default=0,
                   help="also report the mean of the last N attention dispatches")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--steady", type=int, default=3)
    c.add_argument("--flops", type=float, default=0.0, help="algorithmic FLOPs per call")
    c.add_argument("--workload", default="720p steady chunk (8356 keys)")
    c.add_argument("--kernel", default=ATTN, help="kernel name (substring) to summarise")
    c.add_argument("--out", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--calib-mib", type=int, required=True)
    b.add_argument("--steady", type=int, default=3)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--workload", default="720p steady chunk (8356 keys)")
    b.add_argument("--kernel", default=ATTN, help="kernel name (substring) to summarise")
    b.add_argument("--stats-dir", default=None,
                   help="kernel-trace run of the same command: mean duration of the same "
                        "dispatches, for GB/s")
    b.add_argument("--algo-bytes", type=float, default=0.0,
                   help="algorithmic bytes per dispatch (reads + writes)")
    b.add_argument("--out", default=None, help="JSON record (the bf16 attention kernel)")
    b.add_argument("--md", required=True)
    args = ap.parse_args(argv)
    if args.what == "stats":
        open(args.out, "w").write(stats_md(args.dir, args.cmd, args.steady))
        return 0
    if args.what == "counters":
        open(args.out, "w").write(counters_md(args.dirs, args.cmd, args.steady, args.flops,
                                              args.workload, args.kernel))
        return 0
    res, total = traffic(args.fetch, args.write, args.calib_mib, args.steady, args.kernel)
    sha = kernel_code_digest()
    if args.out:
        rec = {"kernel": args.kernel, "workload": args.workload, "kernel_code_sha256": sha,
               "hbm_bytes_per_launch": round(total), "counters": res,
               "commands": {"FETCH_SIZE": args.cmd_fetch, "WRITE_SIZE": args.cmd_write}}
        json.dump(rec, open(args.out, "w"), indent=1)
    f, wr = res["FETCH_SIZE"], res["WRITE_SIZE"]
    md = [f"# HBM traffic of {args.kernel} (rocprofv3 counters)", "",
          f"Workload: {args.workload}.  Counters in KiB per dispatch, averaged over the "
          f"last {f['attn_dispatches']} {args.kernel} dispatches (steady state); each counter "
          f"is scaled by bytes / reading of a plain elementwise kernel that reads and writes "
          f"{args.calib_mib} MiB once.", "",
          "Commands (from the repository root):", "", "```", args.cmd_fetch, args.cmd_write,
          "```", "",
          "| counter | kernel KiB/dispatch | calibration KiB/dispatch | scale | bytes/launch |",
          "|---|---|---|---|---|",
          f"| FETCH_SIZE | {f['attn_kib_per_dispatch']:.0f} | {f['calib_kib_per_dispatch']:.0f} | "
          f"{f['scale']:.4f} | {f['attn_bytes'] / 1e6:.1f} MB |",
          f"| WRITE_SIZE | {wr['attn_kib_per_dispatch']:.0f} | {wr['calib_kib_per_dispatch']:.0f} | "
          f"{wr['scale']:.4f} | {wr['attn_bytes'] / 1e6:.1f} MB |",
          "", f"Total HBM bytes per launch: {total / 1e6:.1f} MB."]
    if args.algo_bytes:
        md.append(f"Algorithmic bytes per launch: {args.algo_bytes / 1e6:.1f} MB "
                  f"(measured / algorithmic = {total / args.algo_bytes:.2f}).")
    if args.stats_dir:
        us = steady_mean_us(args.stats_dir, args.kernel, args.steady)
        md.append(f"Mean duration of the same dispatches in a kernel-trace run of the same "
                  f"command: {us:.2f} us, i.e. {total / (us * 1e-6) / 1e9:,.0f} GB/s measured"
                  + (f" and {args.algo_bytes / (us * 1e-6) / 1e9:,.0f} GB/s algorithmic"
                     if args.algo_bytes else "") + " against the 8,000 GB/s HBM peak.")
    if args.kernel == ATTN:
        md.append(f"Kernel code sha256 {sha[:16]}... (the bf16 attention kernel's sources).")
    md.append("")
    open(args.md, "w").write("\n".join(md))
    print(json.dumps({"hbm_bytes_per_launch": round(total)}))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
