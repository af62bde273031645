"""Summaries of rocprofv3 runs of bench.py for profiles/ (measurement tooling, runs on the host).

    python profile_summary.py trace <kernel_trace.csv> --out profiles/<name>.md --command "<cmd>"
    python profile_summary.py mfma <counter_collection.csv> --out profiles/<name>.md --command "<cmd>"
    python profile_summary.py traffic --workload dense_v3 --bench-json <bench.json>
        --fetch <counter_collection.csv> --write <counter_collection.csv>
        --copy-fetch <counter_collection.csv> --copy-write <counter_collection.csv>
        --out-md profiles/<name>.md --out-json profiles/traffic_counters.json --command "<cmds>"

`trace`: per-kernel dispatch count, average and total duration from a --kernel-trace CSV.
`traffic`: HBM bytes per dispatch of every GEMM tile configuration from FETCH_SIZE and
WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for one plain 1 GiB
device copy (`bench.py --copy-calibration`: reads 1 GiB, writes 1 GiB), next to the algorithmic
bytes per launch that bench.py reports for the same kernel.  The JSON record carries the digest
of the GEMM sources, so bench.py uses it only while the kernel is unchanged.
"""

import argparse
import csv
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))


# tile configuration of a gemm_fp8_kernel instance: BN, BM, WN, WM, STAGES (then optional flags), layout
_CFG = re.compile(r"gemm_fp8_kernel<dg::Cfg<(\d+), (\d+), (\d+), (\d+), (\d+)(?:, \w+)*>, (\d)(?:, (true|false))?>")


def short_name(name):
    """'void dg::gemm_fp8_kernel<dg::Cfg<256, 128, 64, 64, 3>, 0>(dg::GemmParams)' ->
    'gemm_fp8_kernel 256x128/8waves (layout 0)'; other kernels: first 70 characters."""
    m = _CFG.search(name)
    if m:
        bn, bm, wn, wm, _, lay = (int(v) for v in m.groups()[:6])
        waves = (bn // wn) * (bm // wm)
        aq = ", activation quantization in the launch" if m.group(7) == "true" else ""
        return f"gemm_fp8_kernel {bn}x{bm}/{waves}waves (layout {lay}{aq})"
    m = re.search(r"dg::(\w+_kernel)", name)
    if m:
        return m.group(1)
    return name[:70]


def gemm_config(name):
    m = _CFG.search(name)
    if not m:
        return None
    bn, bm, wn, wm, _, layout = (int(v) for v in m.groups()[:6])
    # layout 3 (per-row B scales) is labelled like bench.py's configuration of the row-scaled GEMM,
    # and so is the kernel that quantizes its activations in the launch
    return (f"gemm_fp8_kernel {'rowscaled ' if layout == 3 else ''}{bn}x{bm}/{(bn // wn) * (bm // wm)}waves"
            f"{' +act-quant' if m.group(7) == 'true' else ''}")


def is_flush(name, us):
    """bench.py's untimed 512 MB write ahead of every timed GEMM group (a byte fill of ~100 us)."""
    return "FillFunctor" in name and us >= 20.0


def cmd_trace(args):
    per = defaultdict(list)
    disp = []
    with open(args.csv) as fh:
        for r in csv.DictReader(fh):
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per[short_name(r["Kernel_Name"])].append(us)
            disp.append((int(r["Start_Timestamp"]), r["Kernel_Name"], us))
    # the per-launch pass: GEMM dispatches that follow a flush with only GEMM dispatches between
    # (bench.py's R launches over rotated weights); the rest are the step's warm-up and graph replays
    per_launch = defaultdict(list)
    after_flush = False
    for _, name, us in sorted(disp):
        if is_flush(name, us):
            after_flush = True
        elif _CFG.search(name):
            if after_flush:
                per_launch[short_name(name)].append(us)
        else:
            after_flush = False
    rows = sorted(per.items(), key=lambda kv: -sum(kv[1]))
    total = sum(sum(v) for v in per.values())
    lines = [f"# rocprofv3 kernel trace: {args.title}", "", "Command:", "", "```", args.command, "```", "",
             "| kernel | dispatches | avg us | total us | share |", "|---|---|---|---|---|"]
    for k, v in rows:
        lines.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} | {sum(v):.1f} | {100 * sum(v) / total:.1f}% |")
    if per_launch:
        lines += ["", "GEMM dispatches of bench.py's per-launch pass only (those right after its 512 MB flush: "
                  "the launches its per-launch durations and roofline time; the table above also holds the "
                  "step's warm-up and graph-replay dispatches):", "",
                  "| kernel | dispatches | avg us |", "|---|---|---|"]
        for k, v in sorted(per_launch.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {k} | {len(v)} | {sum(v) / len(v):.2f} |")
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_per_dispatch(path, counter):
    """{kernel config or name: [value per dispatch]} for one counter (summed over instances)."""
    acc = defaultdict(float)
    names = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            acc[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    out = defaultdict(list)
    for key, v in acc.items():
        out[gemm_config(names[key]) or short_name(names[key])].append(v)
    return out


def copy_factor(path, counter):
    """Bytes per counter unit: 1 GiB over the counter's reading for the largest copy dispatch."""
    vals = counter_per_dispatch(path, counter)
    best = max((max(v), k) for k, v in vals.items())
    return (1 << 30) / best[0], best[1], best[0]


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_common.hpp", "common.hpp"):
        with open(os.path.join(ROOT, "fp8_block_scaled_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cmd_traffic(args):
    with open(args.bench_json) as fh:
        bench = json.loads(fh.read().strip().splitlines()[-1])
    # algorithmic bytes per launch per tile configuration, from bench.py's per-shape list, each
    # shape weighted by its launches per timed step (its weight copies), as the counter runs
    # dispatch it
    alg = defaultdict(list)
    for sh in bench["shapes"]:
        cfg = "gemm_fp8_kernel " + sh["config"].split("/split")[0]
        if sh["config"].endswith("+act-quant"):
            cfg += " +act-quant"
        alg[cfg] += [sh["gbps"] * sh["us"] * 1e3] * int(sh.get("rotations", 1))   # bytes = GB/s * us * 1e3
    ff, fk, fv = copy_factor(args.copy_fetch, "FETCH_SIZE")
    wf, wk, wv = copy_factor(args.copy_write, "WRITE_SIZE")
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    digest = source_digest()
    try:
        with open(args.out_json) as fh:
            store = json.load(fh)
    except (OSError, ValueError):
        store = {}
    rec = store.setdefault(args.workload, {})
    lines = [f"# HBM traffic per dispatch ({args.workload}): rocprofv3 FETCH_SIZE / WRITE_SIZE", "",
             "Commands:", "", "```", args.command, "```", "",
             f"Calibration (one plain 1 GiB device copy, `bench.py --copy-calibration`): FETCH_SIZE read "
             f"{fv:.0f} for 1 GiB read -> x{ff:.3f} bytes per unit; WRITE_SIZE read {wv:.0f} for 1 GiB "
             f"written -> x{wf:.3f} bytes per unit (copy kernel: {fk[:60]}).", "",
             f"GEMM source digest: `{digest}`.", "",
             "| kernel | dispatches | fetch MB/dispatch | write MB/dispatch | HBM MB/dispatch | algorithmic MB/launch | ratio |",
             "|---|---|---|---|---|---|---|"]
    for cfg in sorted(set(fetch) & set(write)):
        if not cfg.startswith("gemm_fp8_kernel") or cfg not in alg:
            continue
        f_b = sum(fetch[cfg]) / len(fetch[cfg]) * ff
        w_b = sum(write[cfg]) / len(write[cfg]) * wf
        a_b = sum(alg[cfg]) / len(alg[cfg])
        rec[cfg] = {"source_sha": digest, "hbm_bytes_per_launch": round(f_b + w_b),
                    "fetch_bytes_per_launch": round(f_b), "write_bytes_per_launch": round(w_b),
                    "algorithmic_bytes_per_launch": round(a_b), "dispatches": len(fetch[cfg]),
                    "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
        lines.append(f"| {cfg} | {len(fetch[cfg])} | {f_b / 1e6:.1f} | {w_b / 1e6:.1f} | {(f_b + w_b) / 1e6:.1f} | "
                     f"{a_b / 1e6:.1f} | {(f_b + w_b) / a_b:.2f} |")
    with open(args.out_json, "w") as fh:
        json.dump(store, fh, indent=1, sort_keys=True)
        fh.write("\n")
    with open(args.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_mfma(args):
    """MFMA-pipe utilisation per GEMM tile configuration from SQ_VALU_MFMA_BUSY_CYCLES (summed over
    the 1024 SIMDs), SQ_INSTS_MFMA and GRBM_GUI_ACTIVE (summed over the 8 XCDs), per dispatch."""
    import statistics
    acc = defaultdict(lambda: defaultdict(float))
    meta = {}
    with open(args.csv) as fh:
        for r in csv.DictReader(fh):
            d = int(r["Dispatch_Id"])
            acc[d][r["Counter_Name"]] += float(r["Counter_Value"])
            meta[d] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    per = defaultdict(list)
    for d, c in acc.items():
        cfg = gemm_config(meta[d][0])
        if not cfg or not c.get("GRBM_GUI_ACTIVE"):
            continue
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / args.simds            # MFMA-pipe cycles per SIMD
        gui = c["GRBM_GUI_ACTIVE"] / args.xcds                      # active cycles of one XCD
        per[cfg].append((busy / gui, busy / (meta[d][1] * args.clock_ghz),
                         c["SQ_VALU_MFMA_BUSY_CYCLES"] / (32 * c["SQ_INSTS_MFMA"]), meta[d][1] / 1e3, gui / meta[d][1]))
    lines = [f"# MFMA utilisation per GEMM tile configuration ({args.workload}): rocprofv3 counters", "",
             "Command:", "", "```", args.command, "```", "",
             f"Per dispatch: MFMA-pipe cycles per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / {args.simds}; utilisation = "
             f"that over the XCD's active cycles (GRBM_GUI_ACTIVE / {args.xcds}: the counter is summed over the "
             f"XCDs), and over the dispatch's duration at {args.clock_ghz} GHz.  SQ_VALU_MFMA_BUSY_CYCLES equals "
             "32 cycles per 16x16x128 FP8 MFMA (SQ_INSTS_MFMA), the instruction's pipe occupancy at the "
             "published 5.0 PFLOP/s dense FP8 peak.", "",
             "| kernel | dispatches | MFMA util (active cycles) | MFMA util (duration, %.1f GHz) | busy / (32 x MFMAs) | avg us | active cycles per ns |" % args.clock_ghz,
             "|---|---|---|---|---|---|---|"]
    for cfg, v in sorted(per.items()):
        m = lambda i: statistics.mean(x[i] for x in v)
        lines.append(f"| {cfg} | {len(v)} | {100 * m(0):.1f}% | {100 * m(1):.1f}% | {m(2):.3f} | {m(3):.1f} | {m(4):.2f} |")
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="bench.py")
    t.add_argument("--command", required=True)
    c = sub.add_parser("traffic")
    for a in ("--bench-json", "--fetch", "--write", "--copy-fetch", "--copy-write", "--out-md", "--out-json",
              "--command", "--workload"):
        c.add_argument(a, required=True)
    mf = sub.add_parser("mfma")
    mf.add_argument("csv")
    mf.add_argument("--out", required=True)
    mf.add_argument("--command", required=True)
    mf.add_argument("--workload", default="dense_v3")
    mf.add_argument("--simds", type=int, default=1024)
    mf.add_argument("--xcds", type=int, default=8)
    mf.add_argument("--clock-ghz", type=float, default=2.4)
    args = ap.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "mfma": cmd_mfma}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
