"""rocprofv3 summaries for the committed profiles.

Subcommands (run from the repository root):

  copy     --mib M --reps R
           Runs torch's device-to-device copy of M MiB R times: the plain
           copy kernel whose FETCH_SIZE / WRITE_SIZE readings calibrate the
           counters (it reads M MiB and writes M MiB per dispatch).

  stats    --csv <kernel_stats.csv> --cmd "<command>" --out <file.md>
           Markdown table of a --kernel-trace --stats run, plus one
           aggregate line per kernel group (--group NAME=REGEX, repeatable).

  traffic  --fetch <counter_collection.csv> --write <counter_collection.csv>
           --calib-fetch <csv> --calib-write <csv> --calib-bytes B
           --key NAME=REGEX [--key ...] --out profiles/counters.json
           HBM bytes per launch for each kernel group: the mean FETCH_SIZE
           (and WRITE_SIZE) per dispatch of the group's kernels, each scaled
           by (B / the same counter's reading for the calibration copy).
           Stored under NAME with the hash of the kernel sources, so that a
           reader can tell when a kernel has changed since the counters were
           taken.

  gemm     --dtype Q4_K --M 14336 --K 4096 --N 32 --reps R
           Runs qmm_gemm R times on the seeded synthetic blob and activations
           of that shape, over enough copies of the blob to fill 1 GiB (so
           that every launch reads its weights from HBM): the program the
           per-shape counter runs profile.

  counters --csv <counter_collection.csv> --key REGEX --title T --cmd C
           Markdown table of every counter in a --pmc run, the mean per
           dispatch (summed over the device) of the dispatches whose kernel
           name matches REGEX, with the mean dispatch duration.

  sweep    --log <bench --sweep output> --out <file.md>
           Markdown tables of the JSON lines `bench.py --sweep` prints, one
           table per workload.

  spec     --log <bench --spec-verify output> --out <file.md>
           Markdown table of the JSON lines `bench.py --spec-verify` prints.

  mfma     --csv <counter_collection.csv> --key REGEX --flops F --simds S
           Matrix-core utilisation of the dispatches whose kernel name matches
           REGEX, from a run collecting SQ_VALU_MFMA_BUSY_CYCLES,
           SQ_INSTS_VALU_MFMA_MOPS_F16 and GRBM_GUI_ACTIVE (rocprofv3 reports
           each summed over the device: GRBM_GUI_ACTIVE over its --xccs
           dies): busy fraction = MFMA busy cycles / (GUI-active cycles per
           die x S SIMDs), the clock = GUI-active cycles per die / duration,
           the f16 matrix FLOPs the counters saw (MOPS x 512) against the
           algorithmic F per dispatch, and the TFLOP/s of F over the duration.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gguf_block_quant_qmm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _copy(args):
    import torch
    n = args.mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(args.reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {args.mib} MiB x {args.reps}", flush=True)


def _gemm(args):
    import torch

    import gguf_block_quant_qmm_amd as q
    from qmm_inputs import BY_NAME, make_blob, make_x, rng_for
    dt = BY_NAME[args.dtype]
    blob = torch.from_numpy(make_blob(dt, args.M, args.K, rng_for(90, 0))).cuda()
    copies = [blob] + [blob.clone() for _ in range(max(0, -(-(1 << 30) // blob.numel()) - 1))]
    X = torch.from_numpy(make_x(args.N, args.K, rng_for(90, 1))).cuda()
    Y = torch.empty((args.N, args.M), device="cuda")
    for r in range(args.reps):
        q.qmm_gemm(copies[r % len(copies)], dt, args.M, args.K, args.N, X, Y)
    torch.cuda.synchronize()
    print(f"qmm_gemm {args.dtype} {args.M}x{args.K} N={args.N} x {args.reps} (kernel id "
          f"{q.gemm_kernel(dt, args.M, args.K, args.N)}, {len(copies)} copies)", flush=True)


def _counters(args):
    rx = re.compile(args.key)
    per = defaultdict(lambda: defaultdict(float))
    dur = {}
    for r in csv.DictReader(open(args.csv)):
        if not rx.search(r["Kernel_Name"]):
            continue
        d = int(r["Dispatch_Id"])
        per[r["Counter_Name"]][d] += float(r["Counter_Value"])
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    if not per:
        sys.exit("no matching dispatches")
    lines = [f"# {args.title}", "", "Command (from the repository root):", "", "```", args.cmd, "```", "",
             f"{len(dur)} dispatches, mean duration {sum(dur.values()) / len(dur):.2f} us (under the profiler).", "",
             "| counter | mean per dispatch (device total) |", "|---|---:|"]
    for name in sorted(per):
        v = per[name]
        lines.append(f"| {name} | {sum(v.values()) / len(v):,.0f} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def _groups(specs):
    out = []
    for s in specs or []:
        name, rx = s.split("=", 1)
        out.append((name, re.compile(rx)))
    return out


def _stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# {args.title}", "", "Command (from the repository root):", "", "```", args.cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | total ms | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    groups = _groups(args.group)
    if groups:
        lines += ["", "Kernel groups (total time over total calls):", "",
                  "| group | calls | avg us |", "|---|---:|---:|"]
        for name, rx in groups:
            c = sum(int(r["Calls"]) for r in rows if rx.search(r["Name"]))
            t = sum(float(r["TotalDurationNs"]) for r in rows if rx.search(r["Name"]))
            lines.append(f"| {name} | {c} | {t / max(c, 1) / 1e3:.3f} |")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def _per_dispatch(path, counter, rx):
    vals = defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"]):
            vals[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return list(vals.values())


def _traffic(args):
    copy_rx = re.compile(args.calib_regex)
    cf = _per_dispatch(args.calib_fetch, "FETCH_SIZE", copy_rx)
    cw = _per_dispatch(args.calib_write, "WRITE_SIZE", copy_rx)
    if not cf or not cw:
        sys.exit("calibration copy dispatches not found")
    # the copy's last dispatch (warm, steady state)
    kf, kw = args.calib_bytes / cf[-1], args.calib_bytes / cw[-1]
    try:
        with open(args.out) as f:
            db = json.load(f)
    except (OSError, ValueError):
        db = {}
    db["_calibration"] = {"copy_bytes": args.calib_bytes, "fetch_kib_reading": cf[-1], "write_kib_reading": cw[-1],
                          "bytes_per_fetch_unit": kf, "bytes_per_write_unit": kw}
    for spec in args.key:
        name, rx = spec.split("=", 1)
        rx = re.compile(rx)
        f = _per_dispatch(args.fetch, "FETCH_SIZE", rx)
        w = _per_dispatch(args.write, "WRITE_SIZE", rx)
        if not f or not w:
            sys.exit(f"no dispatches for {name}")
        fb = kf * sum(f) / len(f)
        wb = kw * sum(w) / len(w)
        db[name] = {"source_hash": kernel_source_hash(), "dispatches": len(f),
                    "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                    "hbm_bytes_per_launch": round(fb + wb), "kernel_regex": rx.pattern}
        print(name, db[name])
    with open(args.out, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
        fh.write("\n")


def _mfma(args):
    rx = re.compile(args.key)
    per = defaultdict(lambda: defaultdict(float))
    dur = {}
    for r in csv.DictReader(open(args.csv)):
        if not rx.search(r["Kernel_Name"]):
            continue
        d = int(r["Dispatch_Id"])
        name = r["Counter_Name"]
        val = float(r["Counter_Value"])
        per[d][name] += val
        dur[d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not per:
        sys.exit("no matching dispatches")
    rows = []
    for d in sorted(per):
        c = per[d]
        gui = c["GRBM_GUI_ACTIVE"] / args.xccs  # cycles of one die
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * args.simds)
        flops_seen = c["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
        rows.append((d, busy, gui / dur[d] / 1e9, flops_seen / args.flops, args.flops / dur[d] / 1e12,
                     dur[d] * 1e6))
    print("| dispatch | MFMA busy | clock GHz | counted f16 FLOPs / algorithmic | TFLOP/s (algorithmic / duration) | us |")
    print("|---:|---:|---:|---:|---:|---:|")
    for d, busy, ghz, ratio, tf, us in rows:
        print(f"| {d} | {busy * 100:.1f} % | {ghz:.2f} | {ratio:.3f} | {tf:.1f} | {us:.1f} |")
    n = len(rows)
    mean = [sum(r[i] for r in rows) / n for i in range(1, 6)]
    print(f"| mean of {n} | {mean[0] * 100:.1f} % | {mean[1]:.2f} | {mean[2]:.3f} | {mean[3]:.1f} | {mean[4]:.1f} |")


def _valu(args):
    """VALU issue per launch shape: a wave64 VALU instruction occupies a SIMD
    (16 lanes) for 4 cycles, so SQ_INSTS_VALU x 4 / (number of SIMDs) is the
    SIMD time spent issuing VALU work, shown against the dispatch duration at
    the given clocks.  Dispatches are grouped by grid size."""
    rx = re.compile(args.key)
    per = defaultdict(float)
    meta = {}
    for r in csv.DictReader(open(args.csv)):
        if not rx.search(r["Kernel_Name"]) or r["Counter_Name"] != "SQ_INSTS_VALU":
            continue
        d = int(r["Dispatch_Id"])
        per[d] += float(r["Counter_Value"])
        meta[d] = (int(r["Grid_Size"]), int(r["Workgroup_Size"]),
                   (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    if not per:
        sys.exit("no matching dispatches")
    names = dict(spec.split("=", 1) for spec in (args.name or []))
    lo, hi = args.ghz
    groups = defaultdict(list)
    for d in sorted(per):
        grid, wg, us = meta[d]
        cyc = per[d] * 4 / args.simds  # VALU issue cycles per SIMD
        groups[(grid, wg)].append((per[d] / (grid / 64), cyc, us))
    print(f"| launch | workgroups x threads | dispatches | VALU instructions per wavefront | VALU cycles per SIMD "
          f"| that at {hi:g} / {lo:g} GHz, us | dispatch us | VALU share of the dispatch |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    for (grid, wg), rows in groups.items():
        n = len(rows)
        per_wave, cyc, us = (sum(r[i] for r in rows) / n for i in range(3))
        t_hi, t_lo = cyc / (hi * 1e3), cyc / (lo * 1e3)
        label = names.get(str(grid), str(grid))
        print(f"| {label} | {grid // wg} x {wg} | {n} | {per_wave:.0f} | {cyc:.0f} | {t_hi:.2f} / {t_lo:.2f} | {us:.2f} "
              f"| {100 * t_hi / us:.0f}-{100 * t_lo / us:.0f} % |")


def _sweep(args):
    rows = [json.loads(l) for l in open(args.log) if l.startswith("{")]
    out = ["# qmm_gemm over N = 1 .. 512: every dtype at 4096x4096, and the single-configuration workloads", "",
           "Commands (from the repository root): `python3 bench.py --sweep > <log>`, then",
           "`python3 -m gguf_block_quant_qmm_amd.profiling sweep --log <log> --out <this file>`.", "",
           "Each figure is the median (and min) per call over 5 spans of 10 calls, each span after a GPU-side spin that "
           "keeps the",
           "queue ahead of the host; the weights rotate over >= 1 GiB of copies so that every call reads them from HBM.",
           "`path`: f32-gemv = the GEMV's f32 arithmetic for every token (kernel id 100: one launch per token, 101: up "
           "to 4",
           "tokens per weight read), f16-mfma = the matrix cores (ids 0-7 of qmm_gemm_kernel). `repacked`: "
           "qmm_gemm_repacked",
           "on the qmm_repack copy (Q6_K, Q8_0; always the matrix cores).", ""]
    cur = None
    for d in rows:
        if d["workload"] != cur:
            cur = d["workload"]
            out += ["", f"## {cur} ({d['dtype']}, M={d['M']}, K={d['K']})", "",
                    "| N | path | kernel | us median | us min | weight GB/s | TFLOP/s | repacked us (kernel) |",
                    "|---:|---|---:|---:|---:|---:|---:|---:|"]
        r = d.get("repacked")
        rp = f"{r['us_median']:.2f} ({r['kernel_id']})" if r else ""
        out.append(f"| {d['N']} | {d['path']} | {d['kernel_id']} | {d['us_median']:.2f} | {d['us_min']:.2f} | "
                   f"{d['weight_GBps']:.0f} | {d['TFLOPs']:.1f} | {rp} |")
    text = "\n".join(out) + "\n"
    if args.out:
        open(args.out, "w").write(text)
    else:
        print(text, end="")


def _spec(args):
    rows = [json.loads(l) for l in open(args.log) if l.startswith("{")]
    out = ["# Verifying N drafted positions on the Q6_K LM head (128256 x 4096): per-row GEMVs against one call", "",
           "Commands (from the repository root): `python3 bench.py --spec-verify > <log>`, then",
           "`python3 -m gguf_block_quant_qmm_amd.profiling spec --log <log> --out <this file>`.", "",
           "Per N: N separate qmm_gemv calls; one qmm_gemm call (below the crossover the GEMV arithmetic for every "
           "token,",
           "several tokens per weight read, each token with qmm_gemv's bits; above it the matrix cores); and the int8 "
           "form",
           "(qmm_quantize_q8_0 of the N positions + one qmm_gemm_q8act). Each figure is the mean per call over the "
           "timed steps",
           "on rotated weight copies (three copies of the 431 MB head).", "",
           "| N | per-row GEMVs us | one qmm_gemm us | its path | weight GB/s of the one call | int8: quantize + "
           "qmm_gemm_q8act us |",
           "|---:|---:|---:|---|---:|---:|"]
    argmax = None
    for d in rows:
        out.append(f"| {d['N']} | {d['per_row_us']:.1f} | {d['batched_us']:.1f} | {d['batched_path']} | "
                   f"{d['batched_weight_GBps']:.0f} | {d['int8_quantize_plus_q8act_us']:.1f} |")
        argmax = d.get("argmax_us", argmax)
    if argmax is not None:
        out += ["", f"Greedy argmax over the head's outputs (qmm_gemv_argmax, N = 1): {argmax:.1f} us."]
    text = "\n".join(out) + "\n"
    if args.out:
        open(args.out, "w").write(text)
    else:
        print(text, end="")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=512)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="rocprofv3 kernel statistics")
    s.add_argument("--group", action="append")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--calib-fetch", required=True)
    t.add_argument("--calib-write", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--calib-regex", default=r"copy|elementwise")
    t.add_argument("--key", action="append", required=True)
    t.add_argument("--out", default=os.path.join(ROOT, "profiles", "counters.json"))
    g = sub.add_parser("gemm")
    g.add_argument("--dtype", default="Q4_K")
    g.add_argument("--M", type=int, default=14336)
    g.add_argument("--K", type=int, default=4096)
    g.add_argument("--N", type=int, default=32)
    g.add_argument("--reps", type=int, default=20)
    k = sub.add_parser("counters")
    k.add_argument("--csv", required=True)
    k.add_argument("--key", required=True)
    k.add_argument("--title", default="rocprofv3 counters")
    k.add_argument("--cmd", required=True)
    k.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    m.add_argument("--key", required=True)
    m.add_argument("--flops", type=float, required=True)
    m.add_argument("--simds", type=int, default=1024)
    m.add_argument("--xccs", type=int, default=8)
    v = sub.add_parser("valu")
    v.add_argument("--csv", required=True)
    v.add_argument("--key", required=True)
    v.add_argument("--name", action="append", help="GRID=label (grid size in threads)")
    v.add_argument("--simds", type=int, default=1024)
    v.add_argument("--ghz", type=float, nargs=2, default=(2.1, 2.4), help="clock range (low high)")
    w = sub.add_parser("sweep")
    w.add_argument("--log", required=True)
    w.add_argument("--out")
    e = sub.add_parser("spec")
    e.add_argument("--log", required=True)
    e.add_argument("--out")
    a = ap.parse_args(argv)
    {"copy": _copy, "gemm": _gemm, "counters": _counters, "stats": _stats, "traffic": _traffic, "mfma": _mfma,
     "valu": _valu, "sweep": _sweep, "spec": _spec}[a.cmd_name](a)


if __name__ == "__main__":
    main()
