"""Summaries of rocprofv3 output for the measurement records (host-side).

    python -m target_aware_latent_amd.profsum stats KERNEL_STATS_CSV
    python -m target_aware_latent_amd.profsum phases BENCH_JSON_LINE_FILE
    python -m target_aware_latent_amd.profsum layers KERNEL_TRACE_CSV   (c3 forward)
    python -m target_aware_latent_amd.profsum traffic --fetch FETCH_CSV \\
        --write WRITE_CSV --kernel attn_mfma_kernel --label attention_mfma \\
        --source target_aware_latent_amd/csrc/attention.hip [--out FILE]

`stats` prints the per-kernel table of a `--kernel-trace --stats` run.

`phases` prints the attention kernel's phase table from the JSON line of
`bench.py --attn-phases` (one row per attention launch: workgroups, launch
span, each phase's share of workgroup time, its share of the span in
microseconds and the rate of its algorithmic FLOPs over that estimate).

`counters` sums the SQ counters of `--pmc` runs per kernel and prints the
derived ratios: MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over the SIMD-cycles of
the kernel; GRBM_GUI_ACTIVE is summed over the 8 XCDs, 1024 SIMDs in all),
LDS bank-conflict cycles over LDS active cycles, and VALU instructions per
MFMA instruction.

`traffic` turns two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE, in KiB per
dispatch) of a program that also copied 256 MiB device to device
(bench.py --calibrate-copy) into HBM bytes per launch of one kernel: each
counter is scaled by bytes_copied / counter reading of that copy, then
averaged over the kernel's dispatches. The record carries a fingerprint of
the kernel's source and build flags; bench.py reports the traffic only while
the fingerprint still matches.
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20


def fingerprint(source):
    """sha256 of a kernel source file and the build flags it is compiled with."""
    from . import build
    h = hashlib.sha256()
    with open(source, "rb") as f:
        h.update(f.read())
    for inc in ("common.hpp", "kernels.hpp"):
        with open(os.path.join(HERE, "csrc", inc), "rb") as f:
            h.update(f.read())
    name = os.path.basename(source)
    flags = build.FLAGS + build.FILE_FLAGS.get(name, [])
    flags = [f for i, f in enumerate(flags) if f != "-I" and (i == 0 or flags[i - 1] != "-I")]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def _short(name):
    name = re.sub(r"\(.*$", "", name)
    return name[:100]


def stats(path):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [" calls  total_ms    avg_us    pct  kernel"]
    for r in rows:
        out.append("%6d %9.3f %9.2f %6.2f  %s" % (
            int(r["Calls"]), float(r["TotalDurationNs"]) / 1e6,
            float(r["AverageNs"]) / 1e3, float(r["Percentage"]), _short(r["Name"])))
    return "\n".join(out)


XCDS, SIMDS = 8, 1024   # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def counters(paths, kernels):
    """Per kernel (name filter): counter sums over its dispatches and ratios."""
    tot = {k: collections.defaultdict(float) for k in kernels}
    disp = {k: set() for k in kernels}
    for path in paths:
        for r in csv.DictReader(open(path)):
            for k in kernels:
                if k in r["Kernel_Name"]:
                    tot[k][r["Counter_Name"]] += float(r["Counter_Value"])
                    disp[k].add((path, r["Dispatch_Id"]))
    out = []
    for k in kernels:
        t = tot[k]
        per_run = collections.Counter(path for path, _ in disp[k])
        line = {"kernel": k, "dispatches": max(per_run.values(), default=0)}
        if t.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in t:
            line["mfma_busy"] = round(t["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                      (t["GRBM_GUI_ACTIVE"] / XCDS * SIMDS), 4)
        if t.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in t:
            line["lds_conflict_cycles"] = round(t["SQ_LDS_BANK_CONFLICT"] / t["SQ_LDS_IDX_ACTIVE"], 4)
        if t.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in t:
            line["valu_per_mfma"] = round(t["SQ_INSTS_VALU"] / t["SQ_INSTS_MFMA"], 3)
        line["sums"] = {c: v for c, v in sorted(t.items())}
        out.append(line)
    return out


def _dispatches(path, counter):
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = per[int(r["Dispatch_Id"])]
        d["name"] = r["Kernel_Name"]
        d["v"] = d.get("v", 0.0) + float(r["Counter_Value"])
    return list(per.values())


def _factor(disp, counter):
    """bytes copied / counter bytes of the largest device-to-device copy."""
    copies = [d for d in disp if "copyBuffer" in d["name"]]
    if not copies:
        raise SystemExit(f"no copy dispatch in the {counter} run (use --calibrate-copy)")
    kib = max(d["v"] for d in copies)
    return COPY_BYTES / (kib * 1024.0), kib


def traffic(fetch_csv, write_csv, kernel, label, source, launches=None):
    fd = _dispatches(fetch_csv, "FETCH_SIZE")
    wd = _dispatches(write_csv, "WRITE_SIZE")
    ff, fk = _factor(fd, "FETCH_SIZE")
    wf, wk = _factor(wd, "WRITE_SIZE")
    fsel = [d["v"] for d in fd if kernel in d["name"]]
    wsel = [d["v"] for d in wd if kernel in d["name"]]
    if not fsel or not wsel:
        raise SystemExit(f"no dispatch of {kernel}")
    # per launch: over the dispatches, or over `launches` when one launch
    # of the timing label takes several dispatches (split-K products)
    nf = launches or len(fsel)
    nw = launches or len(wsel)
    fetch = sum(fsel) / nf * 1024.0 * ff
    write = sum(wsel) / nw * 1024.0 * wf
    return {"kernel": label, "bytes": round(fetch + write), "fetch_bytes": round(fetch),
            "write_bytes": round(write), "dispatches": len(fsel), "launches": nf,
            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
            "copy_fetch_kib": fk, "copy_write_kib": wk,
            "fingerprint": fingerprint(source)}


def launches(path, first="plan_layer_kernel"):
    """Median duration of each dispatch position of one forward pass, from a
    rocprofv3 kernel-trace CSV: the passes start at each dispatch of `first`
    and those with the most common number of dispatches are aligned by
    position. Returns [(position, kernel symbol, grid, median us)]."""
    import statistics
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if first in r["Kernel_Name"]]
    passes = [rows[a:b] for a, b in zip(starts, starts[1:])]
    if not passes:
        return []
    n = max(set(map(len, passes)), key=[len(p) for p in passes].count)
    passes = [p for p in passes if len(p) == n]
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    return [(j, passes[0][j]["Kernel_Name"], passes[0][j]["Grid_Size_X"],
             statistics.median(dur(p[j]) for p in passes)) for j in range(n)]


def layers(path):
    """Per-layer table of one c3 forward (B=64, L=1600, d=512, 8x64 heads,
    r=128, pyramid 1600-800-400-200-100-50, 4-seed readout, no candidates)
    from the median dispatch durations of `launches`. The dispatches of a
    pass are: the plan and the query map, the layer-1 norm; per layer W_dkv,
    W_uq, the attention, W_o, W1, W2; then the seeds' broadcast and the
    readout's pre-norm, its six launches (W2 a split-K pair) and W_p (a
    split-K pair). Rates are each launch's algorithmic FLOPs (2MNK; for the
    attention the allowed pairs x 8 heads x 4r plus both absorptions) over
    its median duration."""
    rows = launches(path)
    t = [r[3] for r in rows]
    names = [r[1] for r in rows]
    B, d, h, dk, r, dff = 64, 512, 8, 64, 128, 2048
    shapes = [(1600, 1600), (1600, 800), (800, 400), (400, 200), (200, 100), (100, 50), (50, 4)]
    att = [3 + 6 * l + 2 for l in range(6)] + [3 + 6 * 6 + 2 + 2]
    if len(t) != 50 or any("attn_mfma_kernel" not in names[i] for i in att):
        raise SystemExit("not the c3 forward's dispatch sequence")
    out, idx, total, pre = [], 3, 0.0, []
    for li, (K, n) in enumerate(shapes):
        ro = li == 6
        if ro:
            pre = t[idx:idx + 2]
            idx += 2
        times = []
        for j in range(6):
            if ro and j == 5:
                times.append(t[idx] + t[idx + 1])
                idx += 2
            else:
                times.append(t[idx])
                idx += 1
        pairs = n * K if ro else n * K - n * (n - 1) // 2
        fl = [2 * B * K * d * r, 2 * B * n * d * h * dk,
              B * pairs * h * 4 * r + 2 * 2 * B * n * h * dk * r,
              2 * B * n * h * dk * d, 2 * B * n * d * dff, 2 * B * n * dff * d]
        rates = [f / (x * 1e-6) / 1e12 for f, x in zip(fl, times)]
        total += sum(times)
        lab = "readout" if ro else f"L{li + 1}"
        out.append(f"{lab:<7}{K:>9}/{n:>6}          | " + " ".join(f"{x:6.1f}" for x in times[:2]) +
                   f"  {times[2]:7.1f}  " + " ".join(f"{x:6.1f}" for x in times[3:]) +
                   f" | {sum(times):8.1f} us")
        out.append(" " * 9 + "TFLOP/s              | " + " ".join(f"{x:6.0f}" for x in rates[:2]) +
                   f"  {rates[2]:7.0f}  " + " ".join(f"{x:6.0f}" for x in rates[3:]) + " |")
    out.append(f"stack + readout layers: {total:.1f} us; plan {t[0] + t[1]:.1f} us, layer-1 norm "
               f"{t[2]:.1f} us, readout broadcast {pre[0]:.1f} us and pre-norm {pre[1]:.1f} us, "
               f"W_p {t[idx] + t[idx + 1]:.1f} us")
    out.append(f"all launches of the pass: {sum(t):.1f} us")
    return "\n".join(out)


def phases(path):
    """The phase tables of a bench.py --attn-phases / --gemm-phases line."""
    with open(path) as f:
        rec = json.loads(f.read().strip().splitlines()[-1])
    rows = ["                       | share of workgroup time | us (span x share)     | TFLOP/s",
            "launch  workgroups   span_us | prologue loop epilogue | prologue loop epilogue | "
            "prologue loop epilogue"]
    for e in rec.get("attention_phases") or []:
        layer = e.get("layer", "?")
        name = f"L{layer}" if isinstance(layer, int) else str(layer)
        rows.append(
            f"{name:8s}{int(e['workgroups']):6d} {e['span_us']:9.1f} |"
            f" {100 * e['prologue_share']:7.1f}% {100 * e['loop_share']:4.1f}% {100 * e['epilogue_share']:6.1f}% |"
            f" {e['prologue_us_est']:8.1f} {e['loop_us_est']:5.1f} {e['epilogue_us_est']:8.1f} |"
            f" {e['prologue_tflops_est']:8.0f} {e['loop_tflops_est']:4.0f} {e['epilogue_tflops_est']:8.0f}")
    g = rec.get("gemm_phases") or []
    if g:
        rows += ["", "                                | share of workgroup time  | us (span x share)      | K loop",
                 "product layer  workgroups span_us | first   loop   epilogue | first   loop  epilogue | TFLOP/s"]
        for e in g:
            rows.append(
                f"{e['product']:8s}{e['layer']:3d} {int(e['workgroups']):9d} {e['span_us']:8.1f} |"
                f" {100 * e['first_share']:5.1f}% {100 * e['loop_share']:5.1f}% {100 * e['epilogue_share']:7.1f}% |"
                f" {e['first_us_est']:6.1f} {e['loop_us_est']:6.1f} {e['epilogue_us_est']:8.1f} |"
                f" {e['loop_tflops_est']:7.0f}")
    return "\n".join(rows)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    t = sub.add_parser("launches")
    t.add_argument("csv")
    ly = sub.add_parser("layers")
    ly.add_argument("csv")
    ph = sub.add_parser("phases")
    ph.add_argument("json")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--label", required=True)
    b.add_argument("--source", required=True)
    b.add_argument("--launches", type=int, default=None,
                   help="launches the dispatches make up (default: one each)")
    b.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.csv))
    elif args.cmd == "phases":
        print(phases(args.json))
    elif args.cmd == "layers":
        print(layers(args.csv))
    elif args.cmd == "launches":
        for j, name, grid, us in launches(args.csv):
            print(f"{j:4d} {us:9.1f} us  grid {grid:>9s}  {name[:100]}")
    elif args.cmd == "counters":
        for line in counters(args.csv, args.kernel):
            print(json.dumps(line))
    else:
        rec = traffic(args.fetch, args.write, args.kernel, args.label, args.source,
                      args.launches)
        text = json.dumps(rec)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
