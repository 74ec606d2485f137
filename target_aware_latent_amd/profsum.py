"""Summaries of rocprofv3 output for the measurement records (host-side).

    python -m target_aware_latent_amd.profsum stats KERNEL_STATS_CSV
    python -m target_aware_latent_amd.profsum traffic --fetch FETCH_CSV \\
        --write WRITE_CSV --kernel attn_mfma_kernel --label attention_mfma \\
        --source target_aware_latent_amd/csrc/attention.hip [--out FILE]

`stats` prints the per-kernel table of a `--kernel-trace --stats` run.

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


def traffic(fetch_csv, write_csv, kernel, label, source):
    fd = _dispatches(fetch_csv, "FETCH_SIZE")
    wd = _dispatches(write_csv, "WRITE_SIZE")
    ff, fk = _factor(fd, "FETCH_SIZE")
    wf, wk = _factor(wd, "WRITE_SIZE")
    fsel = [d["v"] for d in fd if kernel in d["name"]]
    wsel = [d["v"] for d in wd if kernel in d["name"]]
    if not fsel or not wsel:
        raise SystemExit(f"no dispatch of {kernel}")
    fetch = sum(fsel) / len(fsel) * 1024.0 * ff
    write = sum(wsel) / len(wsel) * 1024.0 * wf
    return {"kernel": label, "bytes": round(fetch + write), "fetch_bytes": round(fetch),
            "write_bytes": round(write), "dispatches": len(fsel),
            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
            "copy_fetch_kib": fk, "copy_write_kib": wk,
            "fingerprint": fingerprint(source)}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--label", required=True)
    b.add_argument("--source", required=True)
    b.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.csv))
    elif args.cmd == "counters":
        for line in counters(args.csv, args.kernel):
            print(json.dumps(line))
    else:
        rec = traffic(args.fetch, args.write, args.kernel, args.label, args.source)
        text = json.dumps(rec)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
