"""Summaries of rocprofv3 output for the kernels of this library (host-side text processing).

    python -m tiled_attention_10_amd.profiling stats DIR
        Markdown table of DIR's kernel statistics (``*_kernel_stats.csv`` of a
        ``rocprofv3 --kernel-trace --stats --output-format csv`` run).

    python -m tiled_attention_10_amd.profiling blocks DIR [--kernel SUBSTR] [--min-calls N]
        The same run's dispatches in launch order, grouped into contiguous blocks of
        one kernel (``*_kernel_trace.csv``), with each block's count and durations.
        bench.py launches each workload's kernel as one block, so a block separates
        one leg of the benchmark from the others that use the same kernel instance.

    python -m tiled_attention_10_amd.profiling counters DIR [DIR ...]
        SQ counter summary of the attention kernels from rocprofv3 --pmc runs of the
        same command (``*_counter_collection.csv``; each directory one pass): the
        longest dispatch of each kernel, matrix-core busy share, LDS bank-conflict
        share, VALU and transcendental instructions per MFMA, and the raw values.

    python -m tiled_attention_10_amd.profiling traffic --fetch DIR --write DIR
            --copy-fetch DIR --copy-write DIR --workload NAME [--record]
        HBM bytes per dispatch of each attention kernel from two counter runs
        (``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` of the same
        command), each scaled by what the same counter reads for a plain device
        copy of known size (``bench.py --copy-calibration`` under the same
        counter).  With --record the figures go to profiles/traffic.json under
        "<kernel>:<workload>" together with the hash of the kernel's sources, so
        bench.py reports them only while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30          # bench.py --copy-calibration moves 1 GiB per copy


def _one(directory: str, suffix: str) -> str:
    found = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not found:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return found[0]


def short_name(kernel: str) -> str:
    """``void tattn::(anonymous namespace)::attn_fwd16_kernel<...>(...)`` -> ``attn_fwd16_kernel<...>``."""
    name = kernel.split("(anonymous namespace)::", 1)[-1]
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("tattn::", "")


def stats(directory: str) -> str:
    rows = list(csv.DictReader(open(_one(directory, "kernel_stats.csv"))))
    out = ["| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    return "\n".join(out)


def blocks(directory: str, kernel: str | None = None, min_calls: int = 1) -> str:
    rows = list(csv.DictReader(open(_one(directory, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    runs = []
    for r in rows:
        name = short_name(r["Kernel_Name"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if runs and runs[-1][0] == name:
            runs[-1][1].append(dur)
        else:
            runs.append((name, [dur]))
    out = ["| block | kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|---|"]
    for i, (name, d) in enumerate(runs):
        if (kernel and kernel not in name) or len(d) < min_calls:
            continue
        out.append(f"| {i} | `{name}` | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    return "\n".join(out)


def counter_means(directory: str, counter: str) -> dict:
    """Mean value of ``counter`` per dispatch and the dispatch count, by kernel name."""
    per = {}
    for r in csv.DictReader(open(_one(directory, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in per.items()}


def counters(directories) -> str:
    """Markdown summary of the longest dispatch of each attention kernel (the benchmarked
    workload's, where a run also launches the kernel on smaller ones) over the counter passes."""
    vals = {}
    for d in directories:
        per = {}
        for r in csv.DictReader(open(_one(d, "counter_collection.csv"))):
            name = short_name(r["Kernel_Name"])
            if not name.startswith("attn_"):
                continue
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            cv = per.setdefault(name, {}).setdefault(int(r["Dispatch_Id"]), [dur, {}])[1]
            cv[r["Counter_Name"]] = cv.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        for name, disp in per.items():
            vals.setdefault(name, {}).update(max(disp.values(), key=lambda x: x[0])[1])
    out = ["| kernel | XCD active cycles | MFMA busy | LDS bank-conflict cycles / LDS active cycles | "
           "non-MFMA VALU instructions per MFMA | transcendental per MFMA | SQ_WAVES |", "|---|---|---|---|---|---|---|"]
    for name, v in vals.items():
        xcd = v.get("GRBM_GUI_ACTIVE", float("nan")) / 8
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (xcd * 1024)
        conf = v.get("SQ_LDS_BANK_CONFLICT", float("nan")) / v.get("SQ_LDS_IDX_ACTIVE", float("nan"))
        mf = v.get("SQ_INSTS_MFMA", float("nan"))
        valu = (v.get("SQ_INSTS_VALU", float("nan")) - mf) / mf
        trans = v.get("SQ_INSTS_VALU_TRANS_F32", float("nan")) / mf
        out.append(f"| {name} | {xcd:.4g} | {100 * busy:.1f} % | {100 * conf:.2f} % | {valu:.2f} | {trans:.2f} | "
                   f"{v.get('SQ_WAVES', float('nan')):.0f} |")
    names = list(vals)
    out += ["", "| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for c in sorted({c for v in vals.values() for c in v}):
        out.append(f"| {c} | " + " | ".join(f"{vals[n].get(c, float('nan')):.4g}" for n in names) + " |")
    return "\n".join(out)


def copy_factor(directory: str, counter: str) -> float:
    """Counter KiB per KiB actually moved, from the copy calibration run (the dispatch with
    the largest count is the 1 GiB copy)."""
    means = counter_means(directory, counter)
    best = max(means.values(), key=lambda x: x[0])[0]
    return best / (COPY_BYTES / 1024)


def traffic(fetch: str, write: str, copy_fetch: str, copy_write: str, workload: str) -> dict:
    sys.path.insert(0, ROOT)
    from bench import KERNEL_SOURCES, source_hash

    ff, wf = copy_factor(copy_fetch, "FETCH_SIZE"), copy_factor(copy_write, "WRITE_SIZE")
    fm, wm = counter_means(fetch, "FETCH_SIZE"), counter_means(write, "WRITE_SIZE")
    out = {"_calibration": {"copy_bytes": COPY_BYTES, "FETCH_SIZE_kib_per_true_kib": round(ff, 4),
                            "WRITE_SIZE_kib_per_true_kib": round(wf, 4)}}
    for kernel in KERNEL_SOURCES:
        fk = [k for k in fm if f"::{kernel}<" in k]
        wk = [k for k in wm if f"::{kernel}<" in k]
        if not fk or not wk:
            continue
        # one instance per run (the workload's): the most dispatched one
        fkn = max(fk, key=lambda k: fm[k][1])
        wkn = max(wk, key=lambda k: wm[k][1])
        fb = fm[fkn][0] / ff * 1024
        wb = wm[wkn][0] / wf * 1024
        out[f"{kernel}:{workload}"] = {"source_sha": source_hash(kernel), "instance": short_name(fkn),
                                      "fetch_kib_raw": round(fm[fkn][0], 1), "write_kib_raw": round(wm[wkn][0], 1),
                                      "fetch_bytes": int(fb), "write_bytes": int(wb), "traffic_bytes": int(fb + wb),
                                      "dispatches": [fm[fkn][1], wm[wkn][1]]}
        if kernel == "attn_decode_split_kernel":
            # a decode step is the split kernel and its merge kernel: record the step's bytes
            mf = [k for k in fm if "::attn_decode_merge_kernel<" in k]
            mw = [k for k in wm if "::attn_decode_merge_kernel<" in k]
            if mf and mw:
                mfb, mwb = fm[mf[0]][0] / ff * 1024, wm[mw[0]][0] / wf * 1024
                e = out[f"{kernel}:{workload}"]
                e["scope"] = "one decode step: attn_decode_split_kernel + attn_decode_merge_kernel"
                e["merge_fetch_kib_raw"], e["merge_write_kib_raw"] = round(fm[mf[0]][0], 1), round(wm[mw[0]][0], 1)
                e["fetch_bytes"], e["write_bytes"] = int(fb + mfb), int(wb + mwb)
                e["traffic_bytes"] = int(fb + mfb + wb + mwb)
    return out


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    b = sub.add_parser("blocks")
    b.add_argument("dir")
    b.add_argument("--kernel", default=None)
    b.add_argument("--min-calls", type=int, default=1)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload"):
        t.add_argument(a, required=True)
    t.add_argument("--record", action="store_true")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.dir))
        return
    if args.cmd == "counters":
        print(counters(args.dirs))
        return
    if args.cmd == "blocks":
        print(blocks(args.dir, args.kernel, args.min_calls))
        return
    res = traffic(args.fetch, args.write, args.copy_fetch, args.copy_write, args.workload)
    print(json.dumps(res, indent=1))
    if args.record:
        rec = json.load(open(TRAFFIC)) if os.path.exists(TRAFFIC) else {}
        rec.update(res)
        with open(TRAFFIC, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")


if __name__ == "__main__":
    main()
