"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m clustered_block_sparse_amd.profiling trace STATS_CSV --title T --cmd C
        Markdown table (kernel, calls, total ms, average us, %) from the
        kernel_stats.csv of `rocprofv3 --kernel-trace --stats --output-format csv`.

    python -m clustered_block_sparse_amd.profiling bench JSONL... --title T --cmd C
        Markdown table of bench.py result lines (one JSON object per line,
        other lines ignored): per run the workload, density, ms per layer,
        the stage breakdown, the attention kernels' rate and the dense
        comparison.

    python -m clustered_block_sparse_amd.profiling counters CSV --title T --cmd C
        Markdown table of per-dispatch means of every counter in a
        counter_collection.csv of `rocprofv3 --pmc`, one row per kernel.

    python -m clustered_block_sparse_amd.profiling kernel_traffic --fetch CSV --write CSV \
            --stats KERNEL_STATS_CSV --copy-bytes B --title T --cmd C
        Markdown table of every kernel's HBM traffic per dispatch (the two
        counters, copy-calibrated as below), its average duration from a
        kernel trace of the same command, and the rate they give.

    python -m clustered_block_sparse_amd.profiling traffic --fetch CSV --write CSV \
            --kernel NAME --copy-bytes B --workload W --out JSON [--cmd C]
        HBM bytes per launch of kernel NAME from two counter passes
        (`rocprofv3 --pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`, of a bench run
        with --copy-probe).  Each counter reads in KiB per dispatch; it is
        scaled by what it reads for the probe's device copies of B bytes each
        (B read and B written), which calibrates the counter against a transfer
        of known size.  The JSON keeps the sha256 of the attention kernel
        source it was measured on; bench.py reports the figure only while the
        source is unchanged.

Only summarises files; nothing here touches the GPU.
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

HERE = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCE = os.path.join(HERE, "csrc", "k_attn.hip")


def source_hash(path: str = ATTN_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(n: str) -> str:
    if n.startswith("void at::") or n.startswith("at::") or n.startswith("Cijk_"):
        return "torch (input generation, bench bookkeeping, dense SDPA)"
    n = n.replace("(anonymous namespace)::", "").replace("sa::", "").replace("void ", "")
    n = re.sub(r"\(.*", "", n)
    n = n.replace("HIP_vector_type<unsigned int, 4u>", "uint4").replace("unsigned short", "bf16")
    return n.strip() or "(unnamed)"


def trace_table(stats_csv: str, title: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    agg: dict[str, list[float]] = {}
    for r in rows:
        s = short_name(r["Name"])
        c, t = int(r["Calls"]), float(r["TotalDurationNs"])
        a = agg.setdefault(s, [0, 0.0])
        a[0] += c
        a[1] += t
    total = sum(t for _, t in agg.values()) or 1.0
    out = [f"# {title}", "", "Command (from the repo root, on the MI355X):", "", "```", cmd, "```", "",
           "| kernel | calls | total ms | avg us | % |", "|---|---|---|---|---|"]
    for s, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {s} | {c} | {t / 1e6:.2f} | {t / c / 1e3:.1f} | {100 * t / total:.1f} |")
    return "\n".join(out) + "\n"


def bench_table(paths: list[str], title: str, cmd: str) -> str:
    rows = []
    for path in paths:
        for line in open(path):
            line = line.strip()
            if line.startswith("{"):
                try:
                    rows.append(json.loads(line))
                except ValueError:
                    pass
    out = [f"# {title}", "", "Commands (from the repo root, on the MI355X):", "", "```", cmd, "```", "",
           "| workload | H x N x d | density | cache | ms/layer | step median / min (ms) | cluster | permute V | "
           "select | attention call | attention kernels (ms) | TFLOP/s (frac) | dense own / SDPA (ms) | "
           "speedup | value TFLOP/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        c, st, rf = r["config"], r.get("stage_ms", {}), r["roofline"]
        ev = r.get("step_ms_events", {})
        cl = st.get("cluster_qk", st.get("cluster_q", 0.0) + st.get("cluster_k", 0.0))
        dense = "/".join(f"{x:.1f}" if x else "-" for x in (r.get("dense_ms_own_kernel"), r.get("dense_ms_torch_sdpa")))
        sp = r.get("speedup_vs_dense")
        out.append(
            f"| {c['workload']} | {c['heads']} x {c['n']} x {c['d']} | {100 * c['density']:.2f}% | "
            f"{r.get('cache', 'warm').split(':')[0]} | {r['ms_per_step']:.2f} | "
            f"{ev.get('median', float('nan')):.2f} / {ev.get('min', float('nan')):.2f} | {cl:.2f} | "
            f"{st.get('permute_v', 0.0):.2f} | {st.get('select', 0.0):.2f} | {st.get('attention', 0.0):.2f} | "
            f"{r['attention_kernel_ms']:.2f} | {rf['achieved']:.0f} ({rf['frac']:.3f}) | {dense} | "
            f"{'%.2fx' % sp if sp else '-'} | {r['value']:.0f} |")
    return "\n".join(out) + "\n"


def counters_table(counter_csv: str, title: str, cmd: str) -> str:
    acc: dict[tuple[str, str], dict[str, float]] = defaultdict(lambda: defaultdict(float))
    names: set[str] = set()
    for r in csv.DictReader(open(counter_csv)):
        k = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        names.add(r["Counter_Name"])
    per: dict[str, list[dict[str, float]]] = defaultdict(list)
    for (kn, _), d in acc.items():
        per[kn].append(d)
    cols = sorted(names)
    out = [f"# {title}", "", "Command (from the repo root, on the MI355X):", "", "```", cmd, "```", "",
           "Per-dispatch means.", "", "| kernel | dispatches | " + " | ".join(cols) + " |",
           "|---|---|" + "---|" * len(cols)]
    for kn, ds in sorted(per.items()):
        vals = [sum(d.get(c, 0.0) for d in ds) / len(ds) for c in cols]
        out.append(f"| {kn} | {len(ds)} | " + " | ".join(f"{v:.4g}" for v in vals) + " |")
    return "\n".join(out) + "\n"


def per_dispatch(counter_csv: str, counter: str) -> dict[str, list[float]]:
    """kernel short name -> per-dispatch totals of `counter` (rows of one
    dispatch, e.g. per hardware block, are summed)."""
    acc: dict[tuple[str, str], float] = defaultdict(float)
    for r in csv.DictReader(open(counter_csv)):
        if r.get("Counter_Name") != counter:
            continue
        acc[(short_name(r["Kernel_Name"]), r["Dispatch_Id"])] += float(r["Counter_Value"])
    out: dict[str, list[float]] = defaultdict(list)
    for (k, _), v in acc.items():
        out[k].append(v)
    return out


def copy_reading(d: dict[str, list[float]]) -> float:
    """Mean counter value of the probe's large copies: the copy-kernel
    dispatches within 10% of the largest one."""
    vals = [v for k, vs in d.items() if "copyBuffer" in k or "copy_kernel" in k for v in vs]
    if not vals:
        raise SystemExit("no copy kernel dispatches in the counter file (run the bench with --copy-probe)")
    top = max(vals)
    big = [v for v in vals if v >= 0.9 * top]
    return sum(big) / len(big)


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int) -> dict:
    f, w = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    if kernel not in f or kernel not in w:
        raise SystemExit(f"kernel {kernel!r} not found; kernels: {sorted(f)}")
    fk, wk = sum(f[kernel]) / len(f[kernel]), sum(w[kernel]) / len(w[kernel])
    f_scale = copy_bytes / (copy_reading(f) * 1024.0)
    w_scale = copy_bytes / (copy_reading(w) * 1024.0)
    return {"kernel": kernel, "dispatches": len(f[kernel]),
            "fetch_kib": fk, "write_kib": wk, "fetch_scale": f_scale, "write_scale": w_scale,
            "read_bytes": fk * 1024.0 * f_scale, "write_bytes": wk * 1024.0 * w_scale,
            "bytes_per_launch": fk * 1024.0 * f_scale + wk * 1024.0 * w_scale}


def kernel_traffic_table(fetch_csv: str, write_csv: str, stats_csv: str, copy_bytes: int, title: str,
                         cmd: str) -> str:
    f, w = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    fs = copy_bytes / (copy_reading(f) * 1024.0)
    wsc = copy_bytes / (copy_reading(w) * 1024.0)
    dur: dict[str, list[float]] = {}
    for r in csv.DictReader(open(stats_csv)):
        s = short_name(r["Name"])
        a = dur.setdefault(s, [0, 0.0])
        a[0] += int(r["Calls"])
        a[1] += float(r["TotalDurationNs"])
    rows = []
    for k in sorted(set(f) & set(w)):
        if k.startswith("torch") or "copyBuffer" in k or "fillBuffer" in k or k not in dur:
            continue
        rd = sum(f[k]) / len(f[k]) * 1024.0 * fs
        wr = sum(w[k]) / len(w[k]) * 1024.0 * wsc
        us = dur[k][1] / dur[k][0] / 1e3
        rows.append((dur[k][1], f"| {k} | {len(f[k])} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | {us:.1f} | "
                                f"{(rd + wr) / (us * 1e-6) / 1e12:.2f} |"))
    out = [f"# {title}", "", "Commands (from the repo root, on the MI355X):", "", "```", cmd, "```", "",
           f"Counters scaled by the readings of 1 GiB device copies: FETCH_SIZE x {fs:.3f}, WRITE_SIZE x {wsc:.3f}.",
           "Rows by total time in the trace.", "",
           "| kernel | dispatches | read MB / dispatch | written MB / dispatch | avg us (trace) | TB/s |",
           "|---|---|---|---|---|---|"]
    out += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    b = sub.add_parser("bench")
    b.add_argument("jsonl", nargs="+")
    b.add_argument("--title", required=True)
    b.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    kt = sub.add_parser("kernel_traffic")
    kt.add_argument("--fetch", required=True)
    kt.add_argument("--write", required=True)
    kt.add_argument("--stats", required=True)
    kt.add_argument("--copy-bytes", type=int, required=True)
    kt.add_argument("--title", required=True)
    kt.add_argument("--cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    if a.cmd_name == "trace":
        sys.stdout.write(trace_table(a.stats_csv, a.title, a.cmd))
    elif a.cmd_name == "bench":
        sys.stdout.write(bench_table(a.jsonl, a.title, a.cmd))
    elif a.cmd_name == "counters":
        sys.stdout.write(counters_table(a.csv, a.title, a.cmd))
    elif a.cmd_name == "kernel_traffic":
        sys.stdout.write(kernel_traffic_table(a.fetch, a.write, a.stats, a.copy_bytes, a.title, a.cmd))
    else:
        res = traffic(a.fetch, a.write, a.kernel, a.copy_bytes)
        res.update({"workload": a.workload, "source_sha256": source_hash(), "command": a.cmd})
        with open(a.out, "w") as fh:
            json.dump(res, fh, indent=1)
            fh.write("\n")
        print(json.dumps(res))


if __name__ == "__main__":
    main()
