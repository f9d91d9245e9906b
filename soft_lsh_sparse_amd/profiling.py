"""Summaries of rocprofv3 output for the decode kernels.

Two kinds of text summary are written under profiles/ (each names the full
command that produced its input):

* a kernel-trace summary (``rocprofv3 --kernel-trace --stats``): calls and
  average / min / max duration of every kernel of this library;
* a counter summary: the mean per dispatch of several ``--pmc`` counters
  (one run) for every kernel of this library, e.g. the LDS and VALU
  instruction counts and LDS bank-conflict cycles of the score kernel, or
  the MFMA counters of the hash kernel;
* an HBM-traffic summary: the ``FETCH_SIZE`` and ``WRITE_SIZE`` counters
  (KiB per dispatch, one ``--pmc`` run each) of every kernel, each scaled by
  the factor that turns the same counter into the known byte count of a
  plain device-to-device copy, so that ``traffic = FETCH * f_fetch +
  WRITE * f_write`` bytes per launch.

The traffic summary records a SHA-256 digest of the sources every kernel is
compiled from; ``load_traffic`` returns None for a kernel whose sources have
changed since, so a stale counter reading is never reported as current.

Usage::

    python -m soft_lsh_sparse_amd.profiling trace <stats.csv> <out.md> --command "..."
    python -m soft_lsh_sparse_amd.profiling counters <pmc.csv> <out.md> --command "..."
    python -m soft_lsh_sparse_amd.profiling traffic --fetch <csv> --write <csv> \\
        --copy-fetch <csv> --copy-write <csv> --copy-bytes N --out <md> \\
        --command "..." --copy-command "..."
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel -> sources it is compiled from (besides the shared headers)
KERNEL_SOURCES = {
    "hash_keys_bf16_kernel": ["hash_keys.hip"],
    "hash_keys_f32_kernel": ["hash_keys.hip"],
    "hash_prep_kernel": ["hash_keys.hip"],
    "hash_settle_kernel": ["hash_keys.hip"],
    "bucket_probs_kernel": ["bucket_probs.hip", "soft_prob.hpp"],
    "score_kernel_rot": ["score.hip", "radix.hpp"],
    "score_kernel_generic": ["score.hip", "radix.hpp"],
    "zero_u32_kernel": ["topk.hip", "radix.hpp"],
    "iota_rows_kernel": ["topk.hip", "radix.hpp"],
    "topk_hist_kernel": ["topk.hip", "radix.hpp"],
    "topk_filter_kernel": ["topk.hip", "radix.hpp"],
    "topk_refine_kernel": ["topk.hip", "radix.hpp"],
    "topk_gather_kernel": ["topk.hip", "radix.hpp"],
    "topk_select_kernel": ["topk.hip", "radix.hpp"],
    "sparse_attn_kernel": ["sparse_attn.hip"],
    "attn_merge_kernel": ["sparse_attn.hip"],
}
SHARED_SOURCES = ["common.hpp", "kernels.hpp", "api.hip"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"

_NAME = re.compile(r"socket_lsh::\(anonymous namespace\)::(\w+)")


def short_name(full: str) -> str | None:
    """The library kernel's base name (template arguments dropped), the copy
    kernel's name, or None for anything else."""
    m = _NAME.search(full)
    if m:
        return m.group(1)
    if COPY_KERNEL in full:
        return COPY_KERNEL
    return None


def instance_name(full: str) -> str | None:
    """short_name plus the template arguments of the instance, if any."""
    n = short_name(full)
    if n is None:
        return None
    m = re.search(r"::\w+(<[^()]*?>)?\(", full)
    return n + (m.group(1) if m and m.group(1) else "")


def canonical(name: str) -> str:
    """Decode-stage name used by the benchmark (score_kernel_rot and
    score_kernel_generic are both the score kernel)."""
    return "score_kernel" if name.startswith("score_kernel") else name


def source_digest(kernel: str) -> str:
    files = KERNEL_SOURCES.get(kernel)
    if files is None and kernel == "score_kernel":
        files = ["score.hip", "radix.hpp"]
    if files is None:
        raise KeyError(kernel)
    h = hashlib.sha256()
    for f in sorted(set(files + SHARED_SOURCES)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def kernel_stats(stats_csv: str):
    """rows of (kernel, calls, avg_us, min_us, max_us) from run_kernel_stats.csv"""
    out = []
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            n = instance_name(r["Name"])
            if n is None or n == COPY_KERNEL:
                continue
            out.append((n, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                        float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    return out


def counter_means(pmc_csv: str, counter: str):
    """kernel -> (mean counter value per dispatch, dispatches)"""
    vals = collections.defaultdict(list)
    with open(pmc_csv) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            n = short_name(r["Kernel_Name"])
            if n is not None:
                vals[n].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def counter_table(pmc_csv: str):
    """kernel instance (with its template arguments) -> {counter: mean value
    per dispatch}, and dispatches per instance (the smallest count over its
    counters)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(pmc_csv) as fh:
        for r in csv.DictReader(fh):
            n = instance_name(r["Kernel_Name"])
            if n is None or n == COPY_KERNEL:
                continue
            vals[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    means = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    counts = {k: min(len(v) for v in cs.values()) for k, cs in vals.items()}
    return means, counts


def write_counter_summary(pmc_csv: str, out_md: str, command: str, title: str,
                          notes: str = "") -> dict:
    means, counts = counter_table(pmc_csv)
    counters = sorted({c for cs in means.values() for c in cs})
    lines = [f"# {title}", "", "Command (from the repository root on the GPU host):", "",
             "```", command, "```", "",
             "Mean value per dispatch of each counter (summed over the whole device).", ""]
    if notes:
        lines += [notes, ""]
    lines += ["| kernel | dispatches | " + " | ".join(counters) + " |",
              "|---|---|" + "---|" * len(counters)]
    for k in sorted(means):
        row = [f"{means[k].get(c, float('nan')):.4g}" for c in counters]
        lines.append(f"| `{k}` | {counts[k]} | " + " | ".join(row) + " |")
    data = {"kernels": {k: {"dispatches": counts[k], **{c: round(v, 1) for c, v in means[k].items()}}
                        for k in sorted(means)}}
    lines += ["", "```json", json.dumps(data, indent=1), "```", ""]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))
    return data


def write_trace_summary(stats_csv: str, out_md: str, command: str, title: str) -> None:
    rows = kernel_stats(stats_csv)
    lines = [f"# {title}", "", "Command (from the repository root on the GPU host):", "",
             "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, avg, lo, hi in sorted(rows, key=lambda r: -r[2] * r[1]):
        lines.append(f"| `{name}` | {calls} | {avg:.2f} | {lo:.2f} | {hi:.2f} |")
    lines.append("")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))


def write_traffic_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv,
                          copy_bytes, out_md, command, copy_command, title) -> dict:
    fetch = counter_means(fetch_csv, "FETCH_SIZE")
    write = counter_means(write_csv, "WRITE_SIZE")
    cf = counter_means(copy_fetch_csv, "FETCH_SIZE")[COPY_KERNEL][0]
    cw = counter_means(copy_write_csv, "WRITE_SIZE")[COPY_KERNEL][0]
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k == COPY_KERNEL or (k not in KERNEL_SOURCES and not k.startswith("score_kernel")):
            continue
        fk, nf = fetch[k]
        wk, nw = write[k]
        kernels[canonical(k)] = {
            "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
            "dispatches": min(nf, nw),
            "traffic_bytes": int(round(fk * 1024 * f_fetch + wk * 1024 * f_write)),
            "source_sha256": source_digest(k),
        }
    data = {"copy_bytes": copy_bytes, "copy_fetch_kib": round(cf, 1),
            "copy_write_kib": round(cw, 1), "f_fetch": round(f_fetch, 4),
            "f_write": round(f_write, 4), "kernels": kernels}
    lines = [f"# {title}", "",
             "Counters per dispatch from two `rocprofv3 --pmc` runs (FETCH_SIZE, then",
             "WRITE_SIZE, KiB), each scaled by the factor that maps the same counter onto",
             f"a plain {copy_bytes}-byte device copy (`{COPY_KERNEL}`):",
             f"f_fetch = {f_fetch:.4f} (copy read {cf:.1f} KiB), "
             f"f_write = {f_write:.4f} (copy wrote {cw:.1f} KiB).", "",
             "Commands (from the repository root on the GPU host; COUNTER is FETCH_SIZE,",
             "then WRITE_SIZE, one run each):", "", "```", command, copy_command, "```", "",
             "| kernel | FETCH KiB | WRITE KiB | traffic MB per launch | dispatches |",
             "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append(f"| `{k}` | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} | "
                     f"{v['traffic_bytes'] / 1e6:.2f} | {v['dispatches']} |")
    lines += ["", "Machine-readable copy (the benchmark reads `traffic_bytes` from here",
              "while `source_sha256` still matches the kernel's sources):", "",
              "```json", json.dumps(data, indent=1), "```", ""]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))
    return data


def load_traffic(md_path: str, kernel: str):
    """Counter bytes per launch of `kernel` from a traffic summary, or None
    if there is none or the kernel's sources changed since it was taken."""
    if not os.path.exists(md_path):
        return None
    text = open(md_path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    entry = json.loads(m.group(1)).get("kernels", {}).get(kernel)
    if entry is None:
        return None
    try:
        if entry["source_sha256"] != source_digest(kernel):
            return None
    except KeyError:
        return None
    return entry["traffic_bytes"]


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel trace")
    n = sub.add_parser("counters")
    n.add_argument("pmc_csv")
    n.add_argument("out")
    n.add_argument("--command", required=True)
    n.add_argument("--title", default="Counters")
    n.add_argument("--notes", default="")
    c = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--out",
              "--command", "--copy-command"):
        c.add_argument(a, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--title", default="HBM traffic")
    args = ap.parse_args()
    if args.cmd == "trace":
        write_trace_summary(args.stats_csv, args.out, args.command, args.title)
    elif args.cmd == "counters":
        write_counter_summary(args.pmc_csv, args.out, args.command, args.title, args.notes)
    else:
        write_traffic_summary(args.fetch, args.write, args.copy_fetch, args.copy_write,
                              args.copy_bytes, args.out, args.command,
                              args.copy_command, args.title)


if __name__ == "__main__":
    main()
