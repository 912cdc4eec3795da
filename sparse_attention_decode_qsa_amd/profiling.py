"""Summaries of rocprofv3 CSV output, written as short text files for the profiles folder.

    python -m sparse_attention_decode_qsa_amd.profiling stats --dir D --prefix P --command CMD --out F
        kernel-trace statistics (<D>/<P>_kernel_stats.csv) of the decode chain as a table.
    python -m sparse_attention_decode_qsa_amd.profiling traffic --fetch CSV --write CSV \
            --calib-bytes N --command CMD --out F
        HBM bytes per launch of the indexer scan from a FETCH_SIZE run and a WRITE_SIZE run,
        each scaled by what the same counter reads for qsa_calib_copy (libqsa_calib) moving a
        known number of bytes with the same kind of loads and stores.

The traffic file ends with a JSON block (figures plus a hash of the scan's source files);
bench.py reports the figure only while that hash matches the sources it runs.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
SCAN_SOURCES = ("csrc/index_score.hip", "csrc/qsa_device.h")
SCAN_KERNEL = "index_score_kernel"
CALIB_KERNEL = "calib_copy_kernel"
CHAIN = ("cache_append_kernel", "index_score_kernel", "index_score_pooled_kernel", "index_score_mq_kernel",
         "index_score_pooled_multi_kernel", "topk_select_kernel", "sparse_attn_kernel", "sparse_attn_pair_kernel",
         "slice_merge_kernel",
         "slice_merge_v4_kernel",
         "lse_merge_kernel")


def scan_source_hash() -> str:
    """sha256 over the indexer scan's source files (the kernel the traffic figure belongs to)."""
    h = hashlib.sha256()
    for rel in SCAN_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    return re.sub(r"^void ", "", name.split("(")[0])


def stats_table(stats_csv: str) -> list[dict]:
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        name = _short(r["Name"])
        if any(k in name for k in CHAIN):
            rows.append(dict(kernel=name, calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3,
                             min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3,
                             share=float(r["Percentage"])))
    order = {k: i for i, k in enumerate(CHAIN)}
    rows.sort(key=lambda r: min(order[k] for k in CHAIN if k + "<" in r["kernel"] or r["kernel"].endswith(k)))
    return rows


def chain_span_us(trace_csv: str, skip: int = 20) -> float | None:
    """Median span of one whole call in the trace: from the start of the first kernel of a
    call (the cache append when there is one, else the scan) to the end of the merge."""
    tr = [r for r in csv.DictReader(open(trace_csv)) if "qsa::" in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    spans = []
    for i in range(len(tr) - 3):
        n0 = tr[i]["Kernel_Name"]
        j = i + 1 if "cache_append" in n0 else i          # the scan
        if j + 3 >= len(tr) + 0 and j + 3 > len(tr) - 1:
            break
        names = [tr[j + d]["Kernel_Name"] for d in range(4)]
        if ("index_score" in names[0] and "topk_select" in names[1] and "sparse_attn" in names[2]
                and "merge" in names[3]) and (j == i or "cache_append" in n0):
            if j == i and i > 0 and "cache_append" in tr[i - 1]["Kernel_Name"]:
                continue                                    # counted from its append
            spans.append((int(tr[j + 3]["End_Timestamp"]) - int(tr[i]["Start_Timestamp"])) / 1e3)
    spans = spans[skip:] or spans
    if not spans:
        return None
    spans.sort()
    return spans[len(spans) // 2]


def chain_timeline(trace_csv: str, skip: int = 10) -> list[dict] | None:
    """Median start and end of each kernel of a whole call (scan, selection, attention, merge),
    in us from the start of the call's scan, over the calls of the trace (the first `skip`
    calls left out)."""
    tr = [r for r in csv.DictReader(open(trace_csv)) if "qsa::" in r["Kernel_Name"]]
    tr.sort(key=lambda r: int(r["Start_Timestamp"]))
    calls, i = [], 0
    while i + 3 < len(tr):
        names = [tr[i + d]["Kernel_Name"] for d in range(4)]
        if ("index_score" in names[0] and "topk_select" in names[1] and "sparse_attn" in names[2]
                and "merge" in names[3]):
            t0 = int(tr[i]["Start_Timestamp"])
            calls.append([(_short(names[d]), int(tr[i + d]["Start_Timestamp"]) - t0,
                           int(tr[i + d]["End_Timestamp"]) - t0) for d in range(4)])
            i += 4
        else:
            i += 1
    calls = calls[skip:] or calls
    if not calls:
        return None

    def med(v):
        v = sorted(v)
        return v[len(v) // 2] / 1e3

    return [dict(kernel=calls[0][d][0], start_us=med([c[d][1] for c in calls]), end_us=med([c[d][2] for c in calls]),
                 dur_us=med([c[d][2] - c[d][1] for c in calls]), calls=len(calls)) for d in range(4)]


def write_stats(dir_: str, prefix: str, command: str, out: str, title: str, note: str = "") -> None:
    rows = stats_table(os.path.join(dir_, f"{prefix}_kernel_stats.csv"))
    span = chain_span_us(os.path.join(dir_, f"{prefix}_kernel_trace.csv"))
    lines = [f"# {title}", "", "Command (from the repository root, on the MI355X):", "", f"    {command}", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['share']:.1f} |")
    lines.append("")
    if span is not None:
        lines.append(f"Median span of one whole call (start of its first kernel to the end of the merge): {span:.2f} us.")
    tl = chain_timeline(os.path.join(dir_, f"{prefix}_kernel_trace.csv"))
    if tl:
        lines += ["", f"Timeline of one call (medians over {tl[0]['calls']} whole calls, us from the start of the scan):", "",
                  "| kernel | start | end | duration |", "|---|---|---|---|"]
        for r in tl:
            lines.append(f"| {r['kernel']} | {r['start_us']:.2f} | {r['end_us']:.2f} | {r['dur_us']:.2f} |")
    if note:
        lines += ["", note]
    open(out, "w").write("\n".join(lines) + "\n")


def _counter_means(path: str, counter: str) -> dict[str, tuple[float, int]]:
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        for k in (SCAN_KERNEL, CALIB_KERNEL):
            if k + "(" in name or k + "<" in name:
                acc[k].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def traffic(fetch_csv: str, write_csv: str, calib_bytes: int) -> dict:
    """Bytes per launch of the scan: counter (KiB) * 1024 / (calibration copy's counter / its bytes)."""
    f = _counter_means(fetch_csv, "FETCH_SIZE")
    w = _counter_means(write_csv, "WRITE_SIZE")
    for k in (SCAN_KERNEL, CALIB_KERNEL):
        if k not in f or k not in w:
            raise ValueError(f"no {k} dispatch with FETCH_SIZE and WRITE_SIZE in the CSV files")
    rf = f[CALIB_KERNEL][0] * 1024 / calib_bytes
    rw = w[CALIB_KERNEL][0] * 1024 / calib_bytes
    read = f[SCAN_KERNEL][0] * 1024 / rf
    write = w[SCAN_KERNEL][0] * 1024 / rw
    return dict(kernel=SCAN_KERNEL, fetch_kib=round(f[SCAN_KERNEL][0], 1), write_kib=round(w[SCAN_KERNEL][0], 1),
                dispatches=f[SCAN_KERNEL][1], calib_bytes=calib_bytes,
                calib_fetch_kib=round(f[CALIB_KERNEL][0], 1), calib_write_kib=round(w[CALIB_KERNEL][0], 1),
                read_factor=round(rf, 4), write_factor=round(rw, 4), read_bytes=int(read),
                write_bytes=int(write), traffic_bytes=int(read + write), source_hash=scan_source_hash())


def write_traffic(res: dict, command_fetch: str, command_write: str, out: str, title: str,
                  algorithmic_bytes: int | None = None) -> None:
    lines = [f"# {title}", "", "Commands (from the repository root, on the MI355X), one counter per run:", "",
             f"    {command_fetch}", f"    {command_write}", "",
             f"Calibration: qsa_calib_copy moved {res['calib_bytes']:,} bytes per dispatch with the scan's kind",
             f"of loads and stores; FETCH_SIZE read {res['calib_fetch_kib']:,} KiB and WRITE_SIZE "
             f"{res['calib_write_kib']:,} KiB for it,",
             f"so 1 KiB counted = {1 / res['read_factor']:.3f} KiB read and {1 / res['write_factor']:.3f} KiB written.",
             "",
             "| per launch of the scan | counted KiB | bytes after scaling |", "|---|---|---|",
             f"| FETCH_SIZE (reads) | {res['fetch_kib']:,} | {res['read_bytes']:,} |",
             f"| WRITE_SIZE (writes) | {res['write_kib']:,} | {res['write_bytes']:,} |",
             f"| total | | {res['traffic_bytes']:,} |", ""]
    if algorithmic_bytes:
        lines.append(f"Algorithmic bytes per launch: {algorithmic_bytes:,}; measured/algorithmic = "
                     f"{res['traffic_bytes'] / algorithmic_bytes:.3f}.")
        lines.append("")
    lines += ["```json", json.dumps(res), "```"]
    open(out, "w").write("\n".join(lines) + "\n")


def read_traffic(path: str) -> dict | None:
    """The JSON block of a traffic file, or None when the file is missing or unreadable."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    try:
        return json.loads(m.group(1))
    except json.JSONDecodeError:
        return None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--prefix", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="Kernel time of the decode chain (rocprofv3 kernel trace)")
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=None)
    t.add_argument("--out", required=True)
    t.add_argument("--title", default="HBM traffic of the indexer scan (rocprofv3 counters)")
    a = ap.parse_args()
    if a.cmd == "stats":
        write_stats(a.dir, a.prefix, a.command, a.out, a.title, a.note)
    else:
        res = traffic(a.fetch, a.write, a.calib_bytes)
        write_traffic(res, a.command_fetch, a.command_write, a.out, a.title, a.algorithmic_bytes)
        print(json.dumps(res))


if __name__ == "__main__":
    main()
