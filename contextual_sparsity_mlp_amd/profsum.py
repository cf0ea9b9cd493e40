"""Summaries of rocprofv3 output for the decode-layer benchmark.

    python -m contextual_sparsity_mlp_amd.profsum stats <kernel_stats.csv> <kernel_trace.csv> <out.md> "<command>" ["<title>"]
    python -m contextual_sparsity_mlp_amd.profsum traffic <fetch counter_collection.csv>
        <write counter_collection.csv> <out.json> "<command>"

`stats` turns a --kernel-trace --stats kernel summary into a short table, and adds
the per-launch durations of the decode kernels from the trace, each launch named by
its kernel (the phase kernel is one template per launch mix; launches of one template
are told apart by grid size).
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) of
`bench.py --sparse-only --copy-calibrate` (batch 1, bf16): the plain 1 GiB copy
calibrates each counter (bytes per counted KiB), and the two launches of the sparse
MLP + MHA step are averaged: "2:0" the row dots (rowdot_kernel<1, 1>), "2:1" the
attention + waiting row sums (phase_kernel<38, 1>), keyed as bench.py's roofline
looks them up (launches of the step : launch).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
# template flags of the decode kernels for each launch slot of the look-ahead step
SLOT_FLAGS = {0: "1", 1: "6", 2: "20"}


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "contextual_sparsity_mlp_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_label(name: str) -> str:
    """Short kernel name with its template arguments (dv::rowdot_kernel<1, 1>)."""
    m = re.search(r"dv::(\w+)(<[^>]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else re.sub(r"\(.*", "", name)[:60]


def stats(src: str, trace: str, out: str, command: str, title: str = ""):
    rows = list(csv.DictReader(open(src)))
    # fp8 weight rows: the row dots and the output row sum carry the fp8 flag (128),
    # and without a next layer the attention runs alone before the row sum
    fp8 = any(re.search(r"(?:phase|rowdot|rowdot_kv)_kernel<129, ", r["Name"]) for r in rows)
    weights = "fp8 (E4M3) weight rows" if fp8 else "bf16 weights"
    mb = re.search(r"--batch (\d+)", command)
    batch = int(mb.group(1)) if mb else 1
    head = title or f"OPT-175B-shaped decode layer, batch {batch}, {weights}"
    lines = [f"# rocprofv3 kernel summary: {head}", "",
             f"Command: `{command}`", "",
             "## Per kernel (rocprofv3 --stats)", "",
             "| kernel | calls | avg us | min us | max us | % time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        short = re.sub(r"\(.*", "", r["Name"])
        if len(short) > 70:
            short = short[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    groups = {}
    seq = []
    names_by_flags = {}
    for r in sorted(csv.DictReader(open(trace)), key=lambda r: int(r["Start_Timestamp"])):
        m = re.search(r"(?:phase|rowdot|rowdot_kv)_kernel(?:_bt)?<(\d+), (\d+)>", r["Kernel_Name"])
        mm = re.search(r"rowdot_mfma(_lds)?_kernel(?:<(\d+)>)?", r["Kernel_Name"])
        if not m and not mm:
            continue
        blocks = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        # matrix-core row dots are listed as flags "mfma", batch tile = token tiles of 16
        fl, bt = (m.group(1), m.group(2)) if m else ("mfma", "lds" if mm.group(1) else mm.group(2))
        groups.setdefault((fl, bt, blocks), []).append(dur)
        names_by_flags.setdefault(fl, kernel_label(r["Kernel_Name"]))
        seq.append((fl, dur))
    # launches of the look-ahead step: a row-dot launch directly followed by the
    # attention + row-sum launch and the row-sum + top-k launch (with a batch of at
    # least 3 tokens: matrix-core row dots and row sums, flag 512, the attention in a
    # launch of its own before the predictor's row sums, and the score histograms in
    # one of their own after them)
    slot_flags = dict(SLOT_FLAGS)
    if fp8:
        slot_flags = {0: "129", 1: "6", 2: "148"}
    elif batch > 16:
        slot_flags = {0: "mfma", 1: "2", 2: "1540", 3: "8", 4: "1556"}
    elif batch >= 3:
        slot_flags = {0: "mfma", 1: "2", 2: "516", 3: "8", 4: "532"}
    order = [slot_flags[k] for k in sorted(slot_flags)]
    slot_durs = {k: [] for k in slot_flags}
    for i in range(len(seq) - len(order) + 1):
        if all(seq[i + j][0] == order[j] for j in range(len(order))):
            for j in range(len(order)):
                slot_durs[j].append(seq[i + j][1])
    lines += ["", "## Decode launches by configuration (from the kernel trace)", "",
              "flags: 1 row dots, 2 attention, 4 row sums, 8 histogram, 16 top-k classify, "
              "32 row sums that wait for in-launch attention, 64 zero fill, 128 fp8 rows, "
              "256 KV stores, 512 matrix-core row sums (sums of these for a mixed launch); "
              "mfma: the matrix-core row dots (batch tile lds: y staged in LDS)", "",
              "| kernel | flags, batch tile | blocks | launches | avg us | median us | min us |",
              "|---|---|---|---|---|---|---|"]
    for (fl, bt, blocks), v in sorted(groups.items(), key=lambda kv: -len(kv[1])):
        lines.append(f"| `{names_by_flags.get(fl, '?')}` | <{fl}, {bt}> | {blocks} | {len(v)} | "
                     f"{statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} |")
    # launches of the sparse MLP + MHA step: row dots, then the single launch of
    # attention and the waiting row sum
    sp_order = (["129", "2", "132"] if fp8 else ["mfma", "2", "1540"] if batch > 16
                else ["mfma", "2", "516"] if batch >= 3 else ["1", "38"])
    sp_durs = {k: [] for k in range(len(sp_order))}
    for i in range(len(seq) - len(sp_order) + 1):
        # (not the first launches of a look-ahead step, whose order starts alike)
        nxt = seq[i + len(sp_order)][0] if i + len(sp_order) < len(seq) else None
        if len(order) > len(sp_order) and nxt == order[len(sp_order)]:
            continue
        if all(seq[i + j][0] == sp_order[j] for j in range(len(sp_order))):
            for j in range(len(sp_order)):
                sp_durs[j].append(seq[i + j][1])
    if slot_durs[0]:
        names = ({0: "row dots (W1, W^Q, A rows)", 1: "attention", 2: "predictor B rows",
                  3: "score histograms", 4: "row sum W2 + W^O rows, combine, top-k"}
                 if len(order) == 5 else
                 {0: "row dots (W1, W^Q, A rows)", 1: "attention + predictor B rows",
                  2: "row sum W2 + W^O rows, combine, top-k"})
        lines += ["", "## Look-ahead decode step, per launch (from the kernel trace)", "",
                  "| launch | kernel | launches | avg us | median us | min us |",
                  "|---|---|---|---|---|---|"]
        for k in sorted(slot_durs):
            v = slot_durs[k]
            lines.append(f"| {k}: {names[k]} | `{names_by_flags.get(slot_flags[k], '?')}` | {len(v)} | "
                         f"{statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} |")
    if sp_durs[0]:
        names = ({0: "row dots (W1, W^Q rows)", 1: "attention, split pieces combined per head",
                  2: "row sum W2 + W^O rows"} if len(sp_order) == 3 else
                 {0: "row dots (W1, W^Q rows)", 1: "attention + row sum W2 then W^O rows"})
        lines += ["", "## Sparse MLP + MHA step, per launch (from the kernel trace)", "",
                  "| launch | kernel | launches | avg us | median us | min us |",
                  "|---|---|---|---|---|---|"]
        for k in sorted(sp_durs):
            v = sp_durs[k]
            lines.append(f"| {k}: {names[k]} | `{names_by_flags.get(sp_order[k], '?')}` | {len(v)} | "
                         f"{statistics.mean(v):.2f} | {statistics.median(v):.2f} | {min(v):.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def _counter_rows(path, counter):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        out.append((r["Kernel_Name"], int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0),
                    float(r["Counter_Value"])))
    return out


# launches of the sparse MLP + MHA step at batch 1 (bf16), keyed as bench.py reads them
SPARSE_LAUNCHES = {"2:0": r"rowdot_kernel<1, 1>", "2:1": r"phase_kernel<38, 1>"}


def _per_launch(rows):
    copy = [v for n, g, v in rows if "copyBuffer" in n]
    per = {}
    for key, pat in SPARSE_LAUNCHES.items():
        vals = [(g, v) for n, g, v in rows if pat in n]
        if not vals:
            continue
        # the decode launches are the most frequent grid size of that kernel
        grids = [g for g, _ in vals]
        common = max(set(grids), key=grids.count)
        per[key] = statistics.median([v for g, v in vals if g == common])
    return (max(copy) if copy else None), per


def traffic(fetch_csv: str, write_csv: str, out: str, command: str):
    f_copy, f_per = _per_launch(_counter_rows(fetch_csv, "FETCH_SIZE"))
    w_copy, w_per = _per_launch(_counter_rows(write_csv, "WRITE_SIZE"))
    f_scale = COPY_BYTES / f_copy if f_copy else None
    w_scale = COPY_BYTES / w_copy if w_copy else None
    per = {}
    for key in sorted(set(f_per) | set(w_per)):
        fb = f_per.get(key, 0.0) * (f_scale or 0)
        wb = w_per.get(key, 0.0) * (w_scale or 0)
        per[key] = {"kernel": SPARSE_LAUNCHES[key], "fetch_bytes": round(fb),
                    "write_bytes": round(wb), "bytes": round(fb + wb)}
    res = {"workload": "OPT-175B-shaped sparse MLP + MHA step, batch 1, bf16 rows",
           "command": command, "source_hash": source_hash(),
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": f_copy, "write_kib": w_copy,
                                "fetch_bytes_per_count": f_scale,
                                "write_bytes_per_count": w_scale},
           "per_launch": {k: v["bytes"] for k, v in per.items()},
           "per_launch_detail": per}
    json.dump(res, open(out, "w"), indent=1)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], *(sys.argv[6:7]))
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    else:
        raise SystemExit(__doc__)
