"""Summarise two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE) of
bench.py into the HBM traffic of the attention kernel.

Each counter is read per dispatch in KiB. It is calibrated against a plain
streaming kernel of known size that bench.py launches in the same process
(torch.neg over 1 GiB of bf16: reads 1 GiB, writes 1 GiB): the factor
known_bytes / (counter KiB * 1024) converts the counter into bytes, and the
attention kernel's traffic per launch is its average counter value times that
factor. Only the last `--last` attention dispatches are used: the kernel timed
alone at the end of bench.py, over the page lists of the step that just ran.

  python3 bench_counters.py FETCH_DIR WRITE_DIR [--last 640] [--out FILE.md]

FETCH_DIR/WRITE_DIR are the rocprofv3 output folders (CSV or rocpd sqlite
output). The markdown written to --out ends with one `traffic-json:` line that
bench.py reads back; it carries the hash of the attention kernel's sources so
that a stale measurement is not reported once the kernel changes.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ["long_context_sparse_summary_amd/csrc/attn.hip",
                "long_context_sparse_summary_amd/csrc/moira_common.h"]
ATTN_NAME = "attn_mfma_kernel"
CALIB_NAME = "neg_kernel"
CALIB_BYTES = 2**30


# the part of attn.hip that the attention kernel is built from: its prologue
# and the kernel itself (everything before the fp32 kernel), and its launcher;
# the combine kernels in the same file do not change its counters
ATTN_END_MARK = b"// ---- fp32 K/V kernel"
ATTN_LAUNCH_MARK = b"hipError_t launch_attn("
ATTN_LAUNCH_END = b"hipError_t launch_combine("


def attn_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            data = f.read()
        if rel.endswith("attn.hip"):
            data = (data[:data.index(ATTN_END_MARK)] +
                    data[data.index(ATTN_LAUNCH_MARK):data.index(ATTN_LAUNCH_END)])
        h.update(data)
    return h.hexdigest()[:16]


def _rows_csv(path):
    with open(path, newline="") as f:
        rd = csv.DictReader(f)
        cols = {c.lower(): c for c in rd.fieldnames or []}
        kn = cols.get("kernel_name")
        cn = cols.get("counter_name")
        cv = cols.get("counter_value")
        di = cols.get("dispatch_id")
        if not (kn and cn and cv):
            raise SystemExit(f"{path}: unexpected columns {rd.fieldnames}")
        for r in rd:
            yield int(r[di]) if di else 0, r[kn], r[cn], float(r[cv])


def _rows_db(path):
    db = sqlite3.connect(path)
    q = ("select dispatch_id, kernel_name, counter_name, value from counters_collection "
         "order by dispatch_id")
    for d, k, c, v in db.execute(q):
        yield int(d), k, c, float(v)


def read_counter(folder: str, counter: str):
    """{kernel name: [(dispatch id, value KiB), ...]} for one counter pass."""
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if files:
        rows = [r for f in files for r in _rows_csv(f)]
    else:
        dbs = glob.glob(os.path.join(folder, "**", "*.db"), recursive=True)
        if not dbs:
            raise SystemExit(f"no counter output under {folder}")
        rows = [r for f in dbs for r in _rows_db(f)]
    out = {}
    for d, k, c, v in rows:
        if c != counter:
            continue
        out.setdefault(k, []).append((d, v))
    for k in out:
        out[k].sort()
    return out


def pick(table, needle):
    names = [k for k in table if needle in k]
    if len(names) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {names}")
    return names[0], [v for _, v in table[names[0]]]


def mean(xs):
    return sum(xs) / len(xs)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("--last", type=int, default=640)
    ap.add_argument("--alg-bytes", type=float, default=None,
                    help="algorithmic bytes per attention launch of the same run")
    ap.add_argument("--command", default="", help="command lines recorded in the summary")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    fetch = read_counter(args.fetch_dir, "FETCH_SIZE")
    write = read_counter(args.write_dir, "WRITE_SIZE")
    cal_name, cal_f = pick(fetch, CALIB_NAME)
    _, cal_w = pick(write, CALIB_NAME)
    attn_name, att_f = pick(fetch, ATTN_NAME)
    _, att_w = pick(write, ATTN_NAME)
    att_f, att_w = att_f[-args.last:], att_w[-args.last:]

    f_factor = CALIB_BYTES / (mean(cal_f) * 1024.0)
    w_factor = CALIB_BYTES / (mean(cal_w) * 1024.0)
    fetch_b = mean(att_f) * 1024.0 * f_factor
    write_b = mean(att_w) * 1024.0 * w_factor
    traffic = fetch_b + write_b

    lines = ["# HBM traffic of attn_mfma_kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE)", ""]
    if args.command:
        lines += ["Commands:", "", "```", args.command.strip(), "```", ""]
    lines += [
        f"Calibration kernel: `{cal_name[:100]}` (reads {CALIB_BYTES} B, writes {CALIB_BYTES} B), "
        f"{len(cal_f)} / {len(cal_w)} dispatches.",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| calibration FETCH_SIZE (KiB/dispatch) | {mean(cal_f):.1f} |",
        f"| calibration WRITE_SIZE (KiB/dispatch) | {mean(cal_w):.1f} |",
        f"| fetch factor (bytes per counted byte) | {f_factor:.4f} |",
        f"| write factor (bytes per counted byte) | {w_factor:.4f} |",
        f"| attention dispatches used | {len(att_f)} / {len(att_w)} |",
        f"| attention FETCH_SIZE (KiB/dispatch, raw) | {mean(att_f):.1f} |",
        f"| attention WRITE_SIZE (KiB/dispatch, raw) | {mean(att_w):.1f} |",
        f"| attention fetched bytes/launch (scaled) | {fetch_b:.0f} |",
        f"| attention written bytes/launch (scaled) | {write_b:.0f} |",
        f"| attention traffic bytes/launch | {traffic:.0f} |",
    ]
    if args.alg_bytes:
        lines.append(f"| algorithmic bytes/launch (same run) | {args.alg_bytes:.0f} |")
        lines.append(f"| traffic / algorithmic | {traffic / args.alg_bytes:.4f} |")
    rec = {"kernel": ATTN_NAME, "source_hash": attn_source_hash(),
           "traffic_bytes_per_launch": round(traffic), "fetch_bytes": round(fetch_b),
           "write_bytes": round(write_b), "fetch_factor": round(f_factor, 5),
           "write_factor": round(w_factor, 5),
           "alg_bytes_per_launch": round(args.alg_bytes) if args.alg_bytes else None}
    lines += ["", "traffic-json: " + json.dumps(rec), ""]
    text = "\n".join(lines)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    sys.exit(main())
