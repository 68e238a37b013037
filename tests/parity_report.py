"""Counts kept by the GPU parity tests and written out when the session ends.

For every test: how many page lists were compared with the oracle, how many
differed, how many differing pages fell in the cumulative band around gamma
(|C_k - gamma| <= 1e-5 gamma) and how many were exact near-ties at the cut,
plus the largest output error and its ratio to the tolerance. The summary is
written to $MOIRA_PARITY_REPORT, else gpurun_out/parity_exceptions.md at the
repository root, and only when a test recorded something (GPU runs).
"""

from __future__ import annotations

import os
import time

REPORT: dict = {}
CURRENT = ["(outside a test)"]

_FIELDS = ("lists", "differing_lists", "band_pages", "near_tie_pages", "outputs")


def record() -> dict:
    return REPORT.setdefault(CURRENT[0], {**{k: 0 for k in _FIELDS}, "max_abs_err": 0.0,
                                          "max_err_over_tol": 0.0, "max_err_over_tight": 0.0})


def note_errors(max_abs: float, over_tol: float, over_tight: float) -> None:
    r = record()
    r["outputs"] += 1
    r["max_abs_err"] = max(r["max_abs_err"], float(max_abs))
    r["max_err_over_tol"] = max(r["max_err_over_tol"], float(over_tol))
    r["max_err_over_tight"] = max(r["max_err_over_tight"], float(over_tight))


def write(root: str, tol: str, tight: str) -> str | None:
    if not REPORT:
        return None
    path = os.environ.get("MOIRA_PARITY_REPORT") or os.path.join(root, "gpurun_out",
                                                                  "parity_exceptions.md")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    tot = {k: sum(r[k] for r in REPORT.values()) for k in _FIELDS}
    worst = max(r["max_err_over_tol"] for r in REPORT.values())
    worst_t = max(r["max_err_over_tight"] for r in REPORT.values())
    lines = [
        "# Parity exceptions of the GPU tests against the fp64 oracle",
        "",
        f"Written {time.strftime('%Y-%m-%d %H:%M:%S')} by the test session.",
        "",
        "Page lists must equal the oracle's except pages in two bands: the cumulative",
        "band (rank positions whose running mass lies within 1e-5 gamma of gamma) and",
        "exact near-ties at the cut (masses within 1e-12 relative). A differing list",
        "must still cover gamma (1 - 1e-5) of the oracle's mass and stay minimal.",
        f"Outputs: |gpu - ref| <= {tol}, and the tighter bound {tight} derived",
        "from the arithmetic; `err / tol` and `err / tight` are the worst ratios.",
        "",
        f"Totals: {tot['lists']} lists compared, {tot['differing_lists']} differing, "
        f"{tot['band_pages']} band pages, {tot['near_tie_pages']} near-tie pages; "
        f"{tot['outputs']} output blocks, worst error / tolerance {worst:.3g}, "
        f"worst error / tight bound {worst_t:.3g}.",
        "",
        "| test | lists | differing | band pages | near-tie pages | output blocks | max abs err | err / tol | err / tight |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for name, r in REPORT.items():
        lines.append(f"| `{name}` | {r['lists']} | {r['differing_lists']} | {r['band_pages']} | "
                     f"{r['near_tie_pages']} | {r['outputs']} | {r['max_abs_err']:.3g} | "
                     f"{r['max_err_over_tol']:.3g} | {r['max_err_over_tight']:.3g} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path
