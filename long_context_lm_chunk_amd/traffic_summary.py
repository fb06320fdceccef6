"""HBM traffic of one kernel from two rocprofv3 counter passes (FETCH_SIZE,
WRITE_SIZE), scaled by a plain device copy of known size run in the same
process.

Usage:
  python -m long_context_lm_chunk_amd.traffic_summary FETCH_DB WRITE_DB --match SUBSTR
         [--probe-mib 1024] [--shape NAME:M:N:K ...] [--bytes-per-weight 14]

FETCH_DB / WRITE_DB are the ``*_results.db`` files of two runs of the same
command, ``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one counter
per pass).  The copy probe (``bench.py --copy-probe MIB``: one elementwise
kernel reading MIB MiB and writing MIB MiB) gives each counter's scale: the
probe's reading divided by the bytes it moved.  The kernel's dispatches
(symbol containing SUBSTR) are grouped by grid size; ``--shape`` names the
groups in increasing grid order with their product shape (the output is
M x N, the reduction K) for the algorithmic bytes: bytes-per-weight per
output element plus both bf16 operands once.  Raw databases stay out of the
repository; only these summaries are kept.
"""
from __future__ import annotations

import argparse
import sqlite3
from collections import defaultdict


def _rows(db: str, counter: str):
    c = sqlite3.connect(db)
    q = ("select kernel_name, grid_size, value from counters_collection "
         "where counter_name = ? order by dispatch_id")
    return list(c.execute(q, (counter,)))


def _probe_scale(rows, mib: int) -> float:
    # the copy probe: the elementwise multiply that moved the most bytes
    vals = [v for (k, g, v) in rows if "MulFunctor" in k]
    if not vals:
        raise SystemExit("no copy probe in the database (run with --copy-probe)")
    return max(vals) / (mib * 1024.0)      # counter KiB per KiB moved


def summarise(fetch_db: str, write_db: str, match: str, probe_mib: int = 1024, shapes=(),
              bytes_per_weight: float = 14.0) -> str:
    out = []
    per = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = _rows(db, counter)
        scale = _probe_scale(rows, probe_mib)
        groups = defaultdict(list)
        for k, g, v in rows:
            if match in k:
                groups[g].append(v / scale * 1024.0)      # bytes
        per[counter] = (scale, groups)
    fs, fg = per["FETCH_SIZE"]
    ws, wg = per["WRITE_SIZE"]
    out.append(f"Scale reference (the copy kernel, {probe_mib} MiB read and {probe_mib} MiB written): "
               f"FETCH_SIZE {fs * probe_mib:.1f} MiB (factor {fs:.3f}), "
               f"WRITE_SIZE {ws * probe_mib:.1f} MiB (factor {ws:.3f}).")
    out.append("")
    out.append("| launch | dispatches | FETCH_SIZE scaled | WRITE_SIZE scaled | total | algorithmic |")
    out.append("|---|---|---|---|---|---|")
    grids = sorted(set(fg) | set(wg))
    tot_meas = tot_alg = 0.0
    n_all = 0
    for i, g in enumerate(grids):
        f = sum(fg.get(g, [])) / max(len(fg.get(g, [])), 1)
        w = sum(wg.get(g, [])) / max(len(wg.get(g, [])), 1)
        n = max(len(fg.get(g, [])), len(wg.get(g, [])))
        name, alg = f"grid {g}", None
        if i < len(shapes):
            name, M, N, K = shapes[i]
            alg = bytes_per_weight * M * N + 2.0 * (M + N) * K
        out.append(f"| {name} | {n} | {f / 1e6:.1f} MB | {w / 1e6:.1f} MB | {(f + w) / 1e6:.1f} MB | "
                   + (f"{alg / 1e6:.1f} MB |" if alg else "— |"))
        tot_meas += (f + w) * n
        tot_alg += (alg or 0.0) * n
        n_all += n
    if n_all:
        out.append(f"| mean per launch | | | | {tot_meas / n_all / 1e6:.1f} MB | "
                   + (f"{tot_alg / n_all / 1e6:.1f} MB |" if tot_alg else "— |"))
        if tot_alg:
            out.append("")
            out.append(f"Measured / algorithmic: {tot_meas / tot_alg:.3f}.")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_db")
    ap.add_argument("write_db")
    ap.add_argument("--match", required=True)
    ap.add_argument("--probe-mib", type=int, default=1024)
    ap.add_argument("--shape", nargs="*", default=[],
                    help="NAME:M:N:K per dispatch group, in increasing grid order")
    ap.add_argument("--bytes-per-weight", type=float, default=14.0)
    a = ap.parse_args()
    shp = []
    for s in a.shape:
        name, M, N, K = s.rsplit(":", 3)
        shp.append((name, int(M), int(N), int(K)))
    print(summarise(a.fetch_db, a.write_db, a.match, a.probe_mib, shp, a.bytes_per_weight))
