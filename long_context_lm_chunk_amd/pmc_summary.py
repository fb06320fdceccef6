"""Summarise rocprofv3 hardware-counter collections into a short markdown table.

Usage:
  python -m long_context_lm_chunk_amd.pmc_summary COUNTER_CSV [COUNTER_CSV ...]
         [--title T] [--cmd C ...] [--match SUBSTR ...] [--top K] [--cus 256]

Reads the per-dispatch ``*_counter_collection.csv`` files that
``rocprofv3 --pmc ... --output-format csv`` writes (several passes may be
given; their counters are merged per kernel symbol) and prints, per kernel:
dispatches, average duration, and whichever of these the counters allow:

  MFMA busy %   rocprof's MfmaUtil: sum(SQ_VALU_MFMA_BUSY_CYCLES) /
                (max(GRBM_GUI_ACTIVE) * SIMD_NUM) * 100
  VALU busy %   rocprof's VALUBusy: 100 * sum(SQ_ACTIVE_INST_VALU) / CU_NUM /
                max(GRBM_GUI_ACTIVE)
  bf16 TFLOP/s  SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 / duration
  HBM GB/s      (FETCH_SIZE + WRITE_SIZE) KiB / duration, unscaled
  LDS active %  rocprof's LDS utilisation: 100 * sum(SQ_LDS_IDX_ACTIVE) /
                (max(GRBM_GUI_ACTIVE) * CU_NUM)
  LDS conflict % the same with SQ_LDS_BANK_CONFLICT (cycles stalled by bank
                conflicts)

The CSV gives every counter summed over its instances; GRBM_GUI_ACTIVE has
one instance per XCD, so its maximum is taken as the sum over the XCDs
divided by their number (the XCDs run the same dispatch).

Under --pmc the dispatches run one at a time, so these are each kernel's
figures alone, not beside the other streams.  Raw collections stay out of
the repository; only these summaries are kept.
"""
from __future__ import annotations

import argparse
import csv
import re
from collections import defaultdict

from .profile_summary import short


def _mangled(name: str) -> str:
    """The CSV prints demangled names; fold template arguments into the
    compact form used by the trace summaries."""
    n = re.sub(r"\s+", " ", name)
    n = n.replace("void ttt::(anonymous namespace)::", "").replace("ttt::(anonymous namespace)::", "")
    n = re.sub(r"\(ttt::.*$", "", n)
    n = re.sub(r"\(.*$", "", n)
    n = n.replace("__hip_bfloat16", "bf16").replace("ttt::bf16", "bf16")
    n = n.replace("bool _Accum, bool, E", "bf16, true")   # how the tool prints "__bf16, true"
    return short(n) if n.startswith("_Z") else n[:90]


def load(paths):
    """{kernel: {"n": dispatches, "ns": total ns, counter: total}} (a kernel's
    duration is counted once per dispatch, whichever pass it comes from)."""
    per = defaultdict(lambda: defaultdict(float))
    seen = set()
    for path in paths:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                k = _mangled(row["Kernel_Name"])
                key = (path, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                counter = row["Counter_Name"]
                per[k][counter] += float(row["Counter_Value"])
                per[k]["_n_" + counter] += 1
                if key not in seen:
                    seen.add(key)
                    per[k]["_dispatch_ns_" + path] += float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
                    per[k]["_dispatches_" + path] += 1
    return per


def summarise(paths, title="", cmds=(), match=None, top=30, cus=256, xcc=8) -> str:
    per = load(paths)
    rows = []
    for k, c in per.items():
        if match and not any(m in k for m in match):
            continue
        # duration and dispatch count from the first pass that saw the kernel
        p0 = next((p for p in paths if c.get("_dispatches_" + p)), None)
        n = c["_dispatches_" + p0]
        ns = c["_dispatch_ns_" + p0]

        def mean(counter):
            # one row per counter and dispatch (its instances summed): the
            # mean over every dispatch that reported it, whichever pass
            cnt = c.get("_n_" + counter)
            return c[counter] / cnt if cnt else None

        gui = mean("GRBM_GUI_ACTIVE")
        mf = mean("SQ_VALU_MFMA_BUSY_CYCLES")
        va = mean("SQ_ACTIVE_INST_VALU")
        mops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        fe, wr = mean("FETCH_SIZE"), mean("WRITE_SIZE")
        lds, bc = mean("SQ_LDS_IDX_ACTIVE"), mean("SQ_LDS_BANK_CONFLICT")
        avg_ns = ns / n
        rows.append(dict(
            k=k, n=int(n), tot_ms=ns / 1e6, avg_us=avg_ns / 1e3,
            mfma=None if (gui is None or mf is None) else 100 * mf / (gui / xcc * 4 * cus),
            valu=None if (gui is None or va is None) else 100 * va / cus / (gui / xcc),
            tf=None if mops is None else mops * 512 / avg_ns / 1e3,
            gbs=None if (fe is None and wr is None) else ((fe or 0) + (wr or 0)) * 1024 / avg_ns,
            lds=None if (gui is None or lds is None) else 100 * lds / (gui / xcc * cus),
            bc=None if (gui is None or bc is None) else 100 * bc / (gui / xcc * cus)))
    rows.sort(key=lambda r: -r["tot_ms"])
    total = sum(r["tot_ms"] for r in rows) or 1.0
    f = lambda v, fmt: "" if v is None else format(v, fmt)   # noqa: E731
    out = [f"# {title}" if title else "# counter summary", ""]
    if cmds:
        out += ["Commands (one counter pass each):", "", "```"] + list(cmds) + ["```", ""]
    cols = [("MFMA busy %", "mfma", ".1f"), ("VALU busy %", "valu", ".1f"), ("bf16 TFLOP/s", "tf", ".0f"),
            ("HBM GB/s (raw)", "gbs", ".0f"), ("LDS active %", "lds", ".1f"), ("LDS conflict %", "bc", ".1f")]
    cols = [c for c in cols if any(r[c[1]] is not None for r in rows)]
    out += ["| kernel | dispatches | total ms | avg us | share | " + " | ".join(c[0] for c in cols) + " |",
            "|---|---|---|---|---|" + "---|" * len(cols)]
    for r in rows[:top]:
        out.append(f"| `{r['k']}` | {r['n']} | {r['tot_ms']:.2f} | {r['avg_us']:.1f} | "
                   f"{100 * r['tot_ms'] / total:.1f}% | " + " | ".join(f(r[c[1]], c[2]) for c in cols) + " |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("csv", nargs="+")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", nargs="*", default=())
    ap.add_argument("--match", nargs="*", default=None)
    ap.add_argument("--top", type=int, default=30)
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--xcc", type=int, default=8)
    a = ap.parse_args()
    print(summarise(a.csv, a.title, a.cmd, a.match, a.top, a.cus, a.xcc))
