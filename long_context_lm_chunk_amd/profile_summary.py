"""Summarise a rocprofv3 kernel-trace database into a short markdown table.

Usage:
  python -m long_context_lm_chunk_amd.profile_summary RESULTS_DB [--title T] [--cmd C]
         [--per N] [--match SUBSTR ...] [--exclude SUBSTR ...] [--top K]
  python -m long_context_lm_chunk_amd.profile_summary RESULTS_DB --streams START_KERNEL INDEX STOP_KERNEL

Reads the per-dispatch kernel table that ``rocprofv3 --kernel-trace`` writes
(SQLite) and prints calls, total and average duration and share per kernel
symbol (the unit in which a HIP-event average over one kernel's launches can
be compared with the trace), with shortened names.  ``--per N`` also divides
calls and time by N (e.g. the number of prefills in the run); ``--match``
keeps only symbols containing one of the substrings, ``--exclude`` drops them.  Raw databases stay out
of the repository; only these summaries are kept.
"""
from __future__ import annotations

import argparse
import re
import sqlite3


def short(name: str) -> str:
    n = re.sub(r"\s+", " ", name)
    n = n.replace("void ttt::(anonymous namespace)::", "").replace("ttt::(anonymous namespace)::", "")
    n = n.replace("bool _Accum, bool, E", "bf16, true")   # how the tool prints "__bf16, true"
    m = re.match(r"_ZN3ttt12_GLOBAL__N_1\d+(\w+?)I(.+?)EEv", n)
    if m:
        toks, a = [], m.group(2)
        while a:
            t = re.match(r"DF16b|f|Lb[01]E|Li-?\d+E", a)
            if not t:
                toks.append(a)
                break
            g = t.group(0)
            toks.append({"DF16b": "bf16", "f": "float", "Lb1E": "true", "Lb0E": "false"}.get(
                g, g[2:-1] if g.startswith("Li") else g))
            a = a[len(g):]
        return f"{m.group(1)}<{', '.join(toks)}>"
    m = re.match(r"_ZN3ttt12_GLOBAL__N_1\d+(\w+?)E", n)
    if m:
        return m.group(1)
    n = re.sub(r"\((ttt::|DecGemv|HIP_vector|float const|int const).*", "", n)
    return n[:90]


def summarise(db: str, title: str = "", cmd: str = "", per: float = 1.0, match=None, top: int = 30,
              exclude=None) -> str:
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), sum(duration), avg(duration) from kernels "
                     "group by name order by sum(duration) desc").fetchall()
    if match:
        rows = [r for r in rows if any(mm in r[0] for mm in match)]
    if exclude:
        rows = [r for r in rows if not any(mm in r[0] for mm in exclude)]
    total = sum(r[2] for r in rows)
    out = [f"# {title}" if title else "# kernel summary", ""]
    if cmd:
        out += ["Command:", "", "```", cmd, "```", ""]
    out += [f"Total kernel time {total / 1e6:.1f} ms over {sum(r[1] for r in rows)} dispatches"
            + (f" ({total / 1e6 / per:.1f} ms per unit, {per:g} units)." if per != 1 else "."), ""]
    hdr = "| kernel | calls | total ms | avg us | share |"
    if per != 1:
        hdr = "| kernel | calls | total ms | calls/unit | ms/unit | avg us | share |"
    out += [hdr, "|" + "---|" * (hdr.count("|") - 1)]
    for name, n, tot, avg in rows[:top]:
        if per != 1:
            out.append(f"| `{short(name)}` | {n} | {tot / 1e6:.2f} | {n / per:g} | {tot / 1e6 / per:.3f} | "
                       f"{avg / 1e3:.1f} | {100 * tot / total:.1f}% |")
        else:
            out.append(f"| `{short(name)}` | {n} | {tot / 1e6:.2f} | {avg / 1e3:.1f} | {100 * tot / total:.1f}% |")
    return "\n".join(out) + "\n"


def streams(db: str, start_kernel: str, start_index: int, stop_kernel: str) -> str:
    """Per-stream occupancy over one window of the trace: from the start of
    the start_index-th dispatch (0-based) whose name holds start_kernel to
    the end of the last dispatch that starts before the next dispatch whose
    name holds stop_kernel.  For every stream: kernels, busy time (the union
    of its dispatches), its share of the window and of the stream's own span,
    and the idle gaps between its dispatches, split at 1 ms."""
    c = sqlite3.connect(db)
    rows = c.execute("select stream_id, start, end, name from kernels order by start").fetchall()
    starts = [r[1] for r in rows if start_kernel in r[3]]
    t0 = starts[start_index]
    stops = [r[1] for r in rows if stop_kernel in r[3] and r[1] > t0]
    t_stop = stops[0] if stops else rows[-1][1] + 1
    t1 = max(r[2] for r in rows if t0 <= r[1] < t_stop)
    span = t1 - t0
    out = [f"Window: {span / 1e6:.1f} ms (dispatch {start_index} of `{start_kernel}` to the last dispatch "
           f"before the next `{stop_kernel}`).", "",
           "| stream | kernels | busy ms | busy % of window | busy % of own span | gaps > 1 ms | their ms | "
           "gaps < 1 ms: ms | median gap us |",
           "|---|---|---|---|---|---|---|---|---|"]
    for sid in sorted({r[0] for r in rows}):
        iv = [(r[1], min(r[2], t1)) for r in rows if r[0] == sid and t0 <= r[1] < t_stop]
        if not iv:
            continue
        busy, gaps = 0, []
        cs, ce = iv[0]
        for s_, e_ in iv[1:]:
            if s_ > ce:
                busy += ce - cs
                gaps.append(s_ - ce)
                cs, ce = s_, e_
            else:
                ce = max(ce, e_)
        busy += ce - cs
        own = max(e for _, e in iv) - iv[0][0]
        big = [g for g in gaps if g > 1e6]
        small = [g for g in gaps if g <= 1e6]
        med = sorted(gaps)[len(gaps) // 2] / 1e3 if gaps else 0.0
        out.append(f"| {sid} | {len(iv)} | {busy / 1e6:.1f} | {100 * busy / span:.1f}% | {100 * busy / own:.1f}% | "
                   f"{len(big)} | {sum(big) / 1e6:.1f} | {sum(small) / 1e6:.1f} | {med:.1f} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--title", default="")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--per", type=float, default=1.0)
    ap.add_argument("--match", nargs="*", default=None)
    ap.add_argument("--exclude", nargs="*", default=None)
    ap.add_argument("--top", type=int, default=30)
    ap.add_argument("--streams", nargs=3, metavar=("START_KERNEL", "INDEX", "STOP_KERNEL"), default=None,
                    help="per-stream occupancy over one window instead of the kernel table")
    a = ap.parse_args()
    if a.streams:
        print(streams(a.db, a.streams[0], int(a.streams[1]), a.streams[2]))
    else:
        print(summarise(a.db, a.title, a.cmd, a.per, a.match, a.top, a.exclude))
