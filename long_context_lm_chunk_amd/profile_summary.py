"""Summarise a rocprofv3 kernel-trace database into a short markdown table.

Usage: python -m long_context_lm_chunk_amd.profile_summary RESULTS_DB [TITLE] [COMMAND]

Reads the per-dispatch kernel table that ``rocprofv3 --kernel-trace``
writes (SQLite) and prints calls, total/average duration and share per
kernel, with demangled-ish short names.  Raw databases stay out of the
repository; only these summaries are kept.
"""
from __future__ import annotations

import re
import sqlite3
import sys


def short(name: str) -> str:
    n = re.sub(r"\s+", " ", name)
    m = re.match(r"_ZN3ttt12_GLOBAL__N_1\d+(\w+?)I(.*)EEvN.*", n)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    return n[:110]


def summarise(db: str, title: str = "", cmd: str = "") -> str:
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), sum(duration), avg(duration) from kernels "
                     "group by name order by sum(duration) desc").fetchall()
    total = sum(r[2] for r in rows)
    out = [f"# {title}" if title else "# kernel summary", ""]
    if cmd:
        out += ["Command:", "", "```", cmd, "```", ""]
    out += [f"Total kernel time {total / 1e6:.1f} ms over {sum(r[1] for r in rows)} dispatches.", "",
            "| kernel | calls | total ms | avg us | share |", "|---|---|---|---|---|"]
    for name, n, tot, avg in rows[:30]:
        out.append(f"| `{short(name)}` | {n} | {tot / 1e6:.2f} | {avg / 1e3:.1f} | {100 * tot / total:.1f}% |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    print(summarise(sys.argv[1], sys.argv[2] if len(sys.argv) > 2 else "",
                    sys.argv[3] if len(sys.argv) > 3 else ""))
