"""Summarise a rocprofv3 run (rocpd SQLite output) into a short per-kernel table.

    python -m sparse_attention_hyb_amd.prof_summary <results.db> [--pmc] [--match hyb::]
                                                   [--dispatches PATTERN --min-value V]

Kernel-trace runs: per (kernel, grid) count, average / min / max duration.
Counter runs (--pmc): per (kernel, grid) the average of each collected counter per dispatch;
with --dispatches, every dispatch of the kernels matching PATTERN whose counter value is at least
V (used to pick the 1 GiB calibration copies out of the other copies of a run).
"""

import argparse
import sqlite3


def short(name):
    """Kernel name without the leading 'void ' and the argument list, at most 100 characters."""
    n = name[5:] if name.startswith("void ") else name
    depth = 0
    for k, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n[k:].startswith("(anonymous"):
            n = n[:k]
            break
    return n if len(n) <= 100 else n[:97] + "..."


def kernel_table(db, match):
    cur = db.cursor()
    rows = cur.execute(
        "select name, grid_x / workgroup_x, grid_y, workgroup_x, count(*), avg(end-start)/1000.0, "
        "min(end-start)/1000.0, max(end-start)/1000.0 from kernels where name like ? "
        "group by name, grid_x, grid_y order by name, grid_y", (f"%{match}%",)).fetchall()
    out = ["| kernel | grid (blocks) | block | dispatches | avg us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short(r[0])}` | {r[1]} x {r[2]} | {r[3]} | {r[4]} | {r[5]:.2f} | {r[6]:.2f} | {r[7]:.2f} |")
    return "\n".join(out)


def pmc_table(db, match):
    cur = db.cursor()
    cols = [r[1] for r in cur.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    q = (f"select {name_col}, grid_size, counter_name, count(*), avg(value) from counters_collection "
         f"where {name_col} like ? group by {name_col}, grid_size, counter_name order by {name_col}")
    rows = cur.execute(q, (f"%{match}%",)).fetchall()
    out = ["| kernel | grid (threads) | counter | dispatches | avg per dispatch |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short(r[0])}` | {r[1]} | {r[2]} | {r[3]} | {r[4]:.1f} |")
    return "\n".join(out)


def dispatch_table(db, match, min_value):
    cur = db.cursor()
    cols = [r[1] for r in cur.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    disp_col = "dispatch_id" if "dispatch_id" in cols else "rowid"
    q = (f"select {disp_col}, {name_col}, grid_size, counter_name, value from counters_collection "
         f"where {name_col} like ? and value >= ? order by {disp_col}")
    rows = cur.execute(q, (f"%{match}%", min_value)).fetchall()
    out = ["| dispatch | kernel | grid (threads) | counter | value |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r[0]} | `{short(r[1])}` | {r[2]} | {r[3]} | {r[4]:.1f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--pmc", action="store_true")
    ap.add_argument("--match", default="")
    ap.add_argument("--dispatches", default=None)
    ap.add_argument("--min-value", type=float, default=0.0)
    a = ap.parse_args()
    db = sqlite3.connect(a.db)
    if a.dispatches is not None:
        print(dispatch_table(db, a.dispatches, a.min_value))
    else:
        print(pmc_table(db, a.match) if a.pmc else kernel_table(db, a.match))


if __name__ == "__main__":
    main()
