"""Summarise a rocprofv3 run (rocpd SQLite output) into a short per-kernel table.

    python -m sparse_attention_hyb_amd.prof_summary <results.db> [--pmc] [--match hyb::]

Kernel-trace runs: per (kernel, grid) count, average / min / max duration.
Counter runs (--pmc): per (kernel, grid) the average of each collected counter per dispatch.
"""

import argparse
import sqlite3


def kernel_table(db, match):
    cur = db.cursor()
    rows = cur.execute(
        "select name, grid_x / workgroup_x, grid_y, workgroup_x, count(*), avg(end-start)/1000.0, "
        "min(end-start)/1000.0, max(end-start)/1000.0 from kernels where name like ? "
        "group by name, grid_x, grid_y order by name, grid_y", (f"%{match}%",)).fetchall()
    out = ["| kernel | grid (blocks) | block | dispatches | avg us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r[0].split('(')[0]}` | {r[1]} x {r[2]} | {r[3]} | {r[4]} | {r[5]:.2f} | {r[6]:.2f} | {r[7]:.2f} |")
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
        out.append(f"| `{r[0].split('(')[0]}` | {r[1]} | {r[2]} | {r[3]} | {r[4]:.1f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--pmc", action="store_true")
    ap.add_argument("--match", default="")
    a = ap.parse_args()
    db = sqlite3.connect(a.db)
    print(pmc_table(db, a.match) if a.pmc else kernel_table(db, a.match))


if __name__ == "__main__":
    main()
