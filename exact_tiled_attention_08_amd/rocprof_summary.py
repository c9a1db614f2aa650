"""Summarise a rocprofv3 results database (rocpd SQLite) of this library's kernels.

    python -m exact_tiled_attention_08_amd.rocprof_summary DB [DB ...] --command "..." [--match fa::]

Prints a short Markdown report: per-kernel dispatch counts and durations (kernel trace),
and per-dispatch counter values when the run collected PMC counters (--pmc).
"""
from __future__ import annotations

import argparse
import re
import sqlite3
import statistics


def _short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(fa::\w+\)$", "", name)
    return name.replace("void ", "")


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, duration, grid_x, workgroup_x, lds_size, vgpr_count, accum_vgpr_count, dispatch_id "
        "from kernels").fetchall()
    con.close()
    return rows


def counter_rows(db: str):
    con = sqlite3.connect(db)
    try:
        cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
        rows = con.execute("select * from counters_collection").fetchall()
    except sqlite3.Error:
        rows, cols = [], []
    con.close()
    return [dict(zip(cols, r)) for r in rows]


def summarise(dbs, match: str | None):
    by = {}
    for db in dbs:
        for name, dur, grid, wg, lds, vgpr, agpr, _ in kernel_rows(db):
            if match and match not in name:
                continue
            ent = by.setdefault(_short(name), {"d": [], "grid": grid, "wg": wg, "lds": lds,
                                               "vgpr": vgpr, "agpr": agpr})
            ent["d"].append(dur)
    counters = {}
    for db in dbs:
        for r in counter_rows(db):
            name = _short(str(r.get("kernel_name") or r.get("name") or ""))
            if match and match not in name and match not in str(r.get("kernel_name", "")):
                continue
            cname = r.get("counter_name")
            val = r.get("value", r.get("counter_value"))
            if cname is None or val is None:
                continue
            counters.setdefault((name, cname), []).append(float(val))
    return by, counters


def render(by, counters, command: str) -> str:
    out = ["# rocprofv3 summary", "", "Command:", "", "```", command, "```", ""]
    if by:
        out += ["| kernel | calls | avg us | min us | max us | grid (WGs) | WG size | LDS B | VGPR | AGPR |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        for name, e in sorted(by.items(), key=lambda kv: -sum(kv[1]["d"])):
            d = e["d"]
            out.append(f"| `{name}` | {len(d)} | {statistics.mean(d) / 1e3:.2f} | {min(d) / 1e3:.2f} | "
                       f"{max(d) / 1e3:.2f} | {e['grid'] // max(1, e['wg'])} | {e['wg']} | {e['lds']} | "
                       f"{e['vgpr']} | {e['agpr']} |")
        out.append("")
    if counters:
        out += ["| kernel | counter | dispatches | mean per dispatch | min | max |", "|---|---|---|---|---|---|"]
        for (name, cname), vals in sorted(counters.items()):
            out.append(f"| `{name}` | {cname} | {len(vals)} | {statistics.mean(vals):.6g} | "
                       f"{min(vals):.6g} | {max(vals):.6g} |")
        out.append("")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("dbs", nargs="+")
    ap.add_argument("--command", required=True, help="the command that produced the database")
    ap.add_argument("--match", default=None, help="keep kernels whose name contains this")
    args = ap.parse_args()
    by, counters = summarise(args.dbs, args.match)
    print(render(by, counters, args.command))


if __name__ == "__main__":
    main()
