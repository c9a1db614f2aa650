"""Summarise rocprofv3 results databases (rocpd SQLite) of this library's kernels.

    python -m exact_tiled_attention_08_amd.rocprof_summary DB [DB ...] --command "..." [--match fa::]

prints a short Markdown report: per-kernel dispatch counts and durations (kernel trace),
and per-dispatch counter values when the run collected PMC counters (--pmc).

    python -m exact_tiled_attention_08_amd.rocprof_summary traffic --kind fwd_bf16 --workload 3 \
        --kernel-fetch F.db --kernel-write W.db --copy-fetch CF.db --copy-write CW.db \
        --match fwd_bf16 --out profiles/hbm_traffic.json

turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a kernel into HBM bytes per launch,
scaling each counter by the factor that makes it read exactly 2^30 bytes for a plain
1 GiB device copy measured the same way, and records the result with the hash of the
kernel source it was taken on.

    python -m exact_tiled_attention_08_amd.rocprof_summary mfma DB --match fwd_bf16 --wgs 1024 \
        --workload 3 --command "..."

reports the matrix-core counters of a --pmc run (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16,
SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE): the MFMA busy fraction, the
bf16 MFMA FLOPs the hardware counted (MOPS x 512) next to the algorithmic FLOPs of the
workload, and both as rates over the kernel's average duration in the same run.
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


MARKER = "mfma_probe_kernel"  # bench.py launches it with one workgroup right before timed steps


def marker_ids(db: str):
    """Dispatch ids of the one-workgroup probe launches that mark timed regions, in order."""
    return sorted(did for name, _, grid, wg, *_, did in kernel_rows(db)
                  if MARKER in name and grid // max(1, wg) == 1)


def summarise(dbs, match: str | None, wgs: int | None = None, calls: tuple | None = None,
              after: tuple | None = None):
    """calls=(a, b): keep only dispatches a .. b-1 of each kernel and launch shape, in
    dispatch order (e.g. the timed launches after the warm-up ones). after=(i, n): keep only
    the first n dispatches of each kernel and launch shape that follow the i-th marker
    launch and precede the next one (0-based; bench.py issues one right before each leg's
    timed steps, after its warm-up, whose length depends on time)."""
    by = {}
    lo, hi = {}, {}
    if after is not None:
        for db in dbs:
            ids = marker_ids(db)
            if len(ids) <= after[0]:
                raise SystemExit(f"{db}: no marker launch number {after[0]}")
            lo[db] = ids[after[0]]
            hi[db] = ids[after[0] + 1] if after[0] + 1 < len(ids) else None
    for db in dbs:
        for name, dur, grid, wg, lds, vgpr, agpr, did in kernel_rows(db):
            # the leg's dispatches: after its marker and before the next leg's
            if after is not None and (did <= lo[db] or (hi[db] is not None and did >= hi[db])):
                continue
            if match and match not in name:
                continue
            if wgs is not None and grid // max(1, wg) != wgs:
                continue
            key = (_short(name), grid // max(1, wg))  # one row per kernel and launch shape
            ent = by.setdefault(key, {"d": [], "grid": grid, "wg": wg, "lds": lds,
                                      "vgpr": vgpr, "agpr": agpr})
            ent["d"].append((did, dur))
    for ent in by.values():
        ent["d"].sort()
        if calls is not None:
            ent["d"] = ent["d"][calls[0]:calls[1]]
        if after is not None:
            ent["d"] = ent["d"][:after[1]]
        ent["d"] = [dur for _, dur in ent["d"]]
    by = {k: e for k, e in by.items() if e["d"]}
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
        out += ["| kernel | calls | avg us | min us | max us | grid (WGs) | WG size | LDS B | "
                "VGPR (as reported) | AGPR |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        for (name, _), e in sorted(by.items(), key=lambda kv: -sum(kv[1]["d"])):
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


def _counter_mean(db: str, match: str, counter: str) -> float:
    _, counters = summarise([db], match)
    vals = [v for (name, c), vs in counters.items() if c == counter for v in vs]
    if not vals:
        raise SystemExit(f"no {counter} values for kernels matching {match!r} in {db}")
    return statistics.mean(vals)


def traffic_main(argv):
    import json
    import os
    from exact_tiled_attention_08_amd.provenance import source_hash
    ap = argparse.ArgumentParser(prog="rocprof_summary traffic")
    ap.add_argument("--kind", required=True)
    ap.add_argument("--workload", required=True, help="workload number, or a name such as 'varlen'")
    ap.add_argument("--match", required=True)
    ap.add_argument("--kernel-fetch", required=True)
    ap.add_argument("--kernel-write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-match", default="copyBuffer")
    ap.add_argument("--out", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)
    copy_bytes = float(1 << 30)
    f_copy = _counter_mean(a.copy_fetch, a.copy_match, "FETCH_SIZE") * 1024.0
    w_copy = _counter_mean(a.copy_write, a.copy_match, "WRITE_SIZE") * 1024.0
    fetch_factor, write_factor = copy_bytes / f_copy, copy_bytes / w_copy
    f = _counter_mean(a.kernel_fetch, a.match, "FETCH_SIZE") * 1024.0 * fetch_factor
    w = _counter_mean(a.kernel_write, a.match, "WRITE_SIZE") * 1024.0 * write_factor
    rec = {}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            rec = json.load(fh)
    rec[f"{a.kind}:{a.workload}"] = {
        "bytes_per_launch": f + w, "read_bytes": f, "write_bytes": w,
        "fetch_factor": fetch_factor, "write_factor": write_factor,
        "source_hash": source_hash(a.kind), "command": a.command}
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps(rec[f"{a.kind}:{a.workload}"], indent=1))


def kernel_mfma_count(w, br: int = 256, bc: int | None = None) -> int:
    """Exact number of v_mfma_f32_32x32x16_bf16 the bf16 prefill kernel issues for workload w:
    per wave (32 query rows of a 256-row workgroup), S of the first key tile in the prologue,
    PV + S for every further tile the wave sees, PV only for the workgroup's last tile.
    Compared with SQ_INSTS_VALU_MFMA_MOPS_BF16 it pins what one counted op is."""
    import math
    d = w.d
    bc = bc or (96 if d == 128 else 128)
    npv, ns = (d // 32) * (bc // 16), (bc // 32) * (d // 16)
    off = w.Nk - w.Nq
    total = 0
    for qt in range(math.ceil(w.Nq / br)):
        q0 = qt * br
        kv_end = min(w.Nk, min(q0 + br, w.Nq) - 1 + off + 1) if w.causal else w.Nk
        nt = math.ceil(kv_end / bc) if kv_end > 0 else 0
        for wv in range(br // 32):
            wq0 = q0 + 32 * wv
            if wq0 >= w.Nq or nt == 0:
                continue
            wkv = min(w.Nk, min(wq0 + 31, w.Nq - 1) + off + 1) if w.causal else w.Nk
            if wkv <= 0:
                continue
            c = ns
            c += sum(npv + ns for j in range(nt - 1) if j * bc < wkv)
            c += npv if (nt - 1) * bc < wkv else 0
            total += c
    return total * w.B * w.H


def mfma_main(argv):
    import os
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import workloads as W
    ap = argparse.ArgumentParser(prog="rocprof_summary mfma")
    ap.add_argument("db")
    ap.add_argument("--match", required=True)
    ap.add_argument("--wgs", type=int, default=None)
    ap.add_argument("--workload", type=int, required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--peak-tflops", type=float, default=2516.6)
    a = ap.parse_args(argv)
    by, counters = summarise([a.db], a.match, a.wgs)
    print(render(by, counters, a.command))
    if len(by) != 1:
        raise SystemExit(f"expected one kernel launch shape, found {len(by)}")
    (name, _), ent = next(iter(by.items()))
    dur_s = statistics.mean(ent["d"]) * 1e-9

    def mean(c):
        vals = [v for (n, cn), vs in counters.items() if cn == c for v in vs]
        return statistics.mean(vals) if vals else None

    w = W.WORKLOADS[a.workload]
    mops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    util = mean("MfmaUtil")
    out = ["| derived | value |", "|---|---|"]
    if util is not None:
        out.append(f"| MFMA busy (MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs)) | {util:.1f}% |")
    if mops is not None:
        hw = mops * 512.0
        out.append(f"| bf16 MFMA FLOPs counted per dispatch (MOPS x 512) | {hw:.4g} |")
        out.append(f"| algorithmic FLOPs per launch ({w.name}) | {w.flops:.4g} |")
        out.append(f"| counted / algorithmic | {hw / w.flops:.4f} |")
        n = kernel_mfma_count(w)
        out.append(f"| 32x32x16 MFMAs the kernel issues (from its loop structure) | {n} |")
        out.append(f"| counted MOPS / (64 x issued MFMAs): 1 means one MOP = 512 FLOP | "
                   f"{mops / (64.0 * n):.6f} |")
        out.append(f"| counted MFMA rate over the average duration | {hw / dur_s / 1e12:.1f} TFLOP/s "
                   f"({100 * hw / dur_s / 1e12 / a.peak_tflops:.1f}% of {a.peak_tflops}) |")
    out.append(f"| algorithmic rate over the average duration ({statistics.mean(ent['d']) / 1e3:.1f} us) | "
               f"{w.flops / dur_s / 1e12:.1f} TFLOP/s ({100 * w.flops / dur_s / 1e12 / a.peak_tflops:.1f}%) |")
    print("\n".join(out))


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "traffic":
        traffic_main(sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "mfma":
        mfma_main(sys.argv[2:])
        return
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("dbs", nargs="+")
    ap.add_argument("--command", required=True, help="the command that produced the database")
    ap.add_argument("--match", default=None, help="keep kernels whose name contains this")
    ap.add_argument("--wgs", type=int, default=None, help="keep launches of this many workgroups")
    ap.add_argument("--calls", default=None,
                    help="A:B keeps dispatches A .. B-1 of each kernel, in dispatch order")
    ap.add_argument("--after-marker", default=None,
                    help="I:N keeps the first N dispatches of each kernel after the I-th marker "
                         "launch (the timed steps of bench.py's I-th leg)")
    args = ap.parse_args()
    calls = tuple(int(x) for x in args.calls.split(":")) if args.calls else None
    after = tuple(int(x) for x in args.after_marker.split(":")) if args.after_marker else None
    by, counters = summarise(args.dbs, args.match, args.wgs, calls, after)
    text = render(by, counters, args.command)
    if calls:
        text = text.replace("| kernel | calls |", f"Dispatches {calls[0]} .. {calls[1] - 1} of each kernel "
                            "(in dispatch order) only.\n\n| kernel | calls |", 1)
    if after:
        text = text.replace("| kernel | calls |", f"The {after[1]} dispatches of each kernel that follow "
                            f"marker launch {after[0]} (the timed steps of that benchmark leg, after "
                            "its warm-up) only.\n\n| kernel | calls |", 1)
    print(text)


if __name__ == "__main__":
    main()
