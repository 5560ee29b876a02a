"""Summaries of rocprofv3 output databases (rocpd SQLite) for profiles/.

    python -m mamba_s6_selective_amd.rocprof_summary stats [--by-grid] RUN_results.db ...
        per-kernel call count and average / total duration (kernel trace);
        with --by-grid, one line per (kernel, grid size in work-items), so
        that launches of one kernel on different problem sizes stay apart

    python -m mamba_s6_selective_amd.rocprof_summary counters RUN_results.db
        per-kernel median over dispatches of every counter the run collected

    python -m mamba_s6_selective_amd.rocprof_summary traffic \\
        --fetch FETCH_results.db --write WRITE_results.db \\
        --kernel linear_scan_kernel --copy-bytes 1073741824 \\
        --source linear_scan.hip scan_common.h \\
        --out profiles/linear_scan_traffic.json
        HBM bytes per launch of a kernel (or summed over several kernels, one
        dispatch each: the passes of one call) from two counter runs
        (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled by
        the ratio of the bytes the copy kernel moves (copy_bytes read,
        copy_bytes written) to what the same counter reads for it.
        With --key NAME the record is merged into the --out file under NAME.
        With --largest-grid only each kernel's dispatches of its largest grid
        count (a run that also launches it on smaller problems).

    python -m mamba_s6_selective_amd.rocprof_summary valu VALU_results.db \\
        --kernel s6_chunk_kernel s6_carry_kernel s6_fix_kernel --tdn 1073741824 \\
        --source s6_scan.hip s6_internal.h --out profiles/s6_valu.json --key NAME
        Per kernel (median over dispatches): VALUBusy, and VALU and
        transcendental instructions per (b, t, d, n) element (wave
        instructions x 64 lanes / tdn), from a run that collected VALUBusy,
        SQ_INSTS_VALU, SQ_INSTS_VALU_TRANS_F32 and SQ_WAVES.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import sqlite3
import statistics
import sys
from collections import defaultdict
from pathlib import Path

CSRC = Path(__file__).resolve().parent / "csrc"
COPY_KERNEL = "copy_kernel"


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def kernel_stats(db: str, by_grid: bool = False):
    """[(name, calls, total_us, avg_us)], longest total first."""
    con = sqlite3.connect(db)
    if not by_grid:
        rows = con.execute("select name, total_calls, total_duration, average from top_kernels")
        return [(short_name(n), int(c), float(t), float(a)) for n, c, t, a in rows]
    rows = con.execute("select name, grid_x * grid_y * grid_z, count(*), sum(duration) "
                       "from kernels group by name, grid_x, grid_y, grid_z")
    out = [(f"{short_name(n)} [grid {g}]", int(c), float(t) / 1e3, float(t) / 1e3 / int(c))
           for n, g, c, t in rows]
    return sorted(out, key=lambda r: -r[2])


def counter_per_dispatch(db: str, counter: str):
    """{kernel short name: [(grid size, value) per dispatch]} for one counter."""
    con = sqlite3.connect(db)
    acc = defaultdict(float)
    names = {}
    for kname, disp, grid, cname, val in con.execute(
            "select kernel_name, dispatch_id, grid_size, counter_name, value "
            "from counters_collection"):
        if cname != counter:
            continue
        acc[disp] += float(val)
        names[disp] = (short_name(kname), int(grid))
    out = defaultdict(list)
    for disp, v in sorted(acc.items()):
        name, grid = names[disp]
        out[name].append((grid, v))
    return out


def source_sha(*files: str) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update((CSRC / f).read_bytes())
    return h.hexdigest()[:16]


def cmd_stats(args):
    width = 84 if args.by_grid else 64
    print(f"{'kernel':<{width}} {'calls':>6} {'avg_us':>10} {'total_us':>12}")
    for db in args.dbs:
        for name, calls, total, avg in kernel_stats(db, args.by_grid):
            print(f"{name[:width]:<{width}} {calls:>6} {avg:>10.2f} {total:>12.1f}")


def cmd_counters(args):
    con = sqlite3.connect(args.db)
    names = sorted({r[0] for r in con.execute(
        "select distinct counter_name from counters_collection")})
    per = {c: counter_per_dispatch(args.db, c) for c in names}
    kernels = sorted({k for d in per.values() for k in d})
    print(f"{'kernel':<64} " + " ".join(f"{c:>24}" for c in names))
    for k in kernels:
        vals = [statistics.median(v for _, v in per[c][k]) if per[c].get(k) else float("nan")
                for c in names]
        print(f"{k[:64]:<64} " + " ".join(f"{v:>24.4g}" for v in vals))


def pick(d, key, largest_grid=False):
    """Values of the dispatches of the first kernel whose name contains key
    (only those of its largest grid with largest_grid)."""
    hits = [k for k in d if key in k]
    if not hits:
        raise SystemExit(f"no dispatches of a kernel matching {key!r}: {sorted(d)}")
    disp = d[hits[0]]
    if largest_grid:
        top = max(g for g, _ in disp)
        disp = [(g, v) for g, v in disp if g == top]
    return [v for _, v in disp]


def cmd_traffic(args):
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    # one kernel, or the sum over the kernels of one step
    kf = sum(statistics.median(pick(fetch, k, args.largest_grid)) for k in args.kernel)
    kw = sum(statistics.median(pick(write, k, args.largest_grid)) for k in args.kernel)
    cf = statistics.median(pick(fetch, COPY_KERNEL))
    cw = statistics.median(pick(write, COPY_KERNEL))
    f_scale = args.copy_bytes / (cf * 1024.0)
    w_scale = args.copy_bytes / (cw * 1024.0)
    rec = {
        "kernel": args.kernel[0] if len(args.kernel) == 1 else args.kernel,
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "bytes_per_launch": kf * 1024.0 * f_scale + kw * 1024.0 * w_scale,
        "kernel_source_sha": source_sha(*args.source),
    }
    write_record(rec, args.out, args.key)


def write_record(rec, out, key):
    """Print rec; write it to out, or merge it into out under key."""
    text = json.dumps(rec, indent=1)
    if out and key:
        f = Path(out)
        d = json.loads(f.read_text()) if f.exists() else {}
        d[key] = rec
        f.write_text(json.dumps(d, indent=1) + "\n")
    elif out:
        Path(out).write_text(text + "\n")
    print(text)


def cmd_valu(args):
    per = {c: counter_per_dispatch(args.db, c)
           for c in ("VALUBusy", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVES")}
    kernels = {}
    for k in args.kernel:
        def med(c):
            return statistics.median(pick(per[c], k))
        kernels[k] = {"VALUBusy_pct": round(med("VALUBusy"), 2),
                      "valu_per_tdn": round(med("SQ_INSTS_VALU") * 64 / args.tdn, 4),
                      "trans_per_tdn": round(med("SQ_INSTS_VALU_TRANS_F32") * 64 / args.tdn, 4),
                      "waves": med("SQ_WAVES")}
    rec = {"kernels": kernels, "tdn": args.tdn, "kernel_source_sha": source_sha(*args.source)}
    write_record(rec, args.out, args.key)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--by-grid", action="store_true")
    s.add_argument("dbs", nargs="+")
    c = sub.add_parser("counters")
    c.add_argument("db")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, nargs="+",
                   help="kernel name (substring); several: bytes summed over one dispatch of each")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--source", required=True, nargs="+",
                   help="csrc files the kernel is built from (hashed in this order)")
    t.add_argument("--out")
    t.add_argument("--key")
    t.add_argument("--largest-grid", action="store_true")
    v = sub.add_parser("valu")
    v.add_argument("db")
    v.add_argument("--kernel", required=True, nargs="+", help="kernel names (substrings)")
    v.add_argument("--tdn", type=float, required=True,
                   help="(b, t, d, n) elements of one call (lane instructions are divided by it)")
    v.add_argument("--source", required=True, nargs="+")
    v.add_argument("--out")
    v.add_argument("--key")
    args = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "traffic": cmd_traffic,
     "valu": cmd_valu}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
