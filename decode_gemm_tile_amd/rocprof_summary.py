"""Summarise rocprofv3 output databases into a short markdown table.

Usage:
  python -m decode_gemm_tile_amd.rocprof_summary trace <dir> [--title T] [--cmd C]
  python -m decode_gemm_tile_amd.rocprof_summary counters <dir> --kernel k_fused [--cmd C]
  python -m decode_gemm_tile_amd.rocprof_summary traffic <fetch_dir> <write_dir>
        --kernel k_fused --workload bf16_mlp --alg-bytes N --source-hash H [--cmd C]

`trace` lists kernel dispatch counts and durations (from --kernel-trace runs).
`counters` lists, for the named kernel, the median per dispatch of every
counter a --pmc run collected.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch, from two --pmc
runs) into HBM bytes per launch of the named kernel, each scaled by what the
same counter reads for the plain 512 MiB device copy that bench.py
--copy-calib performs (the copy reads and writes exactly 512 MiB).
"""

import argparse
import glob
import os
import sqlite3
import statistics
import sys

COPY_BYTES = 512 << 20


def _db(d):
    files = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not files:
        raise SystemExit("no rocprofv3 database under %s" % d)
    return sqlite3.connect(files[0])


def kernel_stats(d):
    cur = _db(d).cursor()
    rows = cur.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), "
                       "sum(end-start) from kernels group by name order by sum(end-start) desc")
    return rows.fetchall()


def counter_per_dispatch(d, counter):
    cur = _db(d).cursor()
    rows = cur.execute("select dispatch_id, name, sum(counter_value) from pmc_events "
                       "where counter_name = ? group by dispatch_id", (counter,)).fetchall()
    by_name = {}
    for _, name, v in rows:
        by_name.setdefault(name, []).append(v)
    return by_name


def _pick(by_name, needle):
    keys = [k for k in by_name if needle in k]
    if not keys:
        raise SystemExit("no dispatch matching %r (have: %s)" % (needle, list(by_name)[:5]))
    vals = by_name[keys[0]]
    # first dispatch is a warm-up of caches / TLB; use the median of the rest
    use = vals[1:] if len(vals) > 2 else vals
    return keys[0], statistics.median(use), len(vals)


def cmd_trace(args):
    st = kernel_stats(args.dir)
    print("# %s" % (args.title or "kernel trace"))
    print()
    if args.cmd:
        print("Command: `%s`" % args.cmd)
        print()
    if args.source_hash:
        print("- source hash: `%s`" % args.source_hash)
        print()
    print("| kernel | dispatches | avg us | min us | max us | total us |")
    print("|---|---|---|---|---|---|")
    for name, n, avg, mn, mx, tot in st[:12]:
        print("| `%s` | %d | %.2f | %.2f | %.2f | %.1f |" % (name[:110], n, avg / 1e3, mn / 1e3,
                                                            mx / 1e3, tot / 1e3))


def cmd_counters(args):
    cur = _db(args.dir).cursor()
    names = [r[0] for r in cur.execute("select distinct counter_name from pmc_events")]
    print("# Counters of `%s`%s" % (args.kernel, (" (%s)" % args.title) if args.title else ""))
    print()
    if args.cmd:
        print("Command: `%s`" % args.cmd)
        print()
    if args.source_hash:
        print("- source hash: `%s`" % args.source_hash)
        print()
    print("| counter | median per dispatch | dispatches |")
    print("|---|---|---|")
    for n in sorted(names):
        _, med, cnt = _pick(counter_per_dispatch(args.dir, n), args.kernel)
        print("| %s | %.6g | %d |" % (n, med, cnt))


def cmd_traffic(args):
    f = counter_per_dispatch(args.fetch_dir, "FETCH_SIZE")
    w = counter_per_dispatch(args.write_dir, "WRITE_SIZE")
    kname, kf, nf = _pick(f, args.kernel)
    _, kw, nw = _pick(w, args.kernel)
    cname, cf, _ = _pick(f, args.copy)
    _, cw, _ = _pick(w, args.copy)
    ff = COPY_BYTES / (cf * 1024.0)
    fw = COPY_BYTES / (cw * 1024.0)
    fetch = kf * 1024.0 * ff
    write = kw * 1024.0 * fw
    print("# HBM traffic of `%s` (%s)" % (args.kernel, args.workload))
    print()
    if args.cmd:
        print("Commands: `%s`" % args.cmd)
        print()
    print("- kernel: `%s` (%d / %d dispatches profiled, median used)" % (kname[:110], nf, nw))
    print("- calibration: `%s` copying 512 MiB read FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB "
          "-> factors %.4f (fetch), %.4f (write)" % (cname[:60], cf, cw, ff, fw))
    print("- kernel FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB per dispatch (raw)" % (kf, kw))
    print("- HBM bytes per launch (scaled): %.6e" % (fetch + write))
    print("- of which read %.6e, written %.6e" % (fetch, write))
    print("- algorithmic bytes per launch: %d (ratio traffic / algorithmic = %.3f)"
          % (args.alg_bytes, (fetch + write) / args.alg_bytes))
    print("- source hash: `%s`" % args.source_hash)


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", default="")
    t.add_argument("--cmd", default="")
    t.add_argument("--source-hash", default="")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--cmd", default="")
    c.add_argument("--source-hash", default="")
    r = sub.add_parser("traffic")
    r.add_argument("fetch_dir")
    r.add_argument("write_dir")
    r.add_argument("--kernel", required=True)
    r.add_argument("--copy", default="copyBuffer")
    r.add_argument("--workload", required=True)
    r.add_argument("--alg-bytes", type=int, required=True)
    r.add_argument("--source-hash", required=True)
    r.add_argument("--cmd", default="")
    args = p.parse_args(argv)
    if args.mode == "trace":
        cmd_trace(args)
    elif args.mode == "counters":
        cmd_counters(args)
    else:
        cmd_traffic(args)


if __name__ == "__main__":
    sys.exit(main())
