"""Text summaries of rocprofv3 output (kernel statistics and PMC counters).

    python3 profile_summary.py counters DIR
        per-kernel totals of every counter in DIR/**/*counter_collection.csv
    python3 profile_summary.py traffic --fetch DIR --write DIR \\
            --kernel k_gateup --copy-bytes 1073741824 --source k_decode.hip [--last N] --out FILE.json
        HBM bytes per dispatch of one kernel from a FETCH_SIZE run and a WRITE_SIZE run.  Each
        counter is scaled by what it reads for the largest plain device-to-device copy in the same
        run (a copy of --copy-bytes bytes reads and writes exactly that many bytes).
    python3 profile_summary.py trace DIR --kernel 'k_gateup<0, 1>' --last 2560
    python3 profile_summary.py trace DIR --kernel 'k_gateup<1, 8, 1>' --skip-first 2 --first 128
        average duration of a kernel's dispatches in DIR/**/*kernel_trace.csv, over all of them and
        over a window by start time: the last N, or the first N after skipping some (the pass a
        bench times, e.g. its first one).

Counters are KiB per dispatch.  On gfx950 FETCH_SIZE reads about half of the bytes a copy
actually fetches, which is why every figure is calibrated against the copy instead of trusted raw.
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_name(raw):
    n = raw.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    return n.replace("eff::", "")


def source_sha(*names):
    """Same hash as the bench's source_sha: sha256 over the named csrc files, 16 hex digits."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "expert_ffn_serving_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_counters(d):
    """{(kernel, counter): [value per dispatch]} from a rocprofv3 --pmc csv directory."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % d)
    per = collections.defaultdict(float)
    for f in files:
        for r in csv.DictReader(open(f)):
            per[(kernel_name(r["Kernel_Name"]), r["Counter_Name"], r.get("Dispatch_Id", ""))] += float(r["Counter_Value"])
    out = collections.defaultdict(list)
    for (k, c, d), v in per.items():
        out[(k, c)].append((int(d) if str(d).isdigit() else 0, v))
    return out


def cmd_counters(a):
    data = read_counters(a.dir)
    print("kernel\tcounter\tdispatches\ttotal\tper_dispatch")
    for (k, c), dv in sorted(data.items()):
        v = [x for _, x in dv]
        print("%s\t%s\t%d\t%.6g\t%.6g" % (k, c, len(v), sum(v), sum(v) / len(v)))


def per_dispatch(data, counter, kernel, last=0):
    """Average of the kernel's dispatches (the last `last` of them by dispatch id, if > 0)."""
    vals = sorted((d, v) for (k, c), dv in data.items() if c == counter and k.startswith(kernel) for d, v in dv)
    if not vals:
        raise SystemExit("no %s dispatches of %s" % (counter, kernel))
    if last > 0:
        vals = vals[-last:]
    return sum(v for _, v in vals) / len(vals), len(vals)


def copy_factor(data, counter, copy_bytes):
    vals = [v for (k, c), dv in data.items() if c == counter and k.startswith(COPY_KERNEL) for _, v in dv]
    if not vals:
        raise SystemExit("no %s copy dispatch to calibrate against" % counter)
    return copy_bytes / (max(vals) * 1024.0)


def cmd_traffic(a):
    fd, wd = read_counters(a.fetch), read_counters(a.write)
    ff, wf = copy_factor(fd, "FETCH_SIZE", a.copy_bytes), copy_factor(wd, "WRITE_SIZE", a.copy_bytes)
    fk, nf = per_dispatch(fd, "FETCH_SIZE", a.kernel, a.last)
    wk, nw = per_dispatch(wd, "WRITE_SIZE", a.kernel, a.last)
    res = {
        "kernel": a.kernel,
        "hbm_bytes_per_launch": int(round(fk * 1024 * ff + wk * 1024 * wf)),
        "fetch_kib_per_dispatch": round(fk, 3), "write_kib_per_dispatch": round(wk, 3),
        "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
        "dispatches": [nf, nw], "copy_bytes": a.copy_bytes,
        "source_sha": source_sha(*a.source),
        "sources": a.source,
    }
    if a.command:
        res["command"] = a.command
    if a.note:
        res["note"] = a.note
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as o:
            o.write(text + "\n")
    print(text)


def read_trace(d):
    """{kernel: [(start_ns, duration_ns)]} from a rocprofv3 --kernel-trace csv directory."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit("no kernel_trace.csv under %s" % d)
    out = collections.defaultdict(list)
    for f in files:
        for r in csv.DictReader(open(f)):
            s, e = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            out[kernel_name(r["Kernel_Name"])].append((s, e - s))
    for v in out.values():
        v.sort()
    return out


def cmd_trace(a):
    data = read_trace(a.dir)
    names = [k for k in data if k.startswith(a.kernel)]
    if not names:
        raise SystemExit("no dispatches of %s" % a.kernel)
    res = {}
    for k in sorted(names):
        d = [x[1] for x in data[k]]
        head = d[:len(d) - a.skip] if a.skip > 0 else d
        if a.first > 0:   # a window from the start instead: skip_first dispatches, then `first` of them
            tail = head[a.skip_first:a.skip_first + a.first]
        else:
            tail = head[-a.last:] if a.last > 0 else head
        if not tail:
            raise SystemExit("no dispatches of %s left after skipping %d" % (k, a.skip))
        res[k] = {"dispatches": len(d), "avg_us": round(sum(d) / len(d) / 1e3, 3),
                  "skipped": a.skip, "skipped_first": a.skip_first, "window": len(tail),
                  "last": len(tail), "last_avg_us": round(sum(tail) / len(tail) / 1e3, 3),
                  "last_min_us": round(min(tail) / 1e3, 3), "last_max_us": round(max(tail) / 1e3, 3)}
    print(json.dumps(res, indent=1))
    return res


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--source", nargs="+", default=["k_decode.hip"])
    t.add_argument("--command", default="")
    t.add_argument("--note", default="")
    t.add_argument("--last", type=int, default=0, help="only the last N dispatches of the kernel")
    t.add_argument("--out", default="")
    r = sub.add_parser("trace")
    r.add_argument("dir")
    r.add_argument("--kernel", required=True)
    r.add_argument("--last", type=int, default=0)
    r.add_argument("--skip", type=int, default=0, help="leave out the last N dispatches before taking the window")
    r.add_argument("--first", type=int, default=0, help="window: the first N dispatches (after --skip-first)")
    r.add_argument("--skip-first", type=int, default=0)
    a = p.parse_args(argv)
    {"counters": cmd_counters, "traffic": cmd_traffic, "trace": cmd_trace}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
