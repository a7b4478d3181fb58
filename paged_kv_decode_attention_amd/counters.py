"""Summaries of rocprofv3 runs of the decode call.

    python -m paged_kv_decode_attention_amd.counters traffic \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-bytes N --config NAME --out FILE.json [--command CMD ...]
    python -m paged_kv_decode_attention_amd.counters trace \\
        --db FILE.db --out FILE.md --title TEXT --command CMD [--note TEXT ...] \\
        [--json FILE.json --sha HASH]
    python -m paged_kv_decode_attention_amd.counters compute \\
        --run DIR --out FILE.md --title TEXT --command CMD [--note TEXT ...]

traffic: HBM bytes of one decode call, from counter runs.

Each DIR holds the ``*_counter_collection.csv`` of one
``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) ``--output-format csv``
run.  The decode runs profile ``bench.py --decode-only``; the copy runs
profile ``bench.py --copy-calibration-mib M``, a plain copy of N = M MiB that
reads N bytes and writes N bytes.  The counters read in KiB per dispatch
and are not taken at face value: the copy kernel's reading of each counter
gives that counter's factor (true bytes per counted KiB), and every decode
kernel's reading is scaled by it.

The result is the bytes one decode call moves (its partition kernel plus its
merge kernel, averaged per dispatch), next to the algorithmic K/V bytes of
the same workload and the hash of the decode sources the runs were taken on.
"""

import argparse
import csv
import glob
import json
import os
import sys
from collections import defaultdict

# Kernels of a decode call, matched by substring of the demangled name.
DECODE_KERNELS = ("decode_mfma", "decode_generic", "merge_")
COPY_KERNEL = "copy_kernel"


def read_counter(run_dir, counter):
    """{kernel name: [per-dispatch values]} of one counter in one run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under " + run_dir)
    out = defaultdict(list)
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter:
                    out[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return out


def short_name(name):
    n = name.replace("void ", "").replace("pa::(anonymous namespace)::", "")
    return n.split("(")[0]


def per_dispatch(readings, keys):
    """Mean reading per dispatch of every kernel whose name holds one of keys."""
    res = {}
    for name, vals in readings.items():
        if any(k in name for k in keys):
            res[short_name(name)] = (sum(vals) / len(vals), len(vals))
    return res


def calibration(run_dir, counter, copy_bytes):
    vals = per_dispatch(read_counter(run_dir, counter), (COPY_KERNEL,))
    if len(vals) != 1:
        raise ValueError("expected one copy kernel in %s, found %s" % (run_dir, list(vals)))
    kib, _ = next(iter(vals.values()))
    return copy_bytes / kib


def trace_table(db):
    """(kernel, calls, avg us, min us, max us, share of traced kernel time)
    per kernel of a rocprofv3 --kernel-trace database, longest total first."""
    import sqlite3
    con = sqlite3.connect(db)
    try:
        rows = con.execute(
            "select name, count(*), avg(end - start), min(end - start), max(end - start), "
            "sum(end - start) from kernels group by name order by sum(end - start) desc"
        ).fetchall()
    finally:
        con.close()
    total = sum(r[5] for r in rows) or 1
    return [(short_name(r[0]), r[1], r[2] / 1e3, r[3] / 1e3, r[4] / 1e3, 100.0 * r[5] / total)
            for r in rows]


# Instruction and utilisation counters of one --pmc run (8 SQ counters and
# one derived metric fit one pass).
COMPUTE_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
                    "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD", "SQ_LDS_BANK_CONFLICT", "MfmaUtil")


def compute_main(a):
    """Per-dispatch means of the compute counters for every decode kernel,
    with instructions per wavefront derived from them."""
    data = {c: per_dispatch(read_counter(a.run, c), DECODE_KERNELS) for c in COMPUTE_COUNTERS}
    kernels = sorted(data["SQ_WAVES"], key=lambda k: -data["SQ_INSTS_VALU"].get(k, (0, 0))[0])
    lines = ["# " + a.title, "", "Command (repository root, one MI355X):", "",
             "    " + a.command, "",
             "Per dispatch (mean over dispatches):", "",
             "| kernel | dispatches | waves | VALU insts | MFMA insts | SALU insts | LDS insts "
             "| VMEM read insts | LDS bank conflict cycles | MFMA busy % |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for k in kernels:
        v = {c: data[c].get(k, (float("nan"), 0))[0] for c in COMPUTE_COUNTERS}
        lines.append("| %s | %d | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.2f |" % (
            k, data["SQ_WAVES"][k][1], v["SQ_WAVES"], v["SQ_INSTS_VALU"], v["SQ_INSTS_MFMA"],
            v["SQ_INSTS_SALU"], v["SQ_INSTS_LDS"], v["SQ_INSTS_VMEM_RD"],
            v["SQ_LDS_BANK_CONFLICT"], v["MfmaUtil"]))
    lines += ["", "Per wavefront:", "",
              "| kernel | VALU | MFMA | SALU | LDS | VMEM read |", "|---|---|---|---|---|---|"]
    for k in kernels:
        w = data["SQ_WAVES"][k][0] or float("nan")
        lines.append("| %s | %.0f | %.0f | %.0f | %.0f | %.0f |" % (
            k, data["SQ_INSTS_VALU"].get(k, (0, 0))[0] / w,
            data["SQ_INSTS_MFMA"].get(k, (0, 0))[0] / w,
            data["SQ_INSTS_SALU"].get(k, (0, 0))[0] / w,
            data["SQ_INSTS_LDS"].get(k, (0, 0))[0] / w,
            data["SQ_INSTS_VMEM_RD"].get(k, (0, 0))[0] / w))
    if a.note:
        lines += [""] + ["- " + t for t in a.note]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def trace_durations(db):
    """Sorted kernel durations (us) per kernel of a --kernel-trace database."""
    import sqlite3
    con = sqlite3.connect(db)
    try:
        rows = con.execute("select name, end - start from kernels").fetchall()
    finally:
        con.close()
    out = {}
    for name, ns in rows:
        out.setdefault(short_name(name), []).append(ns / 1e3)
    return {k: sorted(v) for k, v in out.items()}


def median(xs):
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def trace_main(a):
    lines = ["# " + a.title, "", "Command (repository root, one MI355X):", "",
             "    " + a.command, "",
             "| kernel | calls | avg us | min us | max us | % of traced kernel time |",
             "|---|---|---|---|---|---|"]
    for k, n, avg, lo, hi, share in trace_table(a.db):
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.1f |" % (k, n, avg, lo, hi, share))
    if a.note:
        lines += [""] + ["- " + t for t in a.note]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if a.json:
        # kernel-only durations for bench.py, tied to the decode sources
        rec = {"kernel_src_sha": a.sha, "command": a.command, "kernels": {
            k: {"calls": len(v), "avg_us": sum(v) / len(v), "median_us": median(v),
                "min_us": v[0], "max_us": v[-1]}
            for k, v in trace_durations(a.db).items()}}
        with open(a.json, "w") as fh:
            json.dump(rec, fh, indent=1)
    return 0


def write_traffic_md(rec, path, title):
    """Markdown summary of a traffic record: commands, calibration, per-kernel
    readings and the bytes per call against the algorithmic bytes."""
    lines = ["# " + title, "",
             "Commands (repository root, one MI355X; each counter in a run of its own):", ""]
    lines += ["    " + c for c in rec["commands"]]
    lines += ["",
              "Calibration: a plain %d-byte copy (reads and writes that many bytes) gives "
              "%.1f bytes per FETCH_SIZE KiB and %.1f bytes per WRITE_SIZE KiB." % (
                  rec["copy_calibration_bytes"], rec["fetch_factor_bytes_per_kib"],
                  rec["write_factor_bytes_per_kib"]), "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | "
              "written bytes |", "|---|---|---|---|---|---|"]
    for k, v in rec["kernels"].items():
        lines.append("| %s | %d | %.1f | %.1f | %.0f | %.0f |" % (
            k, v["dispatches"], v["fetch_kib"], v["write_kib"], v["fetch_bytes"],
            v["write_bytes"]))
    lines += ["", "Kernels counted: those whose name holds %s.  Per call: %.1f MB moved against "
              "%.1f MB of algorithmic K/V bytes (ratio %.3f).  Decode sources: kernel_src_sha "
              "%s." % (" or ".join(repr(k) for k in rec["kernel_filter"]),
                       rec["hbm_bytes_per_launch"] / 1e6, rec["alg_bytes_per_launch"] / 1e6,
                       rec["traffic_over_alg"], rec["kernel_src_sha"])]
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main(argv=None):
    top = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = top.add_subparsers(dest="cmd", required=True)
    tr = sub.add_parser("trace", help="kernel table of a --kernel-trace database")
    tr.add_argument("--db", required=True)
    tr.add_argument("--out", required=True)
    tr.add_argument("--title", required=True)
    tr.add_argument("--command", required=True)
    tr.add_argument("--note", action="append", default=[])
    tr.add_argument("--json", default=None)
    tr.add_argument("--sha", default=None)
    cp = sub.add_parser("compute", help="instruction counters of the decode kernels")
    cp.add_argument("--run", required=True)
    cp.add_argument("--out", required=True)
    cp.add_argument("--title", required=True)
    cp.add_argument("--command", required=True)
    cp.add_argument("--note", action="append", default=[])
    ap = sub.add_parser("traffic", help="HBM bytes per decode call from counter runs")
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-bytes", type=int, required=True)
    ap.add_argument("--config", default="qwen7b_gqa_bf16")
    ap.add_argument("--kernels", action="append", default=[],
                    help="count only kernels whose name holds one of these (repeatable; "
                         "default: every decode and merge kernel)")
    ap.add_argument("--alg-factor", type=float, default=1.0,
                    help="algorithmic bytes relative to the config's 16-bit K/V "
                         "(0.5 for 8-bit caches)")
    ap.add_argument("--out", required=True)
    ap.add_argument("--md", default=None, help="also write this markdown summary")
    ap.add_argument("--title", default=None)
    ap.add_argument("--command", action="append", default=[],
                    help="a command the readings came from (repeatable)")
    a = top.parse_args(argv)
    if a.cmd == "trace":
        return trace_main(a)
    if a.cmd == "compute":
        return compute_main(a)

    from . import inputs as I
    from .build import decode_source_hash

    f_fetch = calibration(a.copy_fetch, "FETCH_SIZE", a.copy_bytes)
    f_write = calibration(a.copy_write, "WRITE_SIZE", a.copy_bytes)
    keys = tuple(a.kernels) or DECODE_KERNELS
    fetch = per_dispatch(read_counter(a.fetch, "FETCH_SIZE"), keys)
    write = per_dispatch(read_counter(a.write, "WRITE_SIZE"), keys)
    if not fetch or set(fetch) != set(write):
        raise ValueError("decode kernels differ between runs: %s vs %s"
                         % (sorted(fetch), sorted(write)))
    kernels = {}
    total = 0.0
    for k in sorted(fetch):
        fb = fetch[k][0] * f_fetch
        wb = write[k][0] * f_write
        kernels[k] = {"dispatches": fetch[k][1], "fetch_kib": fetch[k][0],
                      "write_kib": write[k][0], "fetch_bytes": fb, "write_bytes": wb}
        total += fb + wb
    cfg = I.CONFIGS[a.config]
    alg = int(I.kv_bytes_read(cfg, I.draw_context_lens(cfg)) * a.alg_factor)
    rec = {
        "config": a.config,
        "kernel_filter": list(keys),
        "kernel_src_sha": decode_source_hash(),
        "hbm_bytes_per_launch": total,
        "alg_bytes_per_launch": alg,
        "traffic_over_alg": total / alg,
        "fetch_factor_bytes_per_kib": f_fetch,
        "write_factor_bytes_per_kib": f_write,
        "copy_calibration_bytes": a.copy_bytes,
        "kernels": kernels,
        "commands": a.command,
    }
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    if a.md:
        write_traffic_md(rec, a.md, a.title or "HBM traffic of the decode call, " + a.config)
    print(json.dumps({"hbm_bytes_per_launch": total, "alg": alg, "ratio": total / alg,
                      "fetch_factor": f_fetch, "write_factor": f_write}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
