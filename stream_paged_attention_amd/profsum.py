"""Summaries of rocprofv3 output (its SQLite ``*_results.db`` files).

    python -m stream_paged_attention_amd.profsum trace DB
        per-kernel call count and mean / median / min duration
    python -m stream_paged_attention_amd.profsum counters DB
        mean of each collected counter per kernel
    python -m stream_paged_attention_amd.profsum traffic --workload NAME \\
            --kernel SUBSTR --fetch DB --write DB --copy-fetch DB --copy-write DB \\
            --copy-bytes N
        HBM bytes per launch of the matching kernel: FETCH_SIZE and WRITE_SIZE
        (KiB per dispatch), each scaled by the ratio of a plain copy's known
        bytes to what the same counter reads for it; the entry is written to
        profiles/traffic.json with the hash of the kernel sources it describes.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash() -> str:
    """Hash of the device sources: a counter entry is valid only for these."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if p.endswith((".hip", ".hpp")):
            with open(p, "rb") as f:
                h.update(os.path.basename(p).encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def _table(db, name):
    cols = [r[1] for r in db.execute(f"pragma table_info({name})")]
    return [dict(zip(cols, r)) for r in db.execute(f"select * from {name}")]


def kernel_durations(path: str) -> dict:
    db = sqlite3.connect(path)
    out = collections.defaultdict(list)
    for d in _table(db, "kernels"):
        out[d.get("kernel_name") or d.get("name")].append(d["end"] - d["start"])
    return out


def counter_values(path: str) -> dict:
    db = sqlite3.connect(path)
    out = collections.defaultdict(list)
    for d in _table(db, "counters_collection"):
        out[(d.get("kernel_name", "?"), d.get("counter_name"))].append(float(d.get("value")))
    return out


def trace_text(path: str) -> str:
    lines = [f"{'calls':>6} {'mean_us':>10} {'median_us':>10} {'min_us':>10}  kernel"]
    for name, durs in sorted(kernel_durations(path).items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(durs):6d} {statistics.mean(durs) / 1e3:10.3f} "
                     f"{statistics.median(durs) / 1e3:10.3f} {min(durs) / 1e3:10.3f}  {name}")
    return "\n".join(lines)


def counters_text(path: str) -> str:
    lines = [f"{'counter':24s} {'n':>4} {'mean':>16}  kernel"]
    for (k, c), vals in sorted(counter_values(path).items(), key=lambda kv: (kv[0][1], kv[0][0])):
        lines.append(f"{c:24s} {len(vals):4d} {statistics.mean(vals):16.1f}  {k}")
    return "\n".join(lines)


def _mean_for(path: str, counter: str, kernel: str) -> tuple[float, int]:
    vals = [v for (k, c), vs in counter_values(path).items()
            if c == counter and kernel in k for v in vs]
    if not vals:
        raise SystemExit(f"no {counter} values for a kernel matching {kernel!r} in {path}")
    return statistics.mean(vals), len(vals)


def _copy_kib(path: str, counter: str) -> float:
    """Largest mean of the counter over the copy run's kernels (the copy itself)."""
    best = 0.0
    for (k, c), vs in counter_values(path).items():
        if c == counter:
            best = max(best, statistics.mean(vs))
    if best <= 0:
        raise SystemExit(f"no {counter} values in {path}")
    return best


def traffic(args) -> dict:
    fetch_kib, nf = _mean_for(args.fetch, "FETCH_SIZE", args.kernel)
    write_kib, nw = _mean_for(args.write, "WRITE_SIZE", args.kernel)
    f_scale = args.copy_bytes / 1024.0 / _copy_kib(args.copy_fetch, "FETCH_SIZE")
    w_scale = args.copy_bytes / 1024.0 / _copy_kib(args.copy_write, "WRITE_SIZE")
    rd = fetch_kib * 1024.0 * f_scale
    wr = write_kib * 1024.0 * w_scale
    return {"kernel": args.kernel, "kernel_hash": kernel_hash(),
            "fetch_kib_raw": round(fetch_kib, 1), "write_kib_raw": round(write_kib, 1),
            "dispatches": [nf, nw], "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
            "read_bytes_per_launch": int(rd), "write_bytes_per_launch": int(wr),
            "hbm_bytes_per_launch": int(rd + wr)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("trace").add_argument("db")
    sub.add_parser("counters").add_argument("db")
    t = sub.add_parser("traffic")
    for k in ("workload", "kernel", "fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        print(trace_text(args.db))
    elif args.cmd == "counters":
        print(counters_text(args.db))
    else:
        entry = traffic(args)
        try:
            with open(TRAFFIC_FILE) as f:
                data = json.load(f)
        except (OSError, ValueError):
            data = {}
        data[args.workload] = entry
        os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
        print(json.dumps(entry))
    return 0


if __name__ == "__main__":
    sys.exit(main())
