"""Summaries of rocprofv3 output for the measurement record.

    python -m block_diffusion_drafter_fwd_amd.profiling stats KERNEL_STATS_CSV [--trace KERNEL_TRACE_CSV]
        [--marker REGEX] [--command "..."] [--top N]
    python -m block_diffusion_drafter_fwd_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV
        --kernel REGEX [--command "..."] [--source FILE] [--out JSON]

``stats`` prints the per-kernel table of a ``--kernel-trace --stats`` run
(calls, average / min / max duration, share of GPU time) and, given the
trace, the per-round breakdown between consecutive launches of the
unembedding GEMM.  ``traffic`` turns two ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs into HBM bytes per launch of one kernel, each
counter scaled by what it reads for a plain copy of known size in the same
run (the 1 GiB copy and fill bench.py issues with --copy-calibration): a
copy of B bytes should fetch B and write B.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import re
import sys

COPY_BYTES = 1 << 30


def _short(name: str, width: int = 64) -> str:
    name = name.replace("dflash::kern::", "").replace("(GemmArgsT<4>)", "").replace("GemmArgsT<", "GA<")
    return name if len(name) <= width else name[:width - 3] + "..."


def stats(path: str, top: int = 25) -> str:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"{'kernel':64s} {'calls':>6s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'% time':>7s}"]
    for r in rows[:top]:
        out.append(f"{_short(r['Name']):64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{100 * float(r['TotalDurationNs']) / total:7.2f}")
    out.append(f"total GPU kernel time {total / 1e6:.3f} ms over {sum(int(r['Calls']) for r in rows)} launches")
    return "\n".join(out)


def per_round(trace: str, marker: str = r"k_gemm_skinny_p<4, 1") -> str:
    """Kernel time per round: rounds are delimited by launches of `marker`
    (the unembedding GEMM, once per round); the first 5 and last round are
    skipped (warm-up, tail)."""
    rows = list(csv.DictReader(open(trace)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    idx = [i for i, r in enumerate(rows) if re.search(marker, r["Kernel_Name"])]
    if len(idx) < 8:
        return "(too few rounds in the trace)"
    a, b = idx[5], idx[-2]
    seg = rows[a + 1:b + 1]
    nr = len(idx[5:-2])
    by = collections.defaultdict(list)
    for r in seg:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by[_short(r["Kernel_Name"], 56)].append(dur)
    busy = sum(sum(v) for v in by.values())
    span = int(seg[-1]["End_Timestamp"]) - int(rows[a]["End_Timestamp"])
    out = [f"per round over {nr} rounds: kernel busy {busy / nr / 1e3:.1f} us, span {span / nr / 1e3:.1f} us, "
           f"{len(seg) / nr:.1f} launches",
           f"{'kernel':56s} {'us/round':>9s} {'launches':>8s} {'median us':>9s}"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        out.append(f"{k:56s} {sum(v) / nr / 1e3:9.1f} {len(v) / nr:8.1f} {v[len(v) // 2] / 1e3:9.2f}")
    return "\n".join(out)


def _counter(path: str):
    return list(csv.DictReader(open(path)))


def traffic(fetch: str, write: str, kernel: str, source: str = None, copy_kernel: str = "copyBuffer") -> dict:
    def per_kernel(rows, counter, pattern):
        v = [float(r["Counter_Value"]) for r in rows
             if r["Counter_Name"] == counter and re.search(pattern, r["Kernel_Name"])]
        return v

    fr, wr = _counter(fetch), _counter(write)
    k_fetch = per_kernel(fr, "FETCH_SIZE", kernel)
    k_write = per_kernel(wr, "WRITE_SIZE", kernel)
    if not k_fetch or not k_write:
        raise SystemExit(f"no dispatches of /{kernel}/ in the counter files")
    # calibration: the largest dispatch of the copy kernel moved COPY_BYTES each way
    copy_fetch = max(per_kernel(fr, "FETCH_SIZE", copy_kernel))
    copy_write = max(per_kernel(wr, "WRITE_SIZE", copy_kernel))
    f_scale = COPY_BYTES / (copy_fetch * 1024.0)
    w_scale = COPY_BYTES / (copy_write * 1024.0)
    fk = sum(k_fetch) / len(k_fetch)
    wk = sum(k_write) / len(k_write)
    d = {"kernel_regex": kernel, "dispatches": len(k_fetch),
         "fetch_kib_per_dispatch_raw": round(fk, 1), "write_kib_per_dispatch_raw": round(wk, 1),
         "copy_fetch_kib_raw": copy_fetch, "copy_write_kib_raw": copy_write,
         "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
         "hbm_bytes_per_launch": int(round(fk * 1024 * f_scale + wk * 1024 * w_scale))}
    if source:
        d["source"] = source
        d["kernel_source_sha256_16"] = hashlib.sha256(open(source, "rb").read()).hexdigest()[:16]
    return d


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--trace")
    s.add_argument("--command", default="")
    s.add_argument("--top", type=int, default=25)
    s.add_argument("--marker", default=r"k_gemm_skinny_p<4, 1",
                   help="regex of the kernel launched once per round (the unembedding)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source")
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--command", default="")
    t.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        text = []
        if a.command:
            text.append(f"command: {a.command}")
        text.append(stats(a.csv, a.top))
        if a.trace:
            text.append("")
            text.append(per_round(a.trace, a.marker))
        print("\n".join(text))
    else:
        d = traffic(a.fetch, a.write, a.kernel, a.source, a.copy_kernel)
        if a.command:
            d["command"] = a.command
        js = json.dumps(d, indent=1)
        if a.out:
            open(a.out, "w").write(js + "\n")
        print(js)


if __name__ == "__main__":
    sys.exit(main())
