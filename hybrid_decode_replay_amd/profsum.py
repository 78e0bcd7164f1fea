"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

Usage (after the rocprofv3 runs named in the summary headers):
    python -m hybrid_decode_replay_amd.profsum KT_DIR FETCH_DIR WRITE_DIR OUT_PREFIX \
        "KERNEL-TRACE COMMAND" "FETCH_SIZE COMMAND" "WRITE_SIZE COMMAND"

* KT_DIR holds *_kernel_stats.csv from `rocprofv3 --kernel-trace --stats`.
* FETCH_DIR / WRITE_DIR hold *_counter_collection.csv from `--pmc FETCH_SIZE` and
  `--pmc WRITE_SIZE` runs of the same program.
The counters are calibrated on the streaming-copy kernel of the same run, whose
bytes are known (it reads and writes 1 GiB): scale = known bytes / counter bytes.
The traffic per launch of the replay kernel is the mean over its dispatches of
FETCH*scale_fetch + WRITE*scale_write.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30


def _one(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def kernel_key(name: str) -> str:
    for key in ("mamba2_step_kernel", "gdn_step_kernel", "conv_step_kernel", "stream_copy_kernel",
                "stream_read_kernel", "book_commit_kernel", "conv_restore_kernel"):
        if key in name:
            return key
    return name.split("(")[0][:60]


def counters(path, cname):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != cname:
            continue
        out.setdefault(kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def source_sha(files):
    h = hashlib.sha256()
    for p in files:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main(kt_dir, fetch_dir, write_dir, prefix, command, fetch_cmd, write_cmd, kernel="mamba2_step_kernel",
         sources=("hybrid_decode_replay_amd/csrc/mamba2.hip", "hybrid_decode_replay_amd/csrc/common.hpp")):
    stats = list(csv.DictReader(open(_one(os.path.join(kt_dir, "**", "*kernel_stats.csv")))))
    fetch = counters(_one(os.path.join(fetch_dir, "**", "*counter_collection.csv")), "FETCH_SIZE")
    write = counters(_one(os.path.join(write_dir, "**", "*counter_collection.csv")), "WRITE_SIZE")
    cf = sum(fetch["stream_copy_kernel"]) / len(fetch["stream_copy_kernel"])
    cw = sum(write["stream_copy_kernel"]) / len(write["stream_copy_kernel"])
    s_fetch = COPY_BYTES / (cf * 1024)
    s_write = COPY_BYTES / (cw * 1024)
    kf, kw = fetch[kernel], write[kernel]
    n = min(len(kf), len(kw))
    per = [kf[i] * 1024 * s_fetch + kw[i] * 1024 * s_write for i in range(n)]
    traffic = sum(per) / n

    lines = [f"# rocprofv3 kernel trace: {os.path.basename(prefix)}", "",
             "Command (from the repository root; run under `cd /tmp && export TMPDIR=/tmp`):", "",
             f"    {command}", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats[:12]:
        lines.append(f"| {kernel_key(r['Name'])} `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    with open(prefix + "_kernel_trace.md", "w") as f:
        f.write("\n".join(lines) + "\n")

    sha = source_sha(sources)
    txt = [f"# HBM traffic of {kernel} from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (separate runs)",
           f"# FETCH_SIZE run: {fetch_cmd}",
           f"# WRITE_SIZE run: {write_cmd}",
           "# calibration: stream_copy_kernel reads and writes 1 GiB per dispatch",
           f"kernel = {kernel}",
           f"kernel_source_sha = {sha}",
           f"dispatches = {n}",
           f"copy_fetch_kib = {cf:.1f}",
           f"copy_write_kib = {cw:.1f}",
           f"fetch_scale = {s_fetch:.4f}",
           f"write_scale = {s_write:.4f}",
           f"fetch_kib_per_dispatch_mean = {sum(kf[:n]) / n:.1f}",
           f"write_kib_per_dispatch_mean = {sum(kw[:n]) / n:.1f}",
           f"fetch_kib_per_dispatch_min_max = {min(kf):.1f} {max(kf):.1f}",
           f"write_kib_per_dispatch_min_max = {min(kw):.1f} {max(kw):.1f}",
           f"traffic_bytes_per_launch = {traffic:.0f}"]
    for k in sorted(set(fetch) & set(write)):
        if k in (kernel, "stream_copy_kernel") or "at::" in k or k.startswith("void at"):
            continue
        fk, wk = fetch[k], write[k]
        m = min(len(fk), len(wk))
        t = sum(fk[i] * 1024 * s_fetch + wk[i] * 1024 * s_write for i in range(m)) / m
        txt.append(f"other.{k}.traffic_bytes_per_launch = {t:.0f}")
    with open(prefix + "_traffic.txt", "w") as f:
        f.write("\n".join(txt) + "\n")
    print(prefix, "traffic/launch", traffic)


if __name__ == "__main__":
    main(*sys.argv[1:8])
