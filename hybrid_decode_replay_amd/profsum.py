"""Summarise rocprofv3 CSV output into the short text files kept under profiles/.

Usage (after the rocprofv3 runs whose commands are passed in, for the record):
    python -m hybrid_decode_replay_amd.profsum trace KT_DIR OUT.md "COMMAND"
    python -m hybrid_decode_replay_amd.profsum traffic FETCH_DIR WRITE_DIR OUT.txt KERNEL GRID \\
        "FETCH_SIZE COMMAND" "WRITE_SIZE COMMAND"
KERNEL is a name with template arguments as rocprofv3 prints them (one instantiation,
e.g. "mamba2_step_kernel<8, 1, 1, true, 0, 0, 1>") or a bare name (all instantiations).

trace    per (kernel, grid size) call counts and durations from *_kernel_trace.csv of a
         `rocprofv3 --kernel-trace` run (one row per workload of the program).
mfma     flush-step MFMA use (MfmaUtil, MfmaFlopsF32) per (kernel, grid) from a
         `--pmc MfmaUtil MfmaFlopsF32 GRBM_GUI_ACTIVE` run:
             python -m hybrid_decode_replay_amd.profsum mfma PMC_DIR OUT.md "COMMAND"
sweep    the batch 1..512 table from `bench.py --sweep FILE`:
             python -m hybrid_decode_replay_amd.profsum sweep FILE OUT.md "COMMAND"
traffic  HBM bytes per launch of KERNEL dispatches with grid size GRID (threads), from
         *_counter_collection.csv of a `--pmc FETCH_SIZE` and a `--pmc WRITE_SIZE` run.
         Both counters are calibrated on the streaming-copy kernel of the same runs,
         which reads and writes 1 GiB: scale = known bytes / counter bytes.  Fold and
         non-fold dispatches are told apart by their write bytes, and the bytes of a
         16-step window (15 non-fold + 1 fold, per launch) are reported.
dram     the same kernel's L2-to-memory requests from TCC_EA0_RDREQ*/WRREQ* runs, scaled by
         the copy kernel's, against its algorithmic bytes per launch:
             python -m hybrid_decode_replay_amd.profsum dram RD_DIR WR_DIR OUT.txt KERNEL GRID \\
                 "READ COMMAND" "WRITE COMMAND" ALGORITHMIC_BYTES
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30
SOURCES = {
    "mamba2_step_kernel": ("mamba2_kernel.hpp", "mamba2.hip", "ckpt.hpp", "common.hpp", "stage.hpp", "rc.hpp"),
    "gdn_step_kernel": ("gdn_kernel.hpp", "gdn.hip", "ckpt.hpp", "common.hpp", "stage.hpp", "rc.hpp"),
    "conv_step_kernel": ("conv.hip", "ckpt.hpp", "common.hpp"),
}


def _one(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def short(name: str) -> str:
    base = name.split("(")[0]
    return base.replace("void ", "").replace("rs::", "")


def source_sha(kernel):
    h = hashlib.sha256()
    for f in SOURCES[kernel]:
        with open(os.path.join(ROOT, "hybrid_decode_replay_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def trace(kt_dir, out, command):
    rows = list(csv.DictReader(open(_one(os.path.join(kt_dir, "**", "*kernel_trace.csv")))))
    groups = {}
    for r in rows:
        key = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    lines = [f"# rocprofv3 kernel trace: {os.path.basename(out)[:-3]}", "",
             "Command (from the repository root; run under `cd /tmp && export TMPDIR=/tmp`):", "",
             f"    {command}", "",
             "Per (kernel, grid) -- one row per workload of the run; durations in microseconds.", "",
             "| kernel | workgroups x threads | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        if not name.startswith(("mamba2", "gdn", "conv", "stream", "book", "quantize", "logical", "tiles", "rc_")):
            continue
        lines.append(f"| `{name}` | {grid // wg} x {wg} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | "
                     f"{max(d):.1f} | {100 * sum(d) / total:.1f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(path, cname):
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != cname:
            continue
        key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
        out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def _matches(name, want):
    """A kernel given with template arguments matches exactly; a bare name matches every
    instantiation."""
    return name == want if "<" in want else name.split("<")[0] == want


def traffic(fetch_dir, write_dir, out, kernel, grid, fetch_cmd, write_cmd):
    grid = int(grid)
    fetch = counters(_one(os.path.join(fetch_dir, "**", "*counter_collection.csv")), "FETCH_SIZE")
    write = counters(_one(os.path.join(write_dir, "**", "*counter_collection.csv")), "WRITE_SIZE")

    def pick(d, name, g=None):
        vals = [v for (k, gg), vs in d.items() if _matches(k, name) and (g is None or gg == g) for v in vs]
        if not vals:
            raise KeyError((name, g))
        return vals

    cf, cw = pick(fetch, "stream_copy_kernel"), pick(write, "stream_copy_kernel")
    s_fetch = COPY_BYTES / (sum(cf) / len(cf) * 1024)
    s_write = COPY_BYTES / (sum(cw) / len(cw) * 1024)
    kf, kw = pick(fetch, kernel, grid), pick(write, kernel, grid)
    n = min(len(kf), len(kw))
    per = [kf[i] * 1024 * s_fetch + kw[i] * 1024 * s_write for i in range(n)]
    # fold dispatches write the checkpoint; the rest write only entries and outputs.  The two
    # runs dispatch in the same order, so dispatch i of one is dispatch i of the other.
    # Dispatches that fold only some sequences (staggered flush phases) write in between;
    # they are counted but left out of both classes.
    wmax, wmin = max(kw[:n]), min(kw[:n])
    split = wmax > 4 * max(wmin, 1e-9)
    fold = [per[i] for i in range(n) if split and kw[i] > 0.5 * wmax]
    rest = [per[i] for i in range(n) if not split or kw[i] < 2 * wmin]
    partial = n - len(fold) - len(rest)
    lines = [f"# HBM traffic of {kernel} (grid {grid} threads) from rocprofv3 --pmc runs",
             f"# FETCH_SIZE run: {fetch_cmd}",
             f"# WRITE_SIZE run: {write_cmd}",
             "# calibration: stream_copy_kernel reads and writes 1 GiB per dispatch",
             f"kernel = {kernel}",
             f"grid_threads = {grid}",
             f"kernel_source_sha = {source_sha(kernel.split('<')[0])}",
             f"dispatches = {n}",
             f"fetch_scale = {s_fetch:.4f}",
             f"write_scale = {s_write:.4f}",
             f"fetch_kib_per_dispatch_mean = {sum(kf[:n]) / n:.1f}",
             f"write_kib_per_dispatch_mean = {sum(kw[:n]) / n:.1f}",
             f"fetch_kib_per_dispatch_min_max = {min(kf[:n]):.1f} {max(kf[:n]):.1f}",
             f"write_kib_per_dispatch_min_max = {min(kw[:n]):.1f} {max(kw[:n]):.1f}",
             f"traffic_bytes_per_launch = {sum(per) / n:.0f}"]
    if fold and rest:
        nf, f = sum(rest) / len(rest), sum(fold) / len(fold)
        lines += [f"fold_dispatches = {len(fold)}",
                  f"partial_fold_dispatches = {partial}",
                  f"fold_bytes_per_launch = {f:.0f}",
                  f"nonfold_bytes_per_launch = {nf:.0f}",
                  "# a 16-step window: 15 non-fold steps and one fold step",
                  f"window_traffic_bytes_per_launch = {(15 * nf + f) / 16:.0f}"]
    else:
        lines.append(f"window_traffic_bytes_per_launch = {sum(per) / n:.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out, "traffic per launch", sum(per) / n)


def dram(rd_dir, wr_dir, out, kernel, grid, rd_cmd, wr_cmd, algorithmic_bytes):
    """Cross-check of the FETCH_SIZE / WRITE_SIZE scale on the replay kernel itself, from a run
    with --pmc TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_DRAM_sum and one with
    --pmc TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_EA0_WRREQ_DRAM_sum.  Request bytes are
    counted from the request sizes (32 or 64 bytes) without the bubble term; the same count is
    taken on the streaming copy kernel, which moves a known 1 GiB each way, and the ratio
    (known / counted) is applied to the kernel's counts.  The DRAM columns give the share of
    requests the L2 sends to memory (MC) rather than elsewhere."""
    grid = int(grid)
    rd_csv = _one(os.path.join(rd_dir, "**", "*counter_collection.csv"))
    wr_csv = _one(os.path.join(wr_dir, "**", "*counter_collection.csv"))

    def per_dispatch(path, names):
        d = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] in names:
                e = d.setdefault(int(r["Dispatch_Id"]), {"name": short(r["Kernel_Name"]), "grid": int(r["Grid_Size"])})
                e[r["Counter_Name"]] = float(r["Counter_Value"])
        return d

    rd = per_dispatch(rd_csv, ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_DRAM_sum"))
    wr = per_dispatch(wr_csv, ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum"))

    def rbytes(e):
        return (e["TCC_EA0_RDREQ_sum"] - e["TCC_EA0_RDREQ_32B_sum"]) * 64 + e["TCC_EA0_RDREQ_32B_sum"] * 32

    def wbytes(e):
        return (e["TCC_EA0_WRREQ_sum"] - e["TCC_EA0_WRREQ_64B_sum"]) * 32 + e["TCC_EA0_WRREQ_64B_sum"] * 64

    def sel(d, name, g=None):
        return [e for e in d.values() if _matches(e["name"], name) and (g is None or e["grid"] == g)]

    crd, cwr = sel(rd, "stream_copy_kernel"), sel(wr, "stream_copy_kernel")
    s_rd = COPY_BYTES / (sum(map(rbytes, crd)) / len(crd))
    s_wr = COPY_BYTES / (sum(map(wbytes, cwr)) / len(cwr))
    krd, kwr = sel(rd, kernel, grid), sel(wr, kernel, grid)
    n = min(len(krd), len(kwr))
    rb_, wb_ = [rbytes(e) * s_rd for e in krd[:n]], [wbytes(e) * s_wr for e in kwr[:n]]
    wmax = max(wb_)
    split = wmax > 4 * max(min(wb_), 1e-9)
    fold = [i for i in range(n) if split and wb_[i] > 0.5 * wmax]
    rest = [i for i in range(n) if not split or wb_[i] < 2 * min(wb_)]
    tot = [rb_[i] + wb_[i] for i in range(n)]
    win = (15 * sum(tot[i] for i in rest) / len(rest) + sum(tot[i] for i in fold) / len(fold)) / 16 \
        if fold and rest else sum(tot) / n
    dram_rd = sum(e["TCC_EA0_RDREQ_DRAM_sum"] for e in krd[:n]) / max(sum(e["TCC_EA0_RDREQ_sum"] for e in krd[:n]), 1)
    dram_wr = sum(e["TCC_EA0_WRREQ_DRAM_sum"] for e in kwr[:n]) / max(sum(e["TCC_EA0_WRREQ_sum"] for e in kwr[:n]), 1)
    alg = float(algorithmic_bytes)
    lines = [f"# L2-to-memory request cross-check of {kernel} (grid {grid} threads), rocprofv3 --pmc runs",
             f"# read-request run: {rd_cmd}",
             f"# write-request run: {wr_cmd}",
             "# request bytes = 64 x 64-byte requests + 32 x 32-byte requests, scaled by the copy kernel's known 1 GiB",
             f"kernel = {kernel}",
             f"grid_threads = {grid}",
             f"kernel_source_sha = {source_sha(kernel.split('<')[0])}",
             f"dispatches = {n}",
             f"read_scale_from_copy = {s_rd:.4f}",
             f"write_scale_from_copy = {s_wr:.4f}",
             f"dram_share_of_read_requests = {dram_rd:.4f}",
             f"dram_share_of_write_requests = {dram_wr:.4f}",
             f"window_request_bytes_per_launch = {win:.0f}",
             f"algorithmic_bytes_per_launch = {alg:.0f}",
             f"request_over_algorithmic = {win / alg:.4f}"]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out, "request bytes / algorithmic", win / alg)


def mfma(pmc_dir, out, command):
    """Flush-step MFMA use per (kernel, grid) from a `--pmc MfmaUtil MfmaFlops
    MfmaFlopsBF16 GRBM_GUI_ACTIVE` run.  A replay step issues MFMA only when it folds, so
    the dispatches with MfmaFlops > 0 are the flush steps.  MfmaFlops is rocprofv3's
    count over every MFMA type (512 per MOP); MfmaUtil its derived counter: MFMA busy
    cycles summed over SIMDs / (GUI-active cycles x SIMDs)."""
    per = {}
    for r in csv.DictReader(open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": short(r["Kernel_Name"]), "grid": int(r["Grid_Size"]),
                                                  "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    groups = {}
    for d in per.values():
        if d.get("MfmaFlops", 0.0) > 0 and d["name"].startswith(("mamba2", "gdn")):
            groups.setdefault((d["name"], d["grid"]), []).append(d)
    # full folds (every sequence of the batch folds: the most flops seen for the kernel and
    # grid) apart from partial ones (staggered flush phases, forced flushes of some sequences)
    split = {}
    for (name, grid), ds in groups.items():
        top = max(d["MfmaFlops"] for d in ds)
        full = [d for d in ds if d["MfmaFlops"] >= 0.999 * top]
        part = [d for d in ds if d["MfmaFlops"] < 0.999 * top]
        split[(name, grid, "full")] = full
        if part:
            split[(name, grid, "partial")] = part
    lines = [f"# MFMA use on fold (flush) dispatches: {os.path.basename(out)[:-3]}", "",
             "Command (from the repository root; run under `cd /tmp && export TMPDIR=/tmp`):", "",
             f"    {command}", "",
             "Dispatches with MfmaFlops > 0 (replay steps issue MFMA only when they fold).",
             "MfmaFlops: rocprofv3's count over all MFMA types, 512 per MOP, as the hardware counts them (a",
             "16x16x32 bf16 product counts its whole k = 32, zero and repeated operands included).",
             "MfmaUtil: rocprofv3's derived counter, MFMA busy cycles summed over SIMDs / (GUI-active cycles x SIMDs).",
             "TFLOP/s: MfmaFlops / the profiled dispatch duration (counter runs serialise dispatches).", "",
             "Full: every sequence folds (the largest MfmaFlops of the kernel and grid); partial: some do.", "",
             "| kernel | grid (threads) | folds | dispatches | MfmaFlops per dispatch | bf16 share | MfmaUtil % "
             "| profiled us | TFLOP/s |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid, kind), ds in sorted(split.items(), key=lambda kv: (kv[0][2], -kv[0][1], kv[0][0])):
        n = len(ds)
        fl = sum(d["MfmaFlops"] for d in ds) / n
        bf = sum(d.get("MfmaFlopsBF16", 0.0) for d in ds) / n
        ut = sum(d.get("MfmaUtil", 0.0) for d in ds) / n
        us = sum(d["ns"] for d in ds) / n / 1e3
        lines.append(f"| `{name}` | {grid} | {kind} | {n} | {fl:.4g} | {bf / fl:.2f} | {ut:.2f} | {us:.1f} "
                     f"| {fl / us / 1e6:.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out, len(split), "rows")


def sweep(jsonl, out, command):
    """Batch-sweep table from the JSON lines `bench.py --sweep FILE` writes (one per layer
    and batch size)."""
    import json
    rows = [json.loads(line) for line in open(jsonl) if line.strip()]
    lines = ["# Batch sweep: replay vs conventional fused decode, per decode step (MI355X, one GPU)", "",
             f"Command: `{command}`",
             "(per point: 64 timed steps after 16 warm-up steps; bf16 io, fp32 checkpoint, 16-entry buffer;",
             "Mamba-2 H=128 P=64 N=128 G=8; GDN 32 heads d=128).", "",
             "Two timings per point:", "",
             "* **graph** -- 64 back-to-back steps captured in one HIP graph, replayed 8 times (GPU time per step,",
             "  no host launch overhead); the same for the conventional kernel.",
             "* **eager** -- 64 steps launched one by one from Python, back to back between two events (both",
             "  kernels); the non-flush and flush columns come from a second pass with an event pair per launch.",
             "  Consecutive launches cycle through `rotate` copies of the layer state, so that they stream at",
             "  least 512 MiB of distinct state (more than the 256 MiB Infinity Cache holds); the GB/s column is",
             "  from these.  The graph timings use one state: at small batch it can stay in the Infinity Cache.", "",
             "| layer | batch | graph replay ms | graph conv ms | graph speedup | eager replay ms | eager conv ms "
             "| replay non-flush ms | replay flush ms | rotate | replay GB/s (algorithmic, whole windows) |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        g = r["graph"]
        lines.append(f"| {r['kind']} | {r['batch']} | {g['replay_ms_per_step']:.4f} | {g['conventional_ms_per_step']:.4f} "
                     f"| {g['speedup_vs_conventional']:.3f} | {r['ms_per_step']:.4f} | {r['conventional']['ms_per_step']:.4f} "
                     f"| {r['nonflush_step_ms']:.4f} | {r['flush_step_ms']:.4f} | {r.get('rotate', 1)} "
                     f"| {r['achieved_gbs']:.0f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out, len(rows), "points")


if __name__ == "__main__":
    mode, args = sys.argv[1], sys.argv[2:]
    if mode == "trace":
        trace(*args)
    elif mode == "traffic":
        traffic(*args)
    elif mode == "mfma":
        mfma(*args)
    elif mode == "dram":
        dram(*args)
    elif mode == "sweep":
        sweep(*args)
    else:
        raise SystemExit(__doc__)
