"""The profile summariser on small synthetic rocprofv3 outputs (CPU only).

The committed summaries under profiles/ and the `traffic` figure bench.py reports
come from these functions, so their arithmetic is checked here on inputs whose
answers are known: the copy-kernel calibration, per-launch bytes, the split of
fold dispatches into full and partial ones, and the sweep table."""
import csv
import json
import os

from hybrid_decode_replay_amd import profsum

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(did, name, grid, counter, value, ns=1000):
    return {"Dispatch_Id": did, "Grid_Size": grid, "Kernel_Name": name, "Counter_Name": counter,
            "Counter_Value": value, "Start_Timestamp": 0, "End_Timestamp": ns}


def _kv(path):
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    return kv


def test_traffic_calibrates_on_the_copy_kernel(tmp_path):
    copy = "void rs::stream_copy_kernel(f32x4 const*, f32x4*, unsigned long)"
    kern = "void rs::mamba2_step_kernel<8, 1, 1, true, 0, 0>(rs::StepArgs)"
    # the copy kernel moves 1 GiB each way; the counters read half of it on fetch
    _write_csv(str(tmp_path / "f" / "x_counter_collection.csv"), [
        _row(1, copy, 256, "FETCH_SIZE", 524288.0),
        _row(2, kern, 8388608, "FETCH_SIZE", 1000.0),
        _row(3, kern, 8388608, "FETCH_SIZE", 3000.0),
        _row(4, kern, 1024, "FETCH_SIZE", 7.0)])            # another grid: not counted
    _write_csv(str(tmp_path / "w" / "x_counter_collection.csv"), [
        _row(1, copy, 256, "WRITE_SIZE", 1048576.0),
        _row(2, kern, 8388608, "WRITE_SIZE", 10.0),
        _row(3, kern, 8388608, "WRITE_SIZE", 30.0),
        _row(4, kern, 1024, "WRITE_SIZE", 7.0)])
    out = str(tmp_path / "t.txt")
    profsum.traffic(str(tmp_path / "f"), str(tmp_path / "w"), out,
                    "mamba2_step_kernel<8, 1, 1, true, 0, 0>", 8388608, "F", "W")
    kv = _kv(out)
    assert float(kv["fetch_scale"]) == 2.0 and float(kv["write_scale"]) == 1.0
    assert int(kv["dispatches"]) == 2
    # mean over the two launches of (fetch KiB * 2 + write KiB * 1) * 1024
    assert float(kv["traffic_bytes_per_launch"]) == ((1000 + 3000) / 2 * 2 + (10 + 30) / 2) * 1024
    assert kv["kernel_source_sha"] == profsum.source_sha("mamba2_step_kernel")


def test_mfma_splits_full_and_partial_folds(tmp_path):
    kern = "void rs::gdn_step_kernel<8, 1, 1, 0, 0>(rs::StepArgs)"
    rows = []
    for did, flops, util in ((1, 0.0, 0.0), (2, 1.0e10, 30.0), (3, 1.0e10, 32.0), (4, 6.0e8, 3.0)):
        rows += [_row(did, kern, 4194304, "MfmaFlops", flops, ns=200000),
                 _row(did, kern, 4194304, "MfmaFlopsBF16", 0.75 * flops, ns=200000),
                 _row(did, kern, 4194304, "MfmaUtil", util, ns=200000)]
    _write_csv(str(tmp_path / "m" / "x_counter_collection.csv"), rows)
    out = str(tmp_path / "m.md")
    profsum.mfma(str(tmp_path / "m"), out, "CMD")
    table = [line for line in open(out) if line.startswith("| `")]
    full = [line for line in table if "| full |" in line]
    part = [line for line in table if "| partial |" in line]
    assert len(full) == 1 and len(part) == 1
    cells = [c.strip() for c in full[0].split("|")]
    # kernel, grid, kind, dispatches, flops, bf16 share, util, us, TFLOP/s
    assert cells[4] == "2" and float(cells[5]) == 1.0e10 and float(cells[6]) == 0.75 and float(cells[7]) == 31.0
    assert float(cells[8]) == 200.0 and float(cells[9]) == 50.0      # 1e10 flop / 200 us
    assert [c.strip() for c in part[0].split("|")][4] == "1"


def test_sweep_table_rows(tmp_path):
    jl = tmp_path / "s.jsonl"
    pts = []
    for kind, bsz in (("mamba2", 1), ("gdn", 256)):
        pts.append({"kind": kind, "batch": bsz, "ms_per_step": 0.1, "nonflush_step_ms": 0.09,
                    "flush_step_ms": 0.2, "achieved_gbs": 6000.4,
                    "conventional": {"ms_per_step": 0.2},
                    "graph": {"replay_ms_per_step": 0.1, "conventional_ms_per_step": 0.2,
                              "speedup_vs_conventional": 2.0}})
    jl.write_text("\n".join(json.dumps(p) for p in pts) + "\n")
    out = str(tmp_path / "s.md")
    profsum.sweep(str(jl), out, "CMD")
    rows = [line for line in open(out) if line.startswith("| mamba2") or line.startswith("| gdn")]
    assert len(rows) == 2
    assert [c.strip() for c in rows[1].split("|")][1:4] == ["gdn", "256", "0.1000"]
