"""Benchmark: replayed SSM-layer decode on one MI355X.

Workload (default): the batch-256 hybrid-serving Mamba-2 layer -- B=256
sequences, H=128 heads, P=64, N=128, G=8 groups, fp32 checkpoint (4 MiB per
sequence), bf16 x/B/C/dt inputs and bf16 outputs, 16-entry buffer, decoding
from a random N(0, 0.1) checkpoint.  One step = one decode token for every
sequence of the layer (append, buffer scalars, checkpoint read-out, and on
every 16th step the fold with its single checkpoint write).  Inputs for every
timed step are drawn on the device before the timed region.

Printed: one JSON line with tokens/s (sequence-tokens per second for the
layer), the roofline of the replay kernel (algorithmic bytes / measured
per-launch time vs the 8 TB/s HBM peak), the in-run conventional fused decode
kernel on the same workload, a streaming-copy ceiling, and the fp64 CPU
oracle timed on the host's cores over a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "mamba2_step_b256_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "hybrid_decode_replay_amd", "csrc", f) for f in ("mamba2.hip", "common.hpp")]


def mamba2_algorithmic_bytes(B, H, G, P, N, cap=16, io_bytes=2):
    """Bytes the method must move per sequence-token, averaged over a full window of `cap`
    steps with lockstep flushes: checkpoint read every step, written once per window;
    current inputs x, B, C, dt; the new entry x, B, dt written; on average (cap-1)/2 prior
    entries read; output y."""
    S = H * P * N * 4
    entry = (H * P + G * N + H) * io_bytes
    inp = (H * P + 2 * G * N + H) * io_bytes
    out = H * P * io_bytes
    return S + S / cap + inp + entry + (cap - 1) / 2 * entry + out


def conv_algorithmic_bytes(B, H, G, P, N, io_bytes=2):
    S = H * P * N * 4
    inp = (H * P + 2 * G * N + H) * io_bytes
    return 2 * S + inp + H * P * io_bytes


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(units_per_launch):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source (else None)."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    kv = {}
    with open(PROFILE_TRAFFIC) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(B, H, G, P, N, budget_s=10.0, max_s=30.0):
    """The fp64 oracle (ordinary decoding, OpenMP over (sequence, head)) on a bounded sample of
    the same layer shape: 64 sequences (512 MiB of fp64 state, beyond any host cache), steps in
    chunks of 4 until >= budget_s of CPU time."""
    import numpy as np
    from hybrid_decode_replay_amd import synth
    from oracle import replay_oracle as ro
    nseq, chunk = 64, 4
    A, D = synth.mamba2_params(1, H)
    S = synth.checkpoint(1, (nseq, H, P, N)).astype(np.float64)
    elapsed, tokens, steps, c = 0.0, 0, 0, 0
    while elapsed < budget_s and elapsed < max_s:
        toks = synth.mamba2_tokens(100 + c, chunk, nseq, H, G, P, N, dtype="bf16")
        toks = {k: v.astype(np.float64) for k, v in toks.items()}
        t0 = time.perf_counter()
        for t in range(chunk):
            ro.mamba2_token(S, toks["x"][t], toks["Bm"][t], toks["Cm"][t], toks["dt"][t], A, D)
        elapsed += time.perf_counter() - t0
        tokens += nseq * chunk
        steps += chunk
        c += 1
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": ro.threads(), "kind": "oracle",
            "sample": f"{nseq} sequences x {steps} decode steps of the same layer shape (fp64 ordinary decoding, "
                      f"bf16-rounded inputs), {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--conv-steps", type=int, default=256, help="steps of the in-run conventional baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the decode path shards by "
              "sequence and head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_decode_replay_amd import binding as rb, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, G, P, N, cap = args.batch, 128, 8, 64, 128, 16
    K, W = args.steps, args.warmup
    cfg = rb.make_config(rb.MAMBA2, B, H, G, P, N, cap, rb.BF16)
    st = rb.ReplayState(cfg, device=dev)
    S0 = synth.checkpoint_device(1, (B, H, P, N), dev)
    st.load_checkpoint(S0)
    A, D = synth.mamba2_params(1, H)
    params = {"A": torch.from_numpy(A).to(dev), "D": torch.from_numpy(D).to(dev)}
    toks = synth.mamba2_tokens_device(1, K + W, B, H, G, P, N, dev)
    ys = torch.empty((2, 1, B, H, P), dtype=torch.bfloat16, device=dev)
    inputs = [rb.make_inputs(cfg, {k: v[t:t + 1] for k, v in toks.items()}, params) for t in range(K + W)]
    L = rb.lib()
    stream = torch.cuda.current_stream()
    sp = rb.ctypes.c_void_p(stream.cuda_stream)
    yptr = [rb.ctypes.c_void_p(ys[i].data_ptr()) for i in range(2)]

    def step(t):
        s = L.replay_decode_step(st.h, rb.ctypes.byref(inputs[t]), yptr[t & 1], sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "replay_decode_step")

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step(W + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in ev]                  # ms per launch
    total_ms = ev[0][0].elapsed_time(ev[-1][1])
    value = B * K / (total_ms / 1e3)
    lens_flush = [(W + i) % cap == cap - 1 for i in range(K)]
    flush_ms = [p for p, f in zip(per, lens_flush) if f]
    nonflush_ms = [p for p, f in zip(per, lens_flush) if not f]
    avg_ms = sum(per) / len(per)
    bytes_unit = mamba2_algorithmic_bytes(B, H, G, P, N, cap)
    achieved = bytes_unit * B / (avg_ms / 1e3) / 1e9
    traffic = read_traffic(B)
    del inputs, toks

    out = {
        "metric": "SSM-layer decode tokens/s at batch 256; achieved HBM GB/s vs MI355X peak",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, drawn on device; random checkpoint N(0,0.1))",
        "config": {"workload": "Mamba-2 SSM layer replayed decode", "batch": B, "nheads": H, "head_dim": P,
                   "state_dim": N, "ngroups": G, "buffer": cap, "checkpoint": "fp32", "io": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "mamba2_step_kernel", "algorithmic_bytes_per_launch": int(bytes_unit * B),
                     "avg_launch_ms": round(avg_ms, 5)},
        "split": {"flush_step_ms": round(sum(flush_ms) / max(1, len(flush_ms)), 5),
                  "nonflush_step_ms": round(sum(nonflush_ms) / max(1, len(nonflush_ms)), 5),
                  "bytes_per_token_algorithmic": int(bytes_unit)},
    }

    # streaming ceilings: 1 GiB -> 1 GiB copy and 1 GiB read, same stream
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        rb.stream_copy(dst, src, src.numel() * 4)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        rb.stream_copy(dst, src, src.numel() * 4)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * src.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9
    out["copy_ceiling_gbs"] = round(copy_gbs, 1)
    acc = torch.zeros(1, dtype=torch.float32, device=dev)
    for _ in range(3):
        rb.stream_read(src, src.numel() * 4, acc)
    e0.record(stream)
    for _ in range(10):
        rb.stream_read(src, src.numel() * 4, acc)
    e1.record(stream)
    torch.cuda.synchronize()
    out["read_ceiling_gbs"] = round(10 * src.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del src, dst

    if not args.no_conv:
        # in-run conventional fused decode (load, decay and update, output, store) on the same layer
        Kc = min(args.conv_steps, K)
        Sc = S0.clone()
        ctoks = synth.mamba2_tokens_device(2, Kc + 4, B, H, G, P, N, dev)
        cin = [rb.make_inputs(cfg, {k: v[t:t + 1] for k, v in ctoks.items()}, params) for t in range(Kc + 4)]
        cfgp = rb.ctypes.byref(cfg)
        Sp = rb.ctypes.c_void_p(Sc.data_ptr())
        for t in range(4):
            L.replay_conv_decode_step(cfgp, Sp, rb.ctypes.byref(cin[t]), yptr[0], sp)
        torch.cuda.synchronize()
        e0.record(stream)
        for t in range(Kc):
            s = L.replay_conv_decode_step(cfgp, Sp, rb.ctypes.byref(cin[4 + t]), yptr[t & 1], sp)
            if s != rb.OK:
                raise rb.ReplayError(s, "replay_conv_decode_step")
        e1.record(stream)
        torch.cuda.synchronize()
        conv_ms = e0.elapsed_time(e1) / Kc
        conv_bytes = conv_algorithmic_bytes(B, H, G, P, N)
        out["conventional"] = {"tokens_per_s": round(B / (conv_ms / 1e3), 1), "ms_per_step": round(conv_ms, 5),
                               "achieved_gbs": round(conv_bytes * B / (conv_ms / 1e3) / 1e9, 1),
                               "bytes_per_token_algorithmic": int(conv_bytes), "steps": Kc}
        out["replay_speedup_vs_conventional"] = round(conv_ms / (total_ms / K), 3)
        out["state_traffic_reduction_algorithmic"] = round(1 - bytes_unit / conv_bytes, 4)
        del Sc, ctoks, cin

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(B, H, G, P, N)
    out["wall_s_timed_region"] = round(wall, 3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
