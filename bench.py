"""Benchmark: replayed SSM-layer decode on one MI355X.

Headline workload: the batch-256 hybrid-serving Mamba-2 layer -- B=256
sequences, H=128 heads, P=64, N=128, G=8 groups, fp32 checkpoint (4 MiB per
sequence), bf16 x/B/C/dt inputs and bf16 outputs, 16-entry buffer, decoding
from a random N(0, 0.1) checkpoint.  One step = one decode token for every
sequence of the layer (append, buffer scalars, checkpoint read-out, and on
every 16th step the fold with its single checkpoint write).  Inputs for every
timed step are drawn on the device before the timed region.

The JSON line also carries:
  roofline      the replay kernel: algorithmic bytes per launch / measured
                per-launch time (HIP events on the launch stream) vs 8 TB/s
  mamba2        the headline layer in detail, with the in-run conventional
                fused load-decay-update-store kernel on the same layer
  gdn           the batch-256 Gated DeltaNet layer (32 heads, d_k = d_v = 128,
                bf16 q/k/v, fp32 gates), replay and conventional
  spec          speculative rounds at batch 512 (4 drafts per round, accepted
                prefix ~ min(Geometric(0.35) - 1, 4), seeded): replay append +
                commit vs the snapshot-per-draft + restore baseline, both layers
  gdn_read_copy_b128
                the batch-128 GDN layer with an fp32 checkpoint and no copy,
                an FP8 E4M3 read copy, and an MXFP4 read copy
  fp16_checkpoint
                both batch-256 layers with an fp16 recurrence checkpoint, and
                the conventional kernel on an fp16 state
  fp8_checkpoint
                both batch-256 layers with an FP8 E4M3 recurrence checkpoint,
                with no copy (the conventional kernel on an FP8 state beside
                it) and with an MXFP4 read copy
  flush_schedule_mamba2_b256
                per-step launch time (p50, p99, max) with lockstep folds and
                with staggered flush phases
  ragged_b256   both batch-256 layers with a seeded 75 % of the slots active per
                step (masked steps), and with 8 slots taking a fresh checkpoint
                every 16 steps; throughput over active tokens
  hybrid_stack_b256
                a model step over four SSM layers (Mamba-2, GDN, Mamba-2, GDN
                at the shapes above, batch 256) through one layer stack, with
                lockstep and staggered flush phases, against the conventional
                kernel per layer
  standin_kernels_b256
                per-launch time and algorithmic bandwidth of the stand-in
                non-SSM kernels (bf16 projections on MFMA, decode attention over
                a bf16 KV cache) at a model step's shapes
  hybrid_model_step_b256
                a synthetic hybrid decode step: the four SSM layers above
                interleaved with stand-in projections and attention (and
                optionally MLP projections), attention context 1024 or 4096;
                replay vs conventional SSM layers with identical stand-ins, the
                stand-ins' share of the step and the SSM speedup it implies
  flush_mfma    (in each layer report) the fold's MFMA flops per flush step and
                their rate over the measured flush-step time, against the
                fp32 MFMA peak (157.3 TFLOP/s)
  cpu_baseline  the fp64 oracle on the host cores over a bounded sample
With --sweep FILE, both layers are also timed at batch 1..512 (replay and
conventional, eagerly and as HIP-graph replays), one JSON line per point in FILE.

Timing.  Every decode timing starts with the W warm-up steps, then untimed
steps up to the next 16-step window boundary and two more full windows (so the
timed region starts warm and at a window boundary; the count is in the line as
`untimed_steps_before_timed_region`).  `value` and `ms_per_step` come from
exactly K steps launched back to back between two events on the launch stream.
`roofline.achieved` comes from a separate back-to-back pass over four whole
windows (64 steps: 60 non-fold and 4 fold steps), so its per-launch time has
the fold fraction the per-window algorithmic bytes assume, whatever K is; no
event sits between those launches.  A third pass with an event pair around each
launch gives the fold / non-fold split and the launch-time percentiles.

Working sets below 512 MiB per step (the batch sweep's small batches, the
batch-128 read copies) are decoded round-robin over several copies of the layer
state (`rotate`), so that a launch never finds its checkpoint or copy in the
256 MiB Infinity Cache left there by the previous launch.

Measured traffic comes from the committed rocprofv3 byte-counter summaries in
profiles/ (FETCH_SIZE + WRITE_SIZE, calibrated on a streaming copy of known
size), used only while the kernel sources still hash to the profiled version.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC = {("mamba2", "replay"): "mamba2_step_b256_traffic.txt", ("mamba2", "conv"): "conv_step_mamba2_b256_traffic.txt",
           ("gdn", "replay"): "gdn_step_b256_traffic.txt", ("gdn", "conv"): "conv_step_gdn_b256_traffic.txt"}

MAMBA2 = dict(H=128, G=8, C=64, R=128)     # heads, groups, head dim P, state dim N
GDN = dict(H=32, G=32, C=128, R=128)       # heads, q/k heads, d_v, d_k
ROTATE_MIN_BYTES = 512 << 20


def token_sizes(kind, H, G, C, R, io_bytes=2):
    """Bytes per sequence and token: (buffer entry, inputs read, output written).  Entries:
    Mamba-2 x, B, dt; GDN k, v and the fp32 gates; inputs add C (q)."""
    if kind == "mamba2":
        entry = (H * C + G * R + H) * io_bytes
        inp = (H * C + 2 * G * R + H) * io_bytes
    else:
        entry = (H * C + G * R) * io_bytes + 2 * H * 4
        inp = (H * C + 2 * G * R) * io_bytes + 2 * H * 4
    return entry, inp, H * C * io_bytes


def spec_bytes(kind, H, G, C, R, cap, k, acc, io_bytes=2, ckpt_bytes=4):
    """Algorithmic bytes of `len(acc)` speculative rounds of k drafts at accepted counts acc
    [rounds][B], and the per-sequence (len, folds) the bookkeeping must end with.  A round
    reads the checkpoint once, the committed entries once (staged for the outputs, or for
    the fold of the committed prefix when len + k > cap, which also writes the checkpoint),
    the k drafts' inputs, and writes their entries and outputs."""
    import numpy as np
    entry, inp, out = token_sizes(kind, H, G, C, R, io_bytes)
    S = H * C * R * ckpt_bytes
    rounds, B = acc.shape
    lens = np.zeros(B, np.int64)
    folds = np.zeros(B, np.int64)
    hist = 0
    for r in range(rounds):
        hist += int(lens.sum())
        f = lens + k > cap
        folds += f
        lens = np.where(f, 0, lens) + np.clip(acc[r], 0, k)
    total = rounds * B * (S + k * (inp + entry + out)) + hist * entry + int(folds.sum()) * S
    return total, lens, folds


def traffic_model(kind, H, G, C, R, cap=16, io_bytes=2, read_copy=None, ckpt_bytes=4):
    """Algorithmic bytes per sequence-token, by part: (replay, conventional) dicts.

    Replay, averaged over a full window of `cap` steps with lockstep flushes: the checkpoint
    is read every step and written once per window ("ckpt"); the new entry is written and on
    average (cap-1)/2 prior entries are read ("buffer"); the current inputs are read and the
    output written ("io").  With a read copy the cap-1 non-flush steps read the copy and the
    flush step reads and writes the checkpoint and writes the copy.  Conventional: the state
    is read and written every token ("state"), plus the same io.  Entries: Mamba-2 x, B, dt;
    GDN k, v and the fp32 gates.  S is the checkpoint (and conventional state) at
    ckpt_bytes per element."""
    n = H * C * R
    S = n * ckpt_bytes
    entry, inp, out = token_sizes(kind, H, G, C, R, io_bytes)
    ckpt = S + S / cap
    if read_copy is not None:
        copy = n if read_copy == "fp8" else n / 2 + n / 32
        ckpt = (cap - 1) / cap * copy + 2 * S / cap + copy / cap
    replay = {"ckpt": ckpt, "buffer": entry + (cap - 1) / 2 * entry, "io": inp + out}
    conv = {"state": 2 * S, "io": inp + out}
    return replay, conv


def algorithmic_bytes(kind, H, G, C, R, cap=16, io_bytes=2, read_copy=None, ckpt_bytes=4):
    """(replay, conventional) bytes per sequence-token (the sums of traffic_model)."""
    rep, conv = traffic_model(kind, H, G, C, R, cap, io_bytes, read_copy, ckpt_bytes)
    return sum(rep.values()), sum(conv.values())


def reductions(rep, conv):
    """Replay-vs-conventional traffic reduction under three accountings (1 - replay/conv):
    all bytes; state + buffer bytes (io excluded on both sides); checkpoint only (the
    buffer also excluded on the replay side)."""
    return {"all_bytes": round(1 - (rep["ckpt"] + rep["buffer"] + rep["io"]) / (conv["state"] + conv["io"]), 4),
            "state_and_buffer": round(1 - (rep["ckpt"] + rep["buffer"]) / conv["state"], 4),
            "checkpoint_only": round(1 - rep["ckpt"] / conv["state"], 4)}


def read_traffic(name):
    """Window bytes per launch from a committed rocprofv3 counter summary in profiles/, if it
    was taken on the current kernel source (else None)."""
    from hybrid_decode_replay_amd import profsum
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha") != profsum.source_sha(kv["kernel"].split("<")[0]):
            return None
        return float(kv.get("window_traffic_bytes_per_launch", kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError, OSError):
        return None


def measured_reduction(kind, B, rep_model, conv_model):
    """The replay-vs-conventional reduction from the measured counter bytes of both kernels
    (batch-256 layers), with the same three accountings; the io and buffer parts removed for
    the narrower ones are the algorithmic ones (the counters see only totals)."""
    r, c = read_traffic(TRAFFIC[(kind, "replay")]), read_traffic(TRAFFIC[(kind, "conv")])
    if r is None or c is None:
        return None
    r, c = r / B, c / B
    io, buf = rep_model["io"], rep_model["buffer"]
    return {"replay_bytes_per_token": round(r), "conventional_bytes_per_token": round(c),
            "all_bytes": round(1 - r / c, 4),
            "state_and_buffer": round(1 - (r - io) / (c - conv_model["io"]), 4),
            "checkpoint_only": round(1 - (r - io - buf) / (c - conv_model["io"]), 4),
            "source": f"profiles/{TRAFFIC[(kind, 'replay')]}, profiles/{TRAFFIC[(kind, 'conv')]} "
                      "(FETCH_SIZE + WRITE_SIZE per launch, 15:1 non-fold:fold window; io and buffer parts "
                      "algorithmic)"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(kind, nseq, budget_s, seed):
    """Tokens/s of the fp64 oracle (ordinary decoding) on nseq sequences of a layer shape."""
    import numpy as np
    from hybrid_decode_replay_amd import synth
    from oracle import replay_oracle as ro
    shp = MAMBA2 if kind == "mamba2" else GDN
    H, G, C, R = shp["H"], shp["G"], shp["C"], shp["R"]
    chunk = 4
    S = synth.checkpoint(seed, (nseq, H, C, R)).astype(np.float64)
    A, D = synth.mamba2_params(seed, H)
    elapsed, steps, c = 0.0, 0, 0
    while elapsed < budget_s:
        if kind == "mamba2":
            toks = synth.mamba2_tokens(100 + c, chunk, nseq, H, G, C, R, dtype="bf16")
        else:
            toks = synth.gdn_tokens(100 + c, chunk, nseq, H, G, R, C, dtype="bf16")
        toks = {k: v.astype(np.float64) for k, v in toks.items()}
        t0 = time.perf_counter()
        for t in range(chunk):
            if kind == "mamba2":
                ro.mamba2_token(S, toks["x"][t], toks["Bm"][t], toks["Cm"][t], toks["dt"][t], A, D)
            else:
                ro.gdn_token(S, toks["q"][t], toks["k"][t], toks["v"][t], toks["alpha"][t], toks["beta"][t])
        elapsed += time.perf_counter() - t0
        steps += chunk
        c += 1
    return nseq * steps / elapsed, steps, elapsed


def cpu_baseline(budget_s=8.0):
    """The fp64 oracle (ordinary decoding, OpenMP over (sequence, head)) on the host cores, on
    bounded samples: the headline Mamba-2 layer shape with 64 sequences (512 MiB of fp64 state,
    beyond any host cache) on every thread and on one, and the GDN layer shape on every thread;
    steps in chunks of 4 until about budget_s of wall time per leg."""
    from oracle import replay_oracle as ro
    threads = ro.threads()
    m2, m2_steps, m2_s = _oracle_rate("mamba2", 64, budget_s, 1)
    gd, gd_steps, gd_s = _oracle_rate("gdn", 64, 0.75 * budget_s, 2)
    ro.set_threads(1)
    try:
        one, one_steps, one_s = _oracle_rate("mamba2", 4, 0.5 * budget_s, 3)
    finally:
        ro.set_threads(threads)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"value": round(m2, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"64 sequences x {m2_steps} decode steps of the batch-256 Mamba-2 layer shape (fp64 ordinary "
                      f"decoding, bf16-rounded inputs), {m2_s:.1f} s on {threads} threads",
            "nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": _cpu_model(),
            "one_thread_tokens_per_s": round(one, 1),
            "one_thread_sample": f"4 sequences x {one_steps} steps, {one_s:.1f} s",
            "gdn_tokens_per_s": round(gd, 1),
            "gdn_sample": f"64 sequences x {gd_steps} steps of the batch-256 GDN layer shape, {gd_s:.1f} s "
                          f"on {threads} threads"}


class Layer:
    """Device-side state parameters and pre-drawn inputs of one synthetic layer.  The initial
    checkpoint is fp32; the library rounds it to the checkpoint dtype at load."""

    def __init__(self, rb, synth, torch, dev, kind, B, steps, seed, cap=16, read_copy=None, ckpt="f32", flags=0):
        self.rb, self.torch, self.dev, self.kind, self.B = rb, torch, dev, kind, B
        shp = MAMBA2 if kind == "mamba2" else GDN
        self.H, self.G, self.C, self.R = shp["H"], shp["G"], shp["C"], shp["R"]
        self.cap = cap
        self.read_copy = read_copy
        self.ckpt = ckpt
        rc = {None: rb.NONE, "fp8": rb.FP8_E4M3, "mxfp4": rb.MXFP4}[read_copy]
        self.cfg = rb.make_config(rb.MAMBA2 if kind == "mamba2" else rb.GDN, B, self.H, self.G, self.C, self.R,
                                  cap, rb.BF16, read_copy=rc, ckpt_dtype={"f16": rb.F16, "fp8": rb.FP8_E4M3}.get(ckpt, rb.F32),
                                  flags=flags)
        self.S0 = synth.checkpoint_device(seed, (B, self.H, self.C, self.R), dev)
        if kind == "mamba2":
            A, D = synth.mamba2_params(seed, self.H)
            self.params = {"A": torch.from_numpy(A).to(dev), "D": torch.from_numpy(D).to(dev)}
            self.toks = synth.mamba2_tokens_device(seed, steps, B, self.H, self.G, self.C, self.R, dev)
        else:
            self.params = {}
            self.toks = synth.gdn_tokens_device(seed, steps, B, self.H, self.G, self.R, self.C, dev)
        self.ntok = steps

    def inputs(self, t0, n=1):
        return self.rb.make_inputs(self.cfg, {k: v[t0:t0 + n] for k, v in self.toks.items()}, self.params)

    def state_bytes_per_step(self):
        """Bytes a non-fold step streams from the checkpoint or its read copy."""
        n = self.B * self.H * self.C * self.R
        if self.read_copy == "fp8":
            return n
        if self.read_copy == "mxfp4":
            return n // 2 + n // 32
        return n * {"f16": 2, "fp8": 1}.get(self.ckpt, 4)

    def conventional_state(self):
        """The plain logical state for the conventional kernel, in the checkpoint dtype, made by
        the library's own load rounding (a replay state loaded from S0, read back)."""
        st = self.rb.ReplayState(self.cfg, device=self.dev)
        st.load_checkpoint(self.S0)
        S = st.read_checkpoint()
        self.torch.cuda.synchronize()
        return S


def auto_rotate(L, cap_states=64):
    """Copies of the layer state a timing cycles through so that consecutive launches stream
    at least 512 MiB of distinct checkpoint (or read-copy) bytes."""
    return max(1, min(cap_states, -(-ROTATE_MIN_BYTES // L.state_bytes_per_step())))


class Stepper:
    """Decode steps of one layer issued back to back, round-robin over `rotate` states that
    all start from the layer's checkpoint.  Step n runs on state n % rotate with input n mod
    the number of drawn tokens; it is a fold step when that state's own step count
    n // rotate is the last of a window."""

    def __init__(self, L, stream, rotate=1):
        rb, torch = L.rb, L.torch
        self.L, self.rotate, self.cap = L, rotate, L.cap
        self.states = []
        for _ in range(rotate):
            st = rb.ReplayState(L.cfg, device=L.dev)
            st.load_checkpoint(L.S0)
            self.states.append(st)
        self.ys = torch.empty((2, 1, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev)
        self.ins = [L.inputs(t) for t in range(L.ntok)]
        self.lib, self.sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
        self.yp = [rb.ctypes.c_void_p(self.ys[i].data_ptr()) for i in range(2)]
        self.n = 0

    def step(self):
        rb = self.L.rb
        st = self.states[self.n % self.rotate]
        s = self.lib.replay_decode_step(st.h, rb.ctypes.byref(self.ins[self.n % len(self.ins)]), self.yp[self.n & 1],
                                        self.sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "replay_decode_step")
        self.n += 1

    def is_fold(self, n):
        return (n // self.rotate) % self.cap == self.cap - 1

    def align(self):
        """Untimed steps up to the next point where every state starts a window."""
        while self.n % (self.cap * self.rotate):
            self.step()


def time_replay_decode(L, K, W, stream, rotate=1, windows=4):
    """W warm-up steps, untimed steps to the next window boundary plus two full windows per
    state, then K timed steps back to back (the throughput); then, from a window boundary,
    `windows` whole windows per state back to back (the roofline's per-launch time), and two
    whole windows with an event pair around every launch (fold / non-fold split, percentiles)."""
    torch = L.torch
    sp = Stepper(L, stream, rotate)
    for _ in range(W):
        sp.step()
    sp.align()
    for _ in range(2 * sp.cap * rotate):
        sp.step()
    untimed = sp.n
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(K):
        sp.step()
    e1.record(stream)
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1)
    sp.align()
    nw = windows * sp.cap * rotate
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(nw):
        sp.step()
    e1.record(stream)
    torch.cuda.synchronize()
    window_ms = e0.elapsed_time(e1) / nw
    ne = 2 * sp.cap * rotate
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ne)]
    first = sp.n
    for i in range(ne):
        ev[i][0].record(stream)
        sp.step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    flush = [p for i, p in enumerate(per) if sp.is_fold(first + i)]
    nonflush = [p for i, p in enumerate(per) if not sp.is_fold(first + i)]
    srt = sorted(per)
    del sp
    return {"steps": K, "total_ms": total, "untimed_before": untimed, "window_ms_per_step": window_ms,
            "window_steps": nw, "rotate": rotate,
            "flush_ms": sum(flush) / max(1, len(flush)), "nonflush_ms": sum(nonflush) / max(1, len(nonflush)),
            "max_launch_ms": srt[-1], "p99_launch_ms": srt[min(ne - 1, int(0.99 * ne))], "p50_launch_ms": srt[ne // 2]}


def time_conv_decode(L, K, stream, t0=0, rotate=1):
    """K conventional decode steps back to back after 4 warm-up steps, round-robin over
    `rotate` copies of the state."""
    rb, torch = L.rb, L.torch
    Ss = [L.conventional_state() for _ in range(rotate)]
    y = torch.empty((1, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev)
    nin = min(L.ntok - t0, K + 4)
    ins = [L.inputs(t0 + t) for t in range(nin)]
    lib, sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
    cp, yp = rb.ctypes.byref(L.cfg), rb.ctypes.c_void_p(y.data_ptr())
    Sps = [rb.ctypes.c_void_p(S.data_ptr()) for S in Ss]

    def step(t):
        s = lib.replay_conv_decode_step(cp, Sps[t % rotate], rb.ctypes.byref(ins[t % nin]), yp, sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "replay_conv_decode_step")

    for t in range(4 * rotate):
        step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(K):
        step(4 * rotate + t)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def time_stack(layers, K, W, stream):
    """One model step = every layer's decode step in layer order through one ReplayStack
    (one bookkeeping set).  W warm-up model steps, then K timed back to back, then K more
    with an event pair around every model step (p50 / p99).  The conventional baseline
    runs one conventional decode step per layer on plain states, K model steps."""
    rb, torch = layers[0].rb, layers[0].torch
    lib, sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
    states = [rb.ReplayState(L.cfg, device=L.dev) for L in layers]
    stk = rb.ReplayStack(states)
    stk.load([L.S0 for L in layers])
    ys = [torch.empty((1, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev) for L in layers]
    yp = [rb.ctypes.c_void_p(y.data_ptr()) for y in ys]
    ins = [[L.inputs(t) for t in range(K + W)] for L in layers]

    def model_step(t):
        for i in range(len(layers)):
            s = lib.replay_stack_decode_layer(stk.h, i, rb.ctypes.byref(ins[i][t]), yp[i], sp)
            if s != rb.OK:
                raise rb.ReplayError(s, "replay_stack_decode_layer")

    for t in range(W):
        model_step(t)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        model_step(W + i)
    e1.record(stream)
    torch.cuda.synchronize()
    replay_ms = e0.elapsed_time(e1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        model_step(W + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    del stk, states
    conv_S = [L.S0.clone() for L in layers]
    cps = [rb.ctypes.byref(L.cfg) for L in layers]
    Sps = [rb.ctypes.c_void_p(S.data_ptr()) for S in conv_S]

    def conv_step(t):
        for i in range(len(layers)):
            s = lib.replay_conv_decode_step(cps[i], Sps[i], rb.ctypes.byref(ins[i][t]), yp[i], sp)
            if s != rb.OK:
                raise rb.ReplayError(s, "replay_conv_decode_step")

    for t in range(min(W, 4)):
        conv_step(t)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        conv_step(W + i)
    e1.record(stream)
    torch.cuda.synchronize()
    conv_ms = e0.elapsed_time(e1) / K
    B = layers[0].B
    return {"layers": [L.kind for L in layers], "batch": B, "replay_ms_per_model_step": round(replay_ms, 5),
            "replay_tokens_per_s": round(B / (replay_ms / 1e3), 1),
            "model_step_ms_p50": round(per[K // 2], 5), "model_step_ms_p99": round(per[min(K - 1, int(0.99 * K))], 5),
            "conventional_ms_per_model_step": round(conv_ms, 5),
            "speedup_vs_conventional": round(conv_ms / replay_ms, 3)}


def time_graph(L, conventional, n=64, reps=8):
    """Per-step GPU time of n back-to-back decode steps captured in one HIP graph (no host
    launch overhead and no events between steps), averaged over `reps` replays.  n is a
    multiple of the buffer capacity, so every replay covers whole windows and ends at the
    parity it began with."""
    rb, torch = L.rb, L.torch
    lib = rb.lib()
    ins = [L.inputs(t) for t in range(n)]
    y = torch.empty((1, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev)
    yp = rb.ctypes.c_void_p(y.data_ptr())
    if conventional:
        S = L.S0.clone()
        cp, Sp = rb.ctypes.byref(L.cfg), rb.ctypes.c_void_p(S.data_ptr())

        def step(t, sp):
            return lib.replay_conv_decode_step(cp, Sp, rb.ctypes.byref(ins[t]), yp, sp)
    else:
        st = rb.ReplayState(L.cfg, device=L.dev)
        st.load_checkpoint(L.S0)

        def step(t, sp):
            return lib.replay_decode_step(st.h, rb.ctypes.byref(ins[t]), yp, sp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # eager warm-up: one full pass
        for t in range(n):
            status = step(t, rb.ctypes.c_void_p(side.cuda_stream))
            if status != rb.OK:
                raise rb.ReplayError(status, "graph warm-up")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        sp = rb.ctypes.c_void_p(side.cuda_stream)
        for t in range(n):
            status = step(t, sp)
            if status != rb.OK:
                raise rb.ReplayError(status, "graph capture")
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n)
    del g
    return ms


D_MODEL = 4096
STANDIN_ATTN = dict(Hq=32, Hkv=8, D=128)


def standin_shapes(kind):
    """(in, out) projection widths of a mixer at d_model 4096: Mamba-2 in_proj to x, z, B, C, dt
    (2 H P + 2 G N + H) and out_proj from H P; GDN in_proj to q, k, v, an output gate and the two
    gates (4 H d + 2 H) and out_proj from H d_v; attention to q, k, v (Hq + 2 Hkv) D and o_proj
    from Hq D."""
    if kind == "mamba2":
        return 2 * MAMBA2["H"] * MAMBA2["C"] + 2 * MAMBA2["G"] * MAMBA2["R"] + MAMBA2["H"], MAMBA2["H"] * MAMBA2["C"]
    if kind == "gdn":
        return 4 * GDN["H"] * GDN["C"] + 2 * GDN["H"], GDN["H"] * GDN["C"]
    a = STANDIN_ATTN
    return (a["Hq"] + 2 * a["Hkv"]) * a["D"], a["Hq"] * a["D"]


def time_model_step(rb, synth, torch, dev, stream, B, context, mlp, K=32, W=8, d_ff=8192):
    """A synthetic hybrid decode step at batch B: mixers Mamba-2, GDN, attention, Mamba-2, GDN
    (the SSM layers at the shapes above, one layer stack), every mixer with its input and
    output projection (replay_standin_linear, bf16 random weights, d_model 4096), the attention
    layer reading a cache of `context` tokens per sequence (replay_standin_attention, 32 query
    and 8 key/value heads of 128), and with mlp=True a dense MLP after every mixer (d_model ->
    2 d_ff -> d_model as two products; the elementwise gate between them, under 1% of the
    bytes, is not run).  The SSM layers' inputs are drawn separately rather than sliced from
    the projection outputs: bytes and launches are those of a step, values are synthetic.
    Timed three ways over K model steps after W warm-up steps: with replayed SSM layers, with
    the conventional kernel in their place, and the stand-ins alone."""
    g = torch.Generator(device=dev).manual_seed(77 + context + (1 if mlp else 0))

    def weight(n_out, n_in):
        return (torch.randn((n_out, n_in), generator=g, device=dev) * n_in ** -0.5).to(torch.bfloat16)

    pattern = ["mamba2", "gdn", "attn", "mamba2", "gdn"]
    ssm = [Layer(rb, synth, torch, dev, k, B, K + W, seed=60 + i) for i, k in enumerate(p for p in pattern if p != "attn")]
    Wt = []
    for kind in pattern:
        n_in, n_out = standin_shapes(kind)
        Wt.append((weight(n_in, D_MODEL), weight(D_MODEL, n_out)))
    Wm = [(weight(2 * d_ff, D_MODEL), weight(D_MODEL, d_ff)) for _ in pattern] if mlp else None
    a = STANDIN_ATTN
    Kc = torch.randn((B, a["Hkv"], context, a["D"]), generator=g, device=dev).to(torch.bfloat16)
    Vc = torch.randn((B, a["Hkv"], context, a["D"]), generator=g, device=dev).to(torch.bfloat16)
    X = torch.randn((B, D_MODEL), generator=g, device=dev).to(torch.bfloat16)
    proj = {kind: torch.empty((B, standin_shapes(kind)[0]), dtype=torch.bfloat16, device=dev) for kind in set(pattern)}
    att_o = torch.empty((B, a["Hq"], a["D"]), dtype=torch.bfloat16, device=dev)
    X2 = torch.empty_like(X)
    up = torch.empty((B, 2 * d_ff), dtype=torch.bfloat16, device=dev) if mlp else None
    # the down projection's input stands for the gated activation of `up`; the elementwise
    # gate itself (B x d_ff bf16, ~1 % of an MLP's bytes) is not computed in either run
    act = torch.randn((B, d_ff), generator=g, device=dev).to(torch.bfloat16) if mlp else None
    ys = [torch.empty((1, L.B, L.H, L.C), dtype=torch.bfloat16, device=dev) for L in ssm]
    lib, sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
    states = [rb.ReplayState(L.cfg, device=dev) for L in ssm]
    stk = rb.ReplayStack(states)
    stk.load([L.S0 for L in ssm])
    conv_S = [L.conventional_state() for L in ssm]
    ins = [[L.inputs(t) for t in range(K + W)] for L in ssm]
    ptr = rb.ctypes.c_void_p

    def lin(x, w, y):
        st = lib.replay_standin_linear(ptr(x.data_ptr()), ptr(w.data_ptr()), ptr(y.data_ptr()), x.shape[0],
                                       w.shape[1], w.shape[0], sp)
        if st != rb.OK:
            raise rb.ReplayError(st, "replay_standin_linear")

    def step(t, mode):
        li = 0
        for pos, kind in enumerate(pattern):
            w_in, w_out = Wt[pos]
            lin(X, w_in, proj[kind])
            if kind == "attn":
                st = lib.replay_standin_attention(ptr(proj["attn"].data_ptr()), proj["attn"].shape[1],
                                                  ptr(Kc.data_ptr()), ptr(Vc.data_ptr()), ptr(att_o.data_ptr()), B,
                                                  a["Hq"], a["Hkv"], a["D"], context, float(a["D"] ** -0.5), sp)
                if st != rb.OK:
                    raise rb.ReplayError(st, "replay_standin_attention")
                lin(att_o.view(B, -1), w_out, X2)
            else:
                if mode == "replay":
                    st = lib.replay_stack_decode_layer(stk.h, li, rb.ctypes.byref(ins[li][t]), ptr(ys[li].data_ptr()), sp)
                elif mode == "conv":
                    st = lib.replay_conv_decode_step(rb.ctypes.byref(ssm[li].cfg), ptr(conv_S[li].data_ptr()),
                                                     rb.ctypes.byref(ins[li][t]), ptr(ys[li].data_ptr()), sp)
                else:
                    st = rb.OK
                if st != rb.OK:
                    raise rb.ReplayError(st, "SSM layer")
                lin(ys[li].view(B, -1), w_out, X2)
                li += 1
            if mlp:
                w_up, w_down = Wm[pos]
                lin(X2, w_up, up)
                lin(act, w_down, X)

    def timed(mode):
        for t in range(W):
            step(t, mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(K):
            step(W + t, mode)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    rep, conv, rest = timed("replay"), timed("conv"), timed("standins")
    del stk, states
    return {"pattern": pattern, "batch": B, "attention_context": context, "mlp_d_ff": d_ff if mlp else None,
            "replay_ms_per_model_step": round(rep, 4), "conventional_ms_per_model_step": round(conv, 4),
            "standins_alone_ms": round(rest, 4), "speedup_vs_conventional": round(conv / rep, 3),
            "standin_share_of_replay_step": round(rest / rep, 3),
            "ssm_speedup_implied": round((conv - rest) / max(rep - rest, 1e-9), 3),
            "replay_tokens_per_s": round(B / (rep / 1e3), 1)}


def time_ragged(L, K, W, stream, p_active=0.75, arrive_every=16, n_arrive=8, seed=11):
    """A serving batch whose slots come and go: every step a seeded mask marks each slot
    active with probability p_active (masked decode); in a second run, n_arrive slots also
    take a fresh fp32 checkpoint (a prefill hand-over) every arrive_every steps.  K steps
    back to back after W untimed ones; throughput counts active tokens only, and the
    algorithmic bytes are the layer's per-token window bytes times the active tokens (a
    sequence folds once per window of its own steps)."""
    import numpy as np
    rb, torch = L.rb, L.torch
    rng = np.random.default_rng(seed)
    masks_np = (rng.random((K + W, L.B)) < p_active).astype(np.uint8)
    masks = torch.from_numpy(masks_np).to(L.dev)
    lib, sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
    ins = [L.inputs(t % L.ntok) for t in range(K + W)]
    y = torch.empty((1, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev)
    yp = rb.ctypes.c_void_p(y.data_ptr())
    arrivals = [np.sort(rng.choice(L.B, n_arrive, replace=False)).astype(np.int32) for _ in range((K + W) // arrive_every + 1)]
    fresh = L.S0[:n_arrive].clone()
    out = {"batch": L.B, "p_active": p_active}
    for label, arrive in (("masked", False), ("masked_with_arrivals", True)):
        st = rb.ReplayState(L.cfg, device=L.dev)
        st.load_checkpoint(L.S0)
        torch.cuda.synchronize()

        def step(t):
            if arrive and t % arrive_every == 0:
                arr = arrivals[t // arrive_every]
                s = lib.replay_load_slots(st.h, n_arrive, arr.ctypes.data_as(rb.ctypes.POINTER(rb.ctypes.c_int32)),
                                          rb.ctypes.c_void_p(fresh.data_ptr()), sp)
                if s != rb.OK:
                    raise rb.ReplayError(s, "replay_load_slots")
            s = lib.replay_decode_step_masked(st.h, rb.ctypes.byref(ins[t]), rb.ctypes.c_void_p(masks[t].data_ptr()),
                                              yp, sp)
            if s != rb.OK:
                raise rb.ReplayError(s, "replay_decode_step_masked")

        for t in range(W):
            step(t)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(W, W + K):
            step(t)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        act = int(masks_np[W:].sum())
        per_tok = algorithmic_bytes(L.kind, L.H, L.G, L.C, L.R, L.cap)[0]
        r = {"ms_per_step": round(ms, 5), "active_tokens_per_step": round(act / K, 1),
             "active_tokens_per_s": round(act / (ms * K / 1e3), 1)}
        if not arrive:
            gbs = act * per_tok / (ms * K / 1e3) / 1e9
            r.update({"achieved_gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)})
        else:
            r["arrivals"] = f"{n_arrive} slots every {arrive_every} steps"
        out[label] = r
        del st
    return out


def time_standins(rb, torch, dev, stream, B=256, reps=20):
    """Per-launch time and algorithmic bandwidth of the stand-in kernels at the model step's
    shapes: weights (and activations) for the projections, the cache for attention."""
    g = torch.Generator(device=dev).manual_seed(91)
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for name, (n_in, n_out) in (("mamba2_in_proj", (D_MODEL, standin_shapes("mamba2")[0])),
                                ("mamba2_out_proj", (standin_shapes("mamba2")[1], D_MODEL)),
                                ("attn_o_proj", (STANDIN_ATTN["Hq"] * STANDIN_ATTN["D"], D_MODEL))):
        X = torch.randn((B, n_in), generator=g, device=dev).to(torch.bfloat16)
        Wt = torch.randn((n_out, n_in), generator=g, device=dev).to(torch.bfloat16)
        Y = torch.empty((B, n_out), dtype=torch.bfloat16, device=dev)
        ms = run(lambda: rb.standin_linear(X, Wt, Y))
        nbytes = 2 * (n_out * n_in + B * n_in + B * n_out)
        out[name] = {"M": B, "K": n_in, "N": n_out, "ms": round(ms, 5), "gbs": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "tflops": round(2 * B * n_in * n_out / (ms / 1e3) / 1e12, 1)}
        del X, Wt, Y
    a = STANDIN_ATTN
    for L in (1024, 4096):
        q = torch.randn((B, a["Hq"] * a["D"]), generator=g, device=dev).to(torch.bfloat16)
        Kc = torch.randn((B, a["Hkv"], L, a["D"]), generator=g, device=dev).to(torch.bfloat16)
        Vc = torch.randn_like(Kc)
        o = torch.empty((B, a["Hq"], a["D"]), dtype=torch.bfloat16, device=dev)
        ms = run(lambda: rb.standin_attention(q, Kc, Vc, a["D"] ** -0.5, o))
        nbytes = 2 * Kc.numel() * 2
        out[f"attention_L{L}"] = {"ms": round(ms, 5), "gbs": round(nbytes / (ms / 1e3) / 1e9, 1)}
        del q, Kc, Vc, o
    torch.cuda.empty_cache()
    return out


MFMA_F32_PEAK_TFLOPS = 157.3


def fold_flops(kind, H, G, C, R, cap=16):
    """MFMA flops of one full fold (cap entries) per sequence, as the kernels issue them.

    Mamba-2: S^T[N x P] += B^T [N x cap] . (decayed dt x)[cap x P] per head: 2 cap C R.
    GDN (WY form): W = K S0^T (2 cap R C), Gram K K^T (2 cap cap R), U = T . rhs
    (2 cap cap C) and S'^T += K^T U (2 R cap C) per head."""
    if kind == "mamba2":
        return H * 2 * cap * C * R
    return H * (2 * cap * R * C + 2 * cap * cap * R + 2 * cap * cap * C + 2 * R * cap * C)


def decode_report(L, r, conv_ms):
    """One layer's report: throughput over the K timed steps; achieved bandwidth from the
    whole-window pass (algorithmic bytes of a window / its back-to-back time); fold split and
    percentiles from the event-pair pass; bytes per token and the replay-vs-conventional
    reduction, algorithmic and (for the batch-256 fp32 layers) measured."""
    ckb = {"f16": 2, "fp8": 1}.get(L.ckpt, 4)
    rep_m, conv_m = traffic_model(L.kind, L.H, L.G, L.C, L.R, L.cap, read_copy=L.read_copy, ckpt_bytes=ckb)
    replay_b, conv_b = sum(rep_m.values()), sum(conv_m.values())
    ms = r["total_ms"] / r["steps"]
    wms = r["window_ms_per_step"]
    ach = replay_b * L.B / (wms / 1e3) / 1e9
    out = {"batch": L.B, "tokens_per_s": round(L.B / (ms / 1e3), 1), "ms_per_step": round(ms, 5),
           "window_ms_per_step": round(wms, 5), "window_tokens_per_s": round(L.B / (wms / 1e3), 1),
           "flush_step_ms": round(r["flush_ms"], 5), "nonflush_step_ms": round(r["nonflush_ms"], 5),
           "achieved_gbs": round(ach, 1), "frac_of_peak": round(ach / HBM_PEAK_GBS, 4),
           "bytes_per_token_algorithmic": int(replay_b),
           "bytes_per_token_algorithmic_parts": {k: int(v) for k, v in rep_m.items()},
           "rotate": r["rotate"], "untimed_steps_before_timed_region": r["untimed_before"]}
    ff = fold_flops(L.kind, L.H, L.G, L.C, L.R, L.cap) * L.B
    tf = ff / (r["flush_ms"] / 1e3) / 1e12
    out["flush_mfma"] = {"flops_per_flush_step": ff, "tflops": round(tf, 2),
                         "frac_of_fp32_mfma_peak": round(tf / MFMA_F32_PEAK_TFLOPS, 4)}
    if conv_ms is not None:
        out["conventional"] = {"tokens_per_s": round(L.B / (conv_ms / 1e3), 1), "ms_per_step": round(conv_ms, 5),
                               "achieved_gbs": round(conv_b * L.B / (conv_ms / 1e3) / 1e9, 1),
                               "bytes_per_token_algorithmic": int(conv_b)}
        out["speedup_vs_conventional"] = round(conv_ms / ms, 3)
        out["speedup_vs_conventional_window"] = round(conv_ms / wms, 3)
        out["state_traffic_reduction_algorithmic"] = reductions(rep_m, conv_m)
        if L.B == 256 and L.ckpt == "f32" and L.read_copy is None:
            out["state_traffic_reduction_measured"] = measured_reduction(L.kind, L.B, rep_m, conv_m)
    return out


def time_spec(L, rounds, k, stream, seed=3):
    """Speculative rounds: replay (append k drafts + commit the accepted prefix) and the
    conventional baseline (k draft steps writing a snapshot each + restore of snapshot a-1)."""
    import numpy as np
    rb, torch = L.rb, L.torch
    rng = np.random.default_rng(seed)
    acc_np = np.minimum(rng.geometric(0.35, size=(rounds, L.B)) - 1, k).astype(np.int32)
    acc = torch.from_numpy(acc_np).to(L.dev)
    lib, sp = rb.lib(), rb.ctypes.c_void_p(stream.cuda_stream)
    ins = [L.inputs(r * k, k) for r in range(rounds)]
    y = torch.empty((k, L.B, L.H, L.C), dtype=torch.bfloat16, device=L.dev)
    yp = rb.ctypes.c_void_p(y.data_ptr())
    # untimed warm-up rounds of both schemes on throwaway states, so the timed rounds start
    # warm; the timed replay rounds then start from a fresh load
    warm = min(16, rounds)
    st = rb.ReplayState(L.cfg, device=L.dev)
    st.load_checkpoint(L.S0)
    Sw = L.S0.clone()
    snw = torch.empty((k,) + tuple(Sw.shape), dtype=torch.float32, device=L.dev)
    for r in range(warm):
        s = lib.replay_spec_append(st.h, k, rb.ctypes.byref(ins[r]), yp, sp)
        s |= lib.replay_spec_commit(st.h, rb.ctypes.c_void_p(acc[r].data_ptr()), sp)
        s |= lib.replay_conv_spec_step(rb.ctypes.byref(L.cfg), rb.ctypes.c_void_p(Sw.data_ptr()),
                                       rb.ctypes.c_void_p(snw.data_ptr()), k, rb.ctypes.byref(ins[r]), yp, sp)
        s |= lib.replay_conv_spec_restore(rb.ctypes.byref(L.cfg), rb.ctypes.c_void_p(Sw.data_ptr()),
                                          rb.ctypes.c_void_p(snw.data_ptr()), k, rb.ctypes.c_void_p(acc[r].data_ptr()), sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "spec warm-up round")
    torch.cuda.synchronize()
    del st, Sw, snw
    st = rb.ReplayState(L.cfg, device=L.dev)
    st.load_checkpoint(L.S0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(rounds):
        s = lib.replay_spec_append(st.h, k, rb.ctypes.byref(ins[r]), yp, sp)
        s |= lib.replay_spec_commit(st.h, rb.ctypes.c_void_p(acc[r].data_ptr()), sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "replay spec round")
    e1.record(stream)
    torch.cuda.synchronize()
    replay_ms = e0.elapsed_time(e1) / rounds
    # the bytes these rounds move, from the same accepted counts; the bookkeeping the
    # library ends with must be the one the count assumed
    nbytes, lens, folds = spec_bytes(L.kind, L.H, L.G, L.C, L.R, L.cap, k, acc_np)
    ln, _, fc, _ = st.read_book()
    torch.cuda.synchronize()
    if not (np.array_equal(ln.cpu().numpy(), lens) and np.array_equal(fc.cpu().numpy(), folds)):
        raise RuntimeError("spec rounds: bookkeeping differs from the byte count's")
    del st
    S = L.S0.clone()
    snaps = torch.empty((k,) + tuple(S.shape), dtype=torch.float32, device=L.dev)
    cp, Sp, npp = rb.ctypes.byref(L.cfg), rb.ctypes.c_void_p(S.data_ptr()), rb.ctypes.c_void_p(snaps.data_ptr())
    torch.cuda.synchronize()
    e0.record(stream)
    for r in range(rounds):
        s = lib.replay_conv_spec_step(cp, Sp, npp, k, rb.ctypes.byref(ins[r]), yp, sp)
        s |= lib.replay_conv_spec_restore(cp, Sp, npp, k, rb.ctypes.c_void_p(acc[r].data_ptr()), sp)
        if s != rb.OK:
            raise rb.ReplayError(s, "conventional spec round")
    e1.record(stream)
    torch.cuda.synchronize()
    conv_ms = e0.elapsed_time(e1) / rounds
    del snaps, S
    accepted = float(acc_np.sum()) / rounds
    return {"batch": L.B, "drafts": k, "rounds": rounds, "mean_accepted": round(accepted / L.B, 4),
            "replay_ms_per_round": round(replay_ms, 5), "conventional_ms_per_round": round(conv_ms, 5),
            "replay_bytes_per_round_algorithmic": int(nbytes // rounds),
            "replay_achieved_gbs": round(nbytes / rounds / (replay_ms / 1e3) / 1e9, 1),
            "replay_frac_of_peak": round(nbytes / rounds / (replay_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "folded_prefixes_per_round": round(float(folds.sum()) / rounds, 2), "untimed_warmup_rounds": warm,
            "replay_accepted_tokens_per_s": round(accepted / (replay_ms / 1e3), 1),
            "conventional_accepted_tokens_per_s": round(accepted / (conv_ms / 1e3), 1),
            "speedup": round(conv_ms / replay_ms, 3)}


def ceilings(rb, torch, dev, stream):
    """In-run streaming ceilings with the replay kernels' access pattern (32 KiB tiles per
    workgroup, eight 128-bit loads in flight per lane): a 1 GiB copy (read + write) and a
    1 GiB read, each 10 launches back to back after 3 warm-up launches."""
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    nb = src.numel() * 4
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        rb.stream_copy(dst, src, nb)
    e0.record(stream)
    for _ in range(10):
        rb.stream_copy(dst, src, nb)
    e1.record(stream)
    torch.cuda.synchronize()
    copy = 10 * 2 * nb / (e0.elapsed_time(e1) / 1e3) / 1e9
    acc = torch.empty(rb.stream_read_partials(nb), dtype=torch.float32, device=dev)
    for _ in range(3):
        rb.stream_read(src, nb, acc)
    e0.record(stream)
    for _ in range(10):
        rb.stream_read(src, nb, acc)
    e1.record(stream)
    torch.cuda.synchronize()
    read = 10 * nb / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return round(copy, 1), round(read, 1)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--batch", type=int, default=256)
    ap.add_argument("--conv-steps", type=int, default=256, help="steps of the in-run conventional baselines")
    ap.add_argument("--spec-rounds", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline layer only (no GDN, spec, conventional)")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged-occupancy section (its masked launches share the step kernels and grids of "
                         "the other sections, so per-kernel profiles are taken without it)")
    ap.add_argument("--sweep", metavar="FILE", help="also sweep batch 1..512 for both layers, JSON lines to FILE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the decode path shards by "
              "sequence and head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_decode_replay_amd import binding as rb, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    K, W, B = args.steps, args.warmup, args.batch
    ntok = min(K + W + 4, 320)

    log(f"headline: Mamba-2 layer, batch {B}, {K} timed steps")
    m2 = Layer(rb, synth, torch, dev, "mamba2", B, ntok, seed=1)
    r = time_replay_decode(m2, K, W, stream)
    rep_m, _ = traffic_model("mamba2", m2.H, m2.G, m2.C, m2.R)
    replay_b = sum(rep_m.values())
    achieved = replay_b * B / (r["window_ms_per_step"] / 1e3) / 1e9
    conv_ms = None if args.no_extras else time_conv_decode(m2, min(args.conv_steps, K), stream)
    head = decode_report(m2, r, conv_ms)
    del m2
    torch.cuda.empty_cache()
    traffic = read_traffic(TRAFFIC[("mamba2", "replay")]) if B == 256 else None

    out = {
        "metric": "SSM-layer decode tokens/s at batch 256; achieved HBM GB/s vs MI355X peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, drawn on device; random checkpoint N(0,0.1))",
        "config": {"workload": "Mamba-2 SSM layer, replayed decode", "batch": B, "nheads": 128, "head_dim": 64,
                   "state_dim": 128, "ngroups": 8, "buffer": 16, "checkpoint": "fp32", "io": "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "mamba2_step_kernel", "algorithmic_bytes_per_launch": int(replay_b * B),
                     "launch_ms": round(r["window_ms_per_step"], 5),
                     "launch_ms_source": f"{r['window_steps']} steps (4 whole 16-step windows) back to back between "
                                         "two events on the launch stream",
                     "traffic_source": "profiles/mamba2_step_b256_traffic.txt (window bytes per launch; null when "
                                       "the kernel sources changed since it was taken)"},
        "timing": {"untimed_steps_before_timed_region": r["untimed_before"],
                   "note": "W warm-up steps, then untimed steps to a window boundary and two full windows"},
        "mamba2": head,
    }
    log("ceilings")
    out["copy_ceiling_gbs"], out["read_ceiling_gbs"] = ceilings(rb, torch, dev, stream)
    out["mamba2"]["frac_of_read_ceiling"] = round(head["achieved_gbs"] / out["read_ceiling_gbs"], 4)

    if not args.no_extras:
        log("GDN layer")
        gd = Layer(rb, synth, torch, dev, "gdn", B, ntok, seed=2)
        rg = time_replay_decode(gd, K, W, stream)
        out["gdn"] = decode_report(gd, rg, time_conv_decode(gd, min(args.conv_steps, K), stream))
        out["gdn"]["frac_of_read_ceiling"] = round(out["gdn"]["achieved_gbs"] / out["read_ceiling_gbs"], 4)
        del gd
        torch.cuda.empty_cache()
        log("speculative rounds")
        spec = {}
        for kind, seed in (("mamba2", 31), ("gdn", 32)):
            Ls = Layer(rb, synth, torch, dev, kind, 512, args.spec_rounds * 4, seed=seed)
            spec[kind] = time_spec(Ls, args.spec_rounds, 4, stream)
            del Ls
            torch.cuda.empty_cache()
        out["spec"] = spec
        # low-precision reads on the batch-128 GDN layer: fp32, FP8 and MXFP4 read copies,
        # rotated over enough states that no launch finds its copy in the Infinity Cache
        log("read copies")
        lp = {}
        for rc in (None, "fp8", "mxfp4"):
            Lr = Layer(rb, synth, torch, dev, "gdn", 128, 160, seed=4, read_copy=rc)
            rr = time_replay_decode(Lr, 256, 32, stream, rotate=auto_rotate(Lr))
            lp[rc or "fp32"] = decode_report(Lr, rr, None)
            del Lr
            torch.cuda.empty_cache()
        out["gdn_read_copy_b128"] = lp
        # fp16 recurrence checkpoint at batch 256 (the conventional baseline on an fp16 state)
        log("fp16 checkpoints")
        f16 = {}
        for kind, seed in (("mamba2", 6), ("gdn", 7)):
            Lh = Layer(rb, synth, torch, dev, kind, B, 160, seed=seed, ckpt="f16")
            rot = auto_rotate(Lh)
            rh = time_replay_decode(Lh, 256, 32, stream, rotate=rot)
            f16[kind] = decode_report(Lh, rh, time_conv_decode(Lh, 64, stream, rotate=rot))
            del Lh
            torch.cuda.empty_cache()
        out["fp16_checkpoint"] = f16
        # FP8 recurrence checkpoint at batch 256: alone (beside the conventional kernel on an
        # FP8 state) and with an MXFP4 read copy
        log("FP8 checkpoints")
        f8 = {}
        for kind, seed in (("mamba2", 9), ("gdn", 10)):
            for rc in (None, "mxfp4"):
                Lq = Layer(rb, synth, torch, dev, kind, B, 160, seed=seed, ckpt="fp8", read_copy=rc)
                rot = auto_rotate(Lq)
                rq = time_replay_decode(Lq, 256, 32, stream, rotate=rot)
                f8[kind + ("_mxfp4_copy" if rc else "")] = decode_report(
                    Lq, rq, None if rc else time_conv_decode(Lq, 64, stream, rotate=rot))
                del Lq
                torch.cuda.empty_cache()
        out["fp8_checkpoint"] = f8
        # flush schedule at batch 256: lockstep folds (every 16th step folds every sequence)
        # against staggered phases (about 1/16 of the sequences fold on each step)
        log("flush schedules")
        sched = {}
        for name, fl in (("lockstep", 0), ("staggered", rb.FLAG_STAGGER_FLUSH)):
            Lg = Layer(rb, synth, torch, dev, "mamba2", B, 160, seed=8, flags=fl)
            rg = time_replay_decode(Lg, 256, 32, stream)
            sched[name] = {"ms_per_step": round(rg["total_ms"] / rg["steps"], 5),
                           "window_ms_per_step": round(rg["window_ms_per_step"], 5),
                           "launch_ms_p50": round(rg["p50_launch_ms"], 5), "launch_ms_p99": round(rg["p99_launch_ms"], 5),
                           "launch_ms_max": round(rg["max_launch_ms"], 5)}
            del Lg
            torch.cuda.empty_cache()
        out["flush_schedule_mamba2_b256"] = sched
        # a serving batch whose slots come and go: masked steps, per-slot arrivals
        if not args.no_ragged:
            log("ragged occupancy")
            rag = {}
            for kind, seed in (("mamba2", 13), ("gdn", 14)):
                Lr = Layer(rb, synth, torch, dev, kind, B, 160, seed=seed)
                rag[kind] = time_ragged(Lr, 256, 32, stream)
                del Lr
                torch.cuda.empty_cache()
            out["ragged_b256"] = rag
        # a hybrid model's SSM layers decoded as one stack (one bookkeeping set), lockstep
        # and staggered flush phases, against the conventional kernel per layer
        log("hybrid stack")
        stack = {}
        for name, fl in (("lockstep", 0), ("staggered", rb.FLAG_STAGGER_FLUSH)):
            Ls = [Layer(rb, synth, torch, dev, kind, B, 128 + 16, seed=40 + i, flags=fl)
                  for i, kind in enumerate(("mamba2", "gdn", "mamba2", "gdn"))]
            stack[name] = time_stack(Ls, 128, 16, stream)
            del Ls
            torch.cuda.empty_cache()
        out["hybrid_stack_b256"] = stack
        # the SSM layers inside a whole synthetic hybrid decode step (stand-in projections,
        # attention and MLPs identical in both runs): the step-level, diluted gain
        log("hybrid model step with stand-in layers")
        out["standin_kernels_b256"] = time_standins(rb, torch, dev, stream)
        model = {}
        for context in (1024, 4096):
            for mlp in (False, True):
                model[f"context{context}_{'mlp' if mlp else 'nomlp'}"] = time_model_step(
                    rb, synth, torch, dev, stream, B, context, mlp)
                torch.cuda.empty_cache()
        out["hybrid_model_step_b256"] = model

    if args.sweep:
        with open(args.sweep, "w") as f:
            for kind in ("mamba2", "gdn"):
                for bsz in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512):
                    Lw = Layer(rb, synth, torch, dev, kind, bsz, 64 + 16 + 4, seed=5)
                    rot = auto_rotate(Lw)
                    rw = time_replay_decode(Lw, 64, 16, stream, rotate=rot)
                    rep = decode_report(Lw, rw, time_conv_decode(Lw, 64, stream, rotate=rot))
                    rep["kind"] = kind
                    g_rep, g_conv = time_graph(Lw, False), time_graph(Lw, True)
                    rep["graph"] = {"replay_ms_per_step": round(g_rep, 5), "conventional_ms_per_step": round(g_conv, 5),
                                    "speedup_vs_conventional": round(g_conv / g_rep, 3), "rotate": 1}
                    f.write(json.dumps(rep) + "\n")
                    f.flush()
                    print(f"[sweep] {kind} B={bsz} rotate={rot}: replay {rep['ms_per_step']:.4f} ms, conventional "
                          f"{rep['conventional']['ms_per_step']:.4f} ms, speedup {rep['speedup_vs_conventional']}; "
                          f"graph {g_rep:.4f} / {g_conv:.4f} ms", file=sys.stderr, flush=True)
                    del Lw
                    torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
