"""Plain fp64 CPU oracle for the replayed SSM decode path (Mamba-2, Gated DeltaNet).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the GPU library and never imports it.

Pages cited:
  [DE] "ReplaySSM beschleunigt das Decoding von Hybridmodellen durch Caching der
       Eingaben statt des Zustands" (German)
  [ES] its Spanish translation, "ReplaySSM acelera la decodificacion de modelos
       hibridos ..."
  [TR] "NVIDIA ve Dao AI Lab, hibrit model cozumlemesini hizlandirmak icin
       ReplaySSM'i sundu" (Turkish)

Two parts:

* Values.  The replayed path must give the outputs of ordinary token-by-token
  decoding up to rounding ([TR] "ReplaySSM nasil calisir?").  So the value side
  of the oracle is ordinary decoding in fp64 (oracle.c), applied to the
  committed token stream.  Values never depend on when flushes happen.

* Bookkeeping.  A per-sequence integer machine for the buffer pointer (len),
  the pending draft count (pend) and the flush count (fc), with a buffer of
  capacity `cap` (16 on the pages, [TR] "ReplaySSM nasil calisir?"):
    decode      if len+1 > cap: forced flush.  Append at len; len += 1.
                If len == cap afterwards: flush.  (The flush happens on the
                step that fills the buffer: [TR] same section; [DE] "Wie es
                funktioniert".)
    flush       if len > 0: flush.  Not allowed while drafts are pending.
    spec(k)     1 <= k <= cap, no drafts pending.  If len+k > cap: forced
                flush of the committed prefix first.  Drafts occupy
                [len, len+k); pend = k.  ([TR] "Durum trafigini azaltma ve
                rollback'in basitlestirilmesi": drafts are appended without
                verification.)
    commit(a)   a := clamp(a, 0, pend) (flagged when clamped); len += a;
                pend = 0.  The accepted prefix advances the pointer.
    rollback    commit(0): a pointer reset discards the drafts ([DE] "Wie es
                funktioniert", [ES] "Como funciona").
  A flush sets fc += 1 and len = 0 and records the checkpoint image (the
  committed fp64 state at that moment).

  Staggered flush phases (an option; the pages leave the flush schedule to the
  implementation, and values do not depend on it): a window holds lim entries;
  after a load lim = 1 + (b mod cap) for sequence b, after any flush lim = cap,
  and the decode rule "if len == cap afterwards" reads "if len >= lim".

  Ragged serving batches (the pages' gain comes from many concurrent
  sequences, [DE] "Warum es wichtig ist", and every sequence flushes its own
  buffer, [TR] "ReplaySSM nasil calisir?"; the operations below are the
  plainest reading of sequences joining and leaving a batch):
    decode / spec with an active mask
                only the marked sequences take the operation; the others keep
                their state, buffer and (len, fc, lim), and take no drafts
                (pend stays 0).
    load_slots(slots, S)
                the listed sequences take new checkpoints (rounded as a load
                rounds them), with an empty buffer, len = pend = fc = 0 and a
                full window lim = cap; the others keep everything.

The pages leave the following open; the readings taken here are listed with
the design notes: when the flush happens (on the filling step), whether the
output includes the current token (yes), the overflow rule for drafts (forced
flush before appending), and that a load resets len, pend and fc.

Low-precision read copy ([TR] "Kuantizasyon hatasinin sinirlandirilmasi": a
high-precision checkpoint drives the recurrence, a low-precision copy serves
reads).  With a read copy, a step that performs no flush produces its output
from the dequantized copy of the checkpoint followed by the committed tokens
since the last flush; a step that flushes produces it from the full-precision
state.  The copy is the quantization of the checkpoint image rounded to fp32.

Quantized checkpoint (the comparison variant the same section contrasts with:
a low-precision state inside the recurrence).  The checkpoint is rounded to the
copy's grid at load and at every flush, and the recurrence continues from the
rounded state; the output of a step whose own token was folded is read from
the rounded state.

FP16 recurrence checkpoint (the same section pairs low-precision reads with an
FP16 or FP8 recurrence).  The checkpoint is stored as IEEE binary16: rounded to
nearest even at load and at every flush (numpy's float64 -> float16 cast), and
the recurrence and outputs continue from the stored values exactly as in the
quantized-checkpoint case.  The pages give no tolerance for it.

FP8 recurrence checkpoint (same section).  As the FP16 case, with the state
rounded at load and at every flush to the nearest OCP E4M3 value (ties to even,
saturating at +-448, e4m3_encode below) straight from the fp64 fold.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ubp = ctypes.POINTER(ctypes.c_ubyte)


def configure(L):
    """Declare the C signatures on a loaded oracle library handle."""
    i, d = ctypes.c_int, ctypes.c_double
    L.oracle_mamba2_token.argtypes = [i, i, i, i, i, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _ubp]
    L.oracle_mamba2_token.restype = None
    L.oracle_gdn_token.argtypes = [i, i, i, i, i, _dp, _dp, _dp, _dp, _dp, _dp, d, _dp, _ubp]
    L.oracle_gdn_token.restype = None
    L.oracle_e4m3_decode.argtypes = [i]
    L.oracle_e4m3_decode.restype = d
    L.oracle_e4m3_encode.argtypes = [d]
    L.oracle_e4m3_encode.restype = i
    L.oracle_e2m1_decode.argtypes = [i]
    L.oracle_e2m1_decode.restype = d
    L.oracle_e2m1_encode.argtypes = [d]
    L.oracle_e2m1_encode.restype = i
    L.oracle_e8m0_decode.argtypes = [i]
    L.oracle_e8m0_decode.restype = d
    L.oracle_mxfp4_quantize_block.argtypes = [_dp, i, _ubp]
    L.oracle_mxfp4_quantize_block.restype = i
    L.oracle_e4m3_encode_array.argtypes = [_dp, ctypes.c_long, _ubp]
    L.oracle_e4m3_encode_array.restype = None
    L.oracle_e4m3_decode_array.argtypes = [_ubp, ctypes.c_long, _dp]
    L.oracle_e4m3_decode_array.restype = None
    L.oracle_mxfp4_quantize_array.argtypes = [_dp, ctypes.c_long, _ubp, _ubp]
    L.oracle_mxfp4_quantize_array.restype = None
    L.oracle_mxfp4_quantize_array_ceil.argtypes = [_dp, ctypes.c_long, _ubp, _ubp]
    L.oracle_mxfp4_quantize_array_ceil.restype = None
    L.oracle_mxfp4_quantize_block_ceil.argtypes = [_dp, i, _ubp]
    L.oracle_mxfp4_quantize_block_ceil.restype = i
    L.oracle_mxfp4_dequantize_array.argtypes = [_ubp, _ubp, ctypes.c_long, _dp]
    L.oracle_mxfp4_dequantize_array.restype = None
    L.oracle_threads.argtypes = []
    L.oracle_threads.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_set_threads.restype = None
    return L


def lib():
    """Load (building with gcc if absent) the fp64 oracle library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            from oracle import build as _b  # local build on demand
            _b.build()
        _lib = configure(ctypes.CDLL(_LIBPATH))
    return _lib


def use_library(handle):
    """Swap the loaded library (used by the tests that plant mistakes in a copy).

    Returns the previous handle so the caller can restore it."""
    global _lib
    prev = _lib
    _lib = handle
    return prev


def threads():
    """OpenMP threads the oracle's per-token loops run on."""
    return int(lib().oracle_threads())


def set_threads(n):
    """Run the oracle's per-token loops on n threads from now on."""
    lib().oracle_set_threads(int(n))


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


# --------------------------------------------------------------------------
# Per-token recurrences (thin wrappers over oracle.c)
# --------------------------------------------------------------------------

def mamba2_token(S, x, Bm, Cm, dt, A, D, active=None):
    """One ordinary Mamba-2 decode token, in place on S [B,H,P,N] (fp64).

    Returns y [B,H,P] (zeros where the sequence is inactive)."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    Bsz, H, P, N = S.shape
    G = Bm.shape[1]
    x, xp = _f64(x)
    Bm, bp = _f64(Bm)
    Cm, cp = _f64(Cm)
    dt, dtp = _f64(dt)
    A, ap = _f64(A)
    D, dp = _f64(D)
    y = np.zeros((Bsz, H, P), np.float64)
    act = None
    if active is not None:
        active = np.ascontiguousarray(active, dtype=np.uint8)
        act = active.ctypes.data_as(_ubp)
    lib().oracle_mamba2_token(Bsz, H, G, P, N, S.ctypes.data_as(_dp), xp, bp, cp, dtp, ap, dp,
                              y.ctypes.data_as(_dp), act)
    return y


def gdn_token(S, q, k, v, alpha, beta, scale=1.0, active=None):
    """One ordinary Gated DeltaNet decode token, in place on S [B,H,DV,DK] (fp64).

    Returns o [B,H,DV]."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    Bsz, H, DV, DK = S.shape
    G = k.shape[1]
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    alpha, alp = _f64(alpha)
    beta, bep = _f64(beta)
    o = np.zeros((Bsz, H, DV), np.float64)
    act = None
    if active is not None:
        active = np.ascontiguousarray(active, dtype=np.uint8)
        act = active.ctypes.data_as(_ubp)
    lib().oracle_gdn_token(Bsz, H, G, DK, DV, S.ctypes.data_as(_dp), qp, kp, vp, alp, bep,
                           float(scale), o.ctypes.data_as(_dp), act)
    return o


# --------------------------------------------------------------------------
# Quantizers (OCP MX v1.0 element formats)
# --------------------------------------------------------------------------

def e4m3_encode(v):
    v, vp = _f64(np.ravel(v))
    out = np.empty(v.size, np.uint8)
    lib().oracle_e4m3_encode_array(vp, v.size, out.ctypes.data_as(_ubp))
    return out


def e4m3_decode(codes):
    codes = np.ascontiguousarray(np.ravel(codes), dtype=np.uint8)
    out = np.empty(codes.size, np.float64)
    lib().oracle_e4m3_decode_array(codes.ctypes.data_as(_ubp), codes.size, out.ctypes.data_as(_dp))
    return out


def mxfp4_quantize(v, rule="floor"):
    """v [..., 32k]: blocks of 32 along the last axis.  rule "floor": the OCP shared
    exponent floor(log2(amax)) - 2 (a block maximum may clip to 6); "ceil": the smallest
    exponent with amax <= 6 * 2^X (nothing clips).

    Returns (codes uint8 [..., 32k] one 4-bit code per byte, scales uint8 [..., k])."""
    v = np.asarray(v, np.float64)
    assert v.shape[-1] % 32 == 0
    lead = v.shape[:-1]
    nb = v.size // 32
    flat, fp = _f64(v.reshape(nb, 32))
    codes = np.empty((nb, 32), np.uint8)
    scales = np.empty(nb, np.uint8)
    fn = {"floor": lib().oracle_mxfp4_quantize_array, "ceil": lib().oracle_mxfp4_quantize_array_ceil}[rule]
    fn(fp, nb, codes.ctypes.data_as(_ubp), scales.ctypes.data_as(_ubp))
    return codes.reshape(*lead, v.shape[-1]), scales.reshape(*lead, v.shape[-1] // 32)


def mxfp4_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    nb = scales.size
    out = np.empty(nb * 32, np.float64)
    lib().oracle_mxfp4_dequantize_array(codes.ctypes.data_as(_ubp), scales.ctypes.data_as(_ubp),
                                        nb, out.ctypes.data_as(_dp))
    return out.reshape(codes.shape)


def read_copy_values(S_fp64, fmt):
    """Dequantized read copy of a checkpoint image: round to fp32, quantize, dequantize.

    Blocks (MXFP4) run along the last axis (N for Mamba-2, d_k for GDN); "mxfp4_ceil" is
    MXFP4 with the non-clipping scale rule."""
    s32 = np.asarray(S_fp64, np.float64).astype(np.float32).astype(np.float64)
    if fmt is None:
        return s32
    if fmt == "fp8":
        return e4m3_decode(e4m3_encode(s32)).reshape(s32.shape)
    if fmt in ("mxfp4", "mxfp4_ceil"):
        c, s = mxfp4_quantize(s32, "ceil" if fmt == "mxfp4_ceil" else "floor")
        return mxfp4_dequantize(c, s)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# Op runner: values + bookkeeping
# --------------------------------------------------------------------------

class PhaseError(RuntimeError):
    """An operation that the buffer protocol does not allow in the current phase."""


class _Session:
    """Shared bookkeeping for both layer kinds.  Subclasses define _token()."""

    kind = None

    def __init__(self, batch, cap, S0, read_copy=None, quantized_ckpt=False, ckpt_dtype="f32", stagger=False,
                 seq_ids=None):
        if not 1 <= cap <= 16:
            raise ValueError("buffer capacity must be in [1, 16]")
        if read_copy not in (None, "fp8", "mxfp4", "mxfp4_ceil"):
            raise ValueError("read copy must be None, 'fp8', 'mxfp4' or 'mxfp4_ceil'")
        if quantized_ckpt and read_copy is None:
            raise ValueError("a quantized checkpoint needs a format")
        if ckpt_dtype not in ("f32", "f16", "fp8"):
            raise ValueError("checkpoint dtype must be 'f32', 'f16' or 'fp8'")
        if ckpt_dtype == "fp8" and read_copy == "fp8":
            raise ValueError("an FP8 copy of an FP8 checkpoint repeats it")
        if quantized_ckpt and ckpt_dtype != "f32":
            raise ValueError("the quantized-checkpoint variant keeps an fp32 checkpoint")
        self.B = batch
        self.cap = cap
        self.read_copy = read_copy
        self.quantized_ckpt = quantized_ckpt
        self.ckpt_dtype = ckpt_dtype
        self.rounds = quantized_ckpt or ckpt_dtype != "f32"    # folds land on a coarser grid
        self.stagger = stagger
        # batch index of each sequence held here (a session may hold a sample of a batch);
        # the staggered first window depends on it
        self.seq_ids = np.arange(batch) if seq_ids is None else np.asarray(seq_ids, np.int64)
        if self.seq_ids.shape != (batch,):
            raise ValueError("one batch index per sequence")
        self.S = self._round(np.array(S0, np.float64, copy=True))   # committed state
        self.ckpt = self.S.copy()                              # image at last flush
        self.len = np.zeros(batch, np.int32)
        self.pend = np.zeros(batch, np.int32)
        self.fc = np.zeros(batch, np.int32)
        self.lim = self._first_limits()
        self.err = 0
        self.hist = [[] for _ in range(batch)]                 # committed tokens since flush
        self._drafts = None                                    # list of per-draft inputs
        self.flush_events = []                                 # (op index, b) pairs
        self.nops = 0

    # -- helpers -----------------------------------------------------------
    def _first_limits(self):
        if self.stagger:
            return (1 + self.seq_ids % self.cap).astype(np.int32)
        return np.full(self.B, self.cap, np.int32)

    def trace(self):
        return self.len.copy(), self.pend.copy(), self.fc.copy()

    def _round(self, S):
        """The state as the checkpoint keeps it: rounded to binary16 or E4M3 for an
        fp16 or FP8 checkpoint, to the copy's grid in the quantized-checkpoint variant,
        unchanged otherwise."""
        if self.ckpt_dtype == "f16":
            return np.asarray(S, np.float64).astype(np.float16).astype(np.float64)
        if self.ckpt_dtype == "fp8":
            return e4m3_decode(e4m3_encode(S)).reshape(np.shape(S))
        if not self.quantized_ckpt:
            return S
        return read_copy_values(S, self.read_copy).reshape(S.shape)

    def _flush_rows(self, rows, rounded=True):
        """Fold the buffered entries of the sequences `rows` into their checkpoints.
        rounded=False leaves the state unrounded: the caller folds more entries in the
        same pass and rounds once at its end."""
        for b in np.flatnonzero(rows):
            if rounded:
                self.S[b] = self._round(self.S[b:b + 1])[0]
            self.ckpt[b] = self.S[b]
            self.fc[b] += 1
            self.len[b] = 0
            self.lim[b] = self.cap
            self.hist[b] = []
            self.flush_events.append((self.nops, int(b)))

    def _slice(self, inp, b):
        return {k: (v[b:b + 1] if v.ndim >= 1 and v.shape[0] == self.B else v) for k, v in inp.items()}

    def _read_copy_output(self, b, inp):
        """Output for sequence b from the dequantized checkpoint + history + inp."""
        S = read_copy_values(self.ckpt[b:b + 1], self.read_copy).copy()
        for past in self.hist[b]:
            self._token(S, past)
        return self._token(S, self._slice(inp, b))[0]

    # -- operations --------------------------------------------------------
    def load(self, S0):
        if self._drafts is not None:
            raise PhaseError("load while drafts are pending")
        self.S = self._round(np.array(S0, np.float64, copy=True))
        self.ckpt = self.S.copy()
        self.len[:] = 0
        self.pend[:] = 0
        self.fc[:] = 0
        self.lim = self._first_limits()
        self.err = 0
        self.hist = [[] for _ in range(self.B)]
        self.nops += 1

    def _mask(self, active):
        if active is None:
            return np.ones(self.B, bool)
        active = np.asarray(active, bool)
        if active.shape != (self.B,):
            raise ValueError("the active mask has one entry per sequence")
        return active

    def decode(self, inp, active=None):
        """One decode token for the sequences `active` marks (all by default).  Outputs of
        the others are zero here (the GPU leaves their rows untouched)."""
        if self._drafts is not None:
            raise PhaseError("decode while drafts are pending")
        act = self._mask(active)
        forced = act & (self.len + 1 > self.cap)
        # A full buffer is folded before the token is appended.  With a one-entry
        # buffer the token then fills the buffer again and is folded in the same step:
        # the two folds are one pass over both entries, so a low-precision checkpoint
        # is rounded once, after both (reading of the library's one-entry buffer; the
        # pages fix the buffer at 16 entries).
        self._flush_rows(forced, rounded=self.cap > 1)
        y = self._token(self.S, inp, act.astype(np.uint8))
        self.len += act.astype(np.int32)
        full = act & (self.len >= self.lim)
        if self.read_copy:
            no_flush = act & ~(forced | full)
            for b in np.flatnonzero(no_flush):
                y[b] = self._read_copy_output(b, inp)
        for b in np.flatnonzero(act & ~full):
            self.hist[b].append(self._slice(inp, b))
        self._flush_rows(full)
        if self.rounds:
            for b in np.flatnonzero(full):
                y[b] = self._readout(self.S[b], self._slice(inp, b))
        self.nops += 1
        return y

    def flush(self):
        if self._drafts is not None:
            raise PhaseError("flush while drafts are pending")
        self._flush_rows(self.len > 0)
        self.nops += 1

    def spec_append(self, drafts, active=None):
        """drafts: list of k per-token input dicts.  Returns outputs [k] of arrays (zero for
        sequences `active` leaves out; they take no drafts)."""
        k = len(drafts)
        if self._drafts is not None:
            raise PhaseError("spec_append while drafts are pending")
        if not 1 <= k <= self.cap:
            raise ValueError("draft count out of range")
        act = self._mask(active)
        pre = act & (self.len + k > self.cap)
        self._flush_rows(pre)
        S = self.S.copy()
        outs = []
        for j, inp in enumerate(drafts):
            y = self._token(S, inp, act.astype(np.uint8))
            if self.read_copy:
                # a sequence whose committed prefix was not folded reads the copy of its
                # checkpoint, replays its committed history, then drafts 0..j
                for b in np.flatnonzero(act & ~pre):
                    Sq = read_copy_values(self.ckpt[b:b + 1], self.read_copy).copy()
                    for past in self.hist[b]:
                        self._token(Sq, past)
                    for jj in range(j + 1):
                        yq = self._token(Sq, self._slice(drafts[jj], b))
                    y[b] = yq[0]
            outs.append(y)
        self._drafts = list(drafts)
        self.pend[:] = np.where(act, k, 0)
        self.nops += 1
        return outs

    def load_slots(self, slots, S_new):
        """Sequences `slots` take the checkpoints S_new [n, ...] (rounded as a load rounds them),
        with an empty buffer, len = pend = fc = 0 and a full window; the others keep theirs."""
        if self._drafts is not None:
            raise PhaseError("load while drafts are pending")
        slots = [int(b) for b in slots]
        if len(set(slots)) != len(slots) or any(not 0 <= b < self.B for b in slots):
            raise ValueError("slots must be distinct sequence indices")
        S_new = np.asarray(S_new, np.float64)
        for i, b in enumerate(slots):
            self.S[b] = self._round(S_new[i:i + 1].copy())[0]
            self.ckpt[b] = self.S[b]
            self.len[b] = 0
            self.pend[b] = 0
            self.fc[b] = 0
            self.lim[b] = self.cap
            self.hist[b] = []
        self.nops += 1

    def commit(self, accepted):
        if self._drafts is None:
            raise PhaseError("commit or rollback without pending drafts")
        a = np.asarray(accepted, np.int64)
        clamped = np.clip(a, 0, self.pend)
        if (clamped != a).any():
            self.err |= 1
        drafts = self._drafts or []
        for j, inp in enumerate(drafts):
            act = (clamped > j).astype(np.uint8)
            if act.any():
                self._token(self.S, inp, act)
                for b in np.flatnonzero(act):
                    self.hist[b].append(self._slice(inp, b))
        self.len += clamped.astype(np.int32)
        self.pend[:] = 0
        self._drafts = None
        self.nops += 1

    def rollback(self):
        self.commit(np.zeros(self.B, np.int64))


class Mamba2Session(_Session):
    """Mamba-2 layer: state [B,H,P,N]; per-token inputs x [B,H,P], Bm/Cm [B,G,N], dt [B,H]."""

    kind = "mamba2"

    def __init__(self, A, D, S0, cap=16, read_copy=None, quantized_ckpt=False, ckpt_dtype="f32", stagger=False,
                 seq_ids=None):
        self.A = np.asarray(A, np.float64)
        self.D = np.asarray(D, np.float64)
        super().__init__(np.asarray(S0).shape[0], cap, S0, read_copy, quantized_ckpt, ckpt_dtype, stagger, seq_ids)

    def _token(self, S, inp, active=None):
        return mamba2_token(S, inp["x"], inp["Bm"], inp["Cm"], inp["dt"], self.A, self.D, active)

    def _readout(self, S_b, inp_b):
        """y = S C + D x for one sequence, without a state update."""
        H = S_b.shape[0]
        g = np.arange(H) // (H // inp_b["Cm"].shape[1])
        C = np.asarray(inp_b["Cm"][0], np.float64)[g]                 # [H, N]
        x = np.asarray(inp_b["x"][0], np.float64)                     # [H, P]
        return np.einsum("hpn,hn->hp", S_b, C) + self.D[:, None] * x


class GDNSession(_Session):
    """Gated DeltaNet layer: state [B,H,DV,DK]; inputs q/k [B,G,DK], v [B,H,DV], alpha/beta [B,H]."""

    kind = "gdn"

    def __init__(self, S0, cap=16, scale=1.0, read_copy=None, quantized_ckpt=False, ckpt_dtype="f32", stagger=False,
                 seq_ids=None):
        self.scale = float(scale)
        super().__init__(np.asarray(S0).shape[0], cap, S0, read_copy, quantized_ckpt, ckpt_dtype, stagger, seq_ids)

    def _token(self, S, inp, active=None):
        return gdn_token(S, inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], self.scale, active)

    def _readout(self, S_b, inp_b):
        """o = scale S q for one sequence, without a state update."""
        H = S_b.shape[0]
        g = np.arange(H) // (H // inp_b["q"].shape[1])
        q = np.asarray(inp_b["q"][0], np.float64)[g]                  # [H, DK]
        return self.scale * np.einsum("hij,hj->hi", S_b, q)


class StackSession:
    """The SSM layers of one model, each its own session, stepped as one stack.

    Every layer of a hybrid model decodes the same token positions of the same
    sequences ([TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM nasil calisir?"),
    so the layers' bookkeeping moves in lockstep and one set describes them all.
    The protocol: a model step runs each layer once, in layer order, all with the
    same operation and draft count; a commit or rollback applies to every layer;
    loads and flushes act on all layers between steps.  Each layer keeps its own
    session here, so the lockstep claim is checked, not assumed: trace() asserts
    that every layer's bookkeeping is the same."""

    def __init__(self, sessions):
        self.layers = list(sessions)
        if not self.layers:
            raise ValueError("a stack needs at least one layer")
        if len({(s.B, s.cap, s.stagger) for s in self.layers}) != 1:
            raise ValueError("layers of a stack share batch, capacity and the stagger setting")
        self.next = 0
        self.step_op = None          # (operation, draft count) of the step in progress

    def _enter(self, layer, op):
        if layer != self.next:
            raise PhaseError(f"layer {layer} stepped out of order (layer {self.next} is next)")
        if self.next > 0 and op != self.step_op:
            raise PhaseError("every layer of a step runs the same operation and draft count")
        self.step_op = op

    def _leave(self):
        self.next += 1
        if self.next == len(self.layers):
            self.next = 0
            self.step_op = None

    def _idle(self, what):
        if self.next:
            raise PhaseError(f"{what} in the middle of a step")

    @staticmethod
    def _mask_key(active):
        return None if active is None else np.asarray(active, bool).tobytes()

    def decode_layer(self, layer, inp, active=None):
        self._enter(layer, ("decode", 1, self._mask_key(active)))
        y = self.layers[layer].decode(inp, active)
        self._leave()
        return y

    def spec_layer(self, layer, drafts, active=None):
        self._enter(layer, ("spec", len(drafts), self._mask_key(active)))
        ys = self.layers[layer].spec_append(drafts, active)
        self._leave()
        return ys

    def load_slots(self, slots, checkpoints):
        self._idle("load")
        for s, S in zip(self.layers, checkpoints, strict=True):
            s.load_slots(slots, S)

    def flush(self):
        self._idle("flush")
        for s in self.layers:
            s.flush()

    def commit(self, accepted):
        self._idle("commit")
        for s in self.layers:
            s.commit(accepted)

    def rollback(self):
        self._idle("rollback")
        for s in self.layers:
            s.rollback()

    def load(self, checkpoints):
        self._idle("load")
        for s, S0 in zip(self.layers, checkpoints, strict=True):
            s.load(S0)

    @property
    def err(self):
        errs = {s.err for s in self.layers}
        assert len(errs) == 1, "layers disagree on the error word"
        return errs.pop()

    def trace(self):
        self._idle("trace")
        traces = [s.trace() for s in self.layers]
        for t in traces[1:]:
            for a, b in zip(t, traces[0]):
                assert np.array_equal(a, b), "layers of a stack left lockstep"
        return traces[0]


def normwise_error(got, ref, axis=-1):
    """max over vectors of ||got - ref||_inf / max(||ref||_inf, 1e-30), vectors along `axis`."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=axis)
    den = np.maximum(np.max(np.abs(ref), axis=axis), 1e-30)
    return float(np.max(num / den)) if num.size else 0.0
