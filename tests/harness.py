"""Drive the HIP library and the fp64 oracle side by side on identical seeded inputs.

Test-side helper.  Inputs come from the seeded generators (synth); the oracle
never sees a value produced by the HIP path.  Each operation is applied to both
sides and the outputs, the checkpoint (read back in logical layout) and the
bookkeeping are compared:
  outputs      normwise relative error per output vector <= tol
  checkpoint   normwise relative error per (b, h) matrix <= tol
  bookkeeping  len, pend, fc and the error word bit-exact

Tolerances.  Outputs: the io dtype's (1e-4 fp32, 2e-2 bf16: the bf16 output
rounding counts against it).  fp32 checkpoints: 1e-4 whatever the io dtype (the
oracle consumes the same bf16-rounded inputs, so only fp32-vs-fp64 arithmetic
separates the two checkpoints).

With an fp16 checkpoint both sides round every fold to binary16 on their own
(the GPU from its fp32 fold, the oracle from fp64).  The two fold results differ
by fp32 rounding only, so they round to the same binary16 value except within
that distance of a rounding boundary, where they land one ulp apart (at most
2^-10 relative).  A test runs at most four folds, and a difference left by one
fold is carried (scaled by decays <= 1) into the next, so 4 x 2^-10 ~ 3.9e-3
bounds outputs and checkpoints: TOL_F16.

With an FP8 (E4M3) checkpoint one grid step is up to 2^-3 relative, too coarse
for a norm bound to say much, so the checkpoint is held to an element-wise
absolute bound propagated through the arithmetic (Fp8Bound): it starts at zero
(both sides round the same fp32 values at load); at a fold an element's bound
becomes (17/16)(prop(previous bound) + e) + 1.5 step(ref) + 2^-10, where step(ref)
is the larger E4M3 gap next to the oracle's value (the two sides round results
that differ by the carried difference plus the fp32 fold error e), and prop is
the fold's action on an old difference: a factor e^{sum dt A} <= 1 per element for
Mamba-2; for GDN the old difference times a product of gated Householder-like
factors of 2-norm <= 1, so an element is bounded by its row's 2-norm.  A
difference may also appear only rarely: at most FP8_FLIP_FRAC of the codes
(the fp32 fold is within ~1e-6 relative of the fp64 one and E4M3 steps are at
least 2^-4 relative, so about 3e-5 of the elements per fold straddle a midpoint).
Outputs are then held element-wise to tol * |y|_inf plus the read-out of the
checkpoint difference measured at that step (itself inside the derived bound;
the same form holds the outputs that read a read copy of an fp32 or fp16
checkpoint, with the difference of the two sides' copies of their own
checkpoints as dS, nonzero only where a value straddles a quantization boundary):
Mamba-2 sum_n |dS[p, n]| |C_n| (decays <= 1); GDN scale |dS[i, :]|_2 |q|_2 (the
adjoint chain's r_0 has 2-norm <= |q|_2).  With an MXFP4 copy of the FP8
checkpoint the copy difference |Q(S_gpu) - Q(S_ref)| (both quantized by the
oracle) is read out as well.  Pair(..., tol=0.0) asks for bit-exact outputs and
checkpoints (inputs chosen so that every result is exact in fp32).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import replay_oracle as ro
from hybrid_decode_replay_amd import binding as rb

TOL = {rb.F32: 1e-4, rb.BF16: 2e-2}
TOL_CKPT_F32 = 1e-4
TOL_F16 = 4 * 2.0 ** -10
FP8_FLIP_FRAC = 1e-3


def _e4m3_grid():
    grid = ro.e4m3_decode(np.arange(256, dtype=np.uint8))
    return np.unique(grid[np.isfinite(grid)])


def e4m3_grid_index(v):
    """Position of E4M3 values on the sorted grid of finite E4M3 values (+0 and -0 merged)."""
    grid = _e4m3_grid()
    v = np.asarray(v, np.float64)
    idx = np.searchsorted(grid, v)
    assert np.array_equal(grid[np.minimum(idx, grid.size - 1)], v), "value off the E4M3 grid"
    return idx


def e4m3_step(v):
    """The larger of the two gaps of the E4M3 grid next to each (on-grid) value."""
    grid = _e4m3_grid()
    idx = e4m3_grid_index(v)
    up = grid[np.minimum(idx + 1, grid.size - 1)] - grid[idx]
    dn = grid[idx] - grid[np.maximum(idx - 1, 0)]
    return np.maximum(up, dn)


class Fp8Bound:
    """Element-wise bound on |S_gpu - S_oracle| for an FP8 checkpoint [B, H, rows, cols],
    propagated through folds (or per-token updates) as the module docstring derives."""

    def __init__(self, kind, shape, exact=False):
        self.kind = kind
        self.bound = np.zeros(shape, np.float64)
        self.exact = exact

    def _prop(self, bnd):
        if self.kind == "gdn":                               # row 2-norm of the old bound
            return np.broadcast_to(np.sqrt(np.sum(bnd * bnd, axis=-1, keepdims=True)), bnd.shape).copy()
        return bnd                                           # Mamba-2: decay <= 1 per element

    def advance(self, rows, ref):
        """Sequences `rows` (bool [B]) were folded (rounded) once more; ref is the oracle's
        checkpoint after it."""
        if self.exact:
            return
        for b in np.flatnonzero(rows):
            r = np.asarray(ref[b], np.float64)
            eps = 2e-5 * np.max(np.abs(r), axis=(-2, -1), keepdims=True) + 1e-7
            self.bound[b] = (17 / 16) * (self._prop(self.bound[b]) + eps) + 1.5 * e4m3_step(r) + 2.0 ** -10

    def check(self, got, ref, what):
        """Returns the measured element-wise difference after checking it against the bound."""
        d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        over = d > self.bound
        assert not over.any(), (f"{what}: FP8 checkpoint difference {float(d[over].max()):.3e} beyond its derived "
                                f"bound ({int(over.sum())} elements)")
        frac = float(np.mean(d > 0))
        limit = 0.0 if self.exact else FP8_FLIP_FRAC
        assert frac <= limit, f"{what}: {frac:.2e} of the checkpoint codes differ (> {limit:.0e})"
        return d, frac


def readout_bound(kind, dS, tokens, scale=1.0):
    """Element-wise output deviation a checkpoint difference dS [B, H, rows, cols] can cause for
    each token (dicts of [B, ...] arrays): Mamba-2 sum_n dS[p, n] |C_n|; GDN
    scale |dS[i, :]|_2 |q|_2.  Returns [T, B, H, rows]."""
    B, H = dS.shape[:2]
    out = []
    for tok in tokens:
        if kind == "mamba2":
            Cm = np.abs(np.asarray(tok["Cm"], np.float64))
            g = np.arange(H) // (H // Cm.shape[1])
            out.append(np.einsum("bhpn,bhn->bhp", dS, Cm[:, g]))
        else:
            q = np.asarray(tok["q"], np.float64)
            g = np.arange(H) // (H // q.shape[1])
            qn = np.linalg.norm(q, axis=-1)[:, g]
            out.append(scale * np.sqrt(np.einsum("bhin,bhin->bhi", dS, dS)) * qn[:, :, None])
    return np.stack(out)


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


class Pair:
    """A GPU ReplayState and an oracle session fed the same operations."""

    def __init__(self, kind, B, H, G, C, R, cap=16, io=rb.F32, seed=0, S0=None, flags=0, scale=1.0,
                 read_copy=rb.NONE, ckpt=rb.F32, tol=None):
        self.kind = kind
        self.cfg = rb.make_config(kind, B, H, G, C, R, cap, io, read_copy=read_copy, ckpt_dtype=ckpt, flags=flags,
                                  scale=scale)
        self.io = io
        self.iot = torch.bfloat16 if io == rb.BF16 else torch.float32
        self.tol = max(TOL[io], TOL_F16) if ckpt == rb.F16 else TOL[io]
        self.ckpt_tol = TOL_F16 if ckpt == rb.F16 else TOL_CKPT_F32
        if tol is not None:
            self.tol = tol
            self.ckpt_tol = tol
        self.fp8 = ckpt == rb.FP8_E4M3
        self.scale = scale
        self.kname = "mamba2" if kind == rb.MAMBA2 else "gdn"
        self.B, self.H, self.G, self.C, self.R = B, H, G, C, R
        if S0 is None:
            S0 = np.zeros((B, H, C, R), np.float32)
        S0 = np.ascontiguousarray(S0, np.float32)
        # both sides start from the same fp32 values; each rounds them to the checkpoint
        # dtype on its own (the library on the device, the oracle by its encoders)
        self.st = rb.ReplayState(self.cfg)
        self.st.load_checkpoint(torch.from_numpy(S0).cuda())
        rc = {rb.NONE: None, rb.FP8_E4M3: "fp8", rb.MXFP4: "mxfp4"}[read_copy]
        if rc == "mxfp4" and flags & rb.FLAG_MX_SCALE_CEIL:
            rc = "mxfp4_ceil"                       # the non-clipping shared exponent
        self.rc = rc
        cd = {rb.F16: "f16", rb.FP8_E4M3: "fp8"}.get(ckpt, "f32")
        self.fp8b = Fp8Bound(self.kname, (B, H, C, R), exact=(self.tol == 0.0)) if self.fp8 else None
        self.dS = None                              # FP8: measured checkpoint (and copy) difference
        self.max_flip_frac = 0.0
        stagger = bool(flags & rb.FLAG_STAGGER_FLUSH)
        if kind == rb.MAMBA2:
            from hybrid_decode_replay_amd import synth
            A, D = synth.mamba2_params(seed, H)
            self.params = {"A": dev(A, torch.float32), "D": dev(D, torch.float32)}
            self.orc = ro.Mamba2Session(A, D, S0, cap=cap, read_copy=rc, ckpt_dtype=cd, stagger=stagger)
        else:
            self.params = {}
            self.orc = ro.GDNSession(S0, cap=cap, scale=scale, read_copy=rc, ckpt_dtype=cd, stagger=stagger)
        self.fc_seen = self.orc.fc.copy()
        self.max_err = {"y": 0.0, "ckpt": 0.0}
        if not flags & rb.FLAG_QUANTIZED_CKPT:
            self.check_loaded("load")

    def check_loaded(self, what):
        """Right after a load both sides hold the same rounding of the same fp32 values: bit-exact."""
        torch.cuda.synchronize()
        got = self.st.read_checkpoint()
        if self.fp8:
            got = ro.e4m3_decode(got.view(torch.uint8).cpu().numpy()).reshape(got.shape)
        else:
            got = got.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, self.orc.ckpt), f"{what}: loaded checkpoint differs from the oracle's rounding"

    # -- conversions
    def to_dev(self, tok):
        """np token dict (one token [B,...] or k tokens [k,B,...]) -> device tensors in io dtype."""
        out = {}
        for k, v in tok.items():
            dt = torch.float32 if k in ("alpha", "beta") else self.iot
            out[k] = dev(v, dt)
        return out

    # -- comparisons
    def check_outputs(self, y_gpu, y_orc, what, tokens=None):
        """tokens: the per-position input dicts behind the outputs (needed for an FP8
        checkpoint, whose measured difference is read out through them)."""
        got = y_gpu.float().cpu().numpy().reshape(np.shape(y_orc))
        assert np.all(np.isfinite(got)), f"{what}: non-finite GPU outputs"
        if self.dS is not None and self.dS.any():
            g = np.asarray(got, np.float64).reshape(-1, self.B, self.H, self.C)
            r = np.asarray(y_orc, np.float64).reshape(g.shape)
            allow = self.tol * np.max(np.abs(r), axis=-1, keepdims=True) + readout_bound(
                self.kname, self.dS, tokens, self.scale)
            over = np.abs(g - r) > allow
            assert not over.any(), f"{what}: {int(over.sum())} outputs beyond the FP8 read-out bound"
            err = np.max(np.abs(g - r), axis=-1) / np.maximum(np.max(np.abs(r), axis=-1), 1e-30)
            self.max_err["y"] = max(self.max_err["y"], float(err.max()))
            return
        err = ro.normwise_error(got, y_orc)
        self.max_err["y"] = max(self.max_err["y"], err)
        assert err <= self.tol, f"{what}: output error {err:.3e} > {self.tol:.1e}"

    def _check_fp8_state(self, what):
        codes = self.st.read_checkpoint().view(torch.uint8).cpu().numpy()
        got = ro.e4m3_decode(codes).reshape(codes.shape)
        ref = self.orc.ckpt
        reloaded = self.orc.fc < self.fc_seen            # a load since the last check: same values again
        self.fp8b.bound[reloaded] = 0.0
        self.fc_seen[reloaded] = 0
        folds = self.orc.fc - self.fc_seen
        for n in range(int(folds.max(initial=0))):
            self.fp8b.advance(folds > n, ref)
        self.fc_seen = self.orc.fc.copy()
        d, frac = self.fp8b.check(got, ref, what)
        self.max_flip_frac = max(self.max_flip_frac, frac)
        if self.rc is not None and d.any():
            qg = ro.read_copy_values(got, self.rc).reshape(got.shape)
            qr = ro.read_copy_values(ref, self.rc).reshape(ref.shape)
            d = np.maximum(d, np.abs(qg - qr))
        self.dS = d

    def check_state(self, what):
        self.check_ckpt(what)
        self._check_book(what)

    def check_ckpt(self, what):
        """The checkpoint against the oracle's (the bookkeeping is not read: a stack member's
        lives in the stack)."""
        torch.cuda.synchronize()
        if self.fp8:
            self._check_fp8_state(what)
            return
        ck = self.st.read_checkpoint().cpu().numpy().astype(np.float64)
        ref = self.orc.ckpt
        num = np.max(np.abs(ck - ref), axis=(2, 3))
        den = np.maximum(np.max(np.abs(ref), axis=(2, 3)), 1e-30)
        err = float(np.max(num / den))
        # an all-zero reference (e.g. a zero checkpoint never folded) must match exactly
        zero = np.max(np.abs(ref), axis=(2, 3)) == 0
        assert np.all(np.max(np.abs(ck), axis=(2, 3))[zero] == 0), f"{what}: nonzero checkpoint where oracle is 0"
        err = float(np.max(np.where(zero, 0.0, num / den)))
        self.max_err["ckpt"] = max(self.max_err["ckpt"], err)
        assert err <= self.ckpt_tol, f"{what}: checkpoint error {err:.3e} > {self.ckpt_tol:.1e}"
        if self.rc is not None:
            # both sides quantize their own checkpoint: values next to a quantization
            # boundary may land on different codes; the difference of the two copies
            # (each quantized by the oracle) is read out by the next non-folding steps
            d = np.abs(ro.read_copy_values(ck, self.rc).reshape(ck.shape)
                       - ro.read_copy_values(ref, self.rc).reshape(ref.shape))
            self.dS = d if d.any() else None

    def _check_book(self, what):
        check_book(self.st.read_book(), self.orc, what)


    # -- operations
    def decode(self, tok, what="decode", check_state=True, active=None):
        """active: optional bool/uint8 [B]; only those sequences step (masked decode) and only
        their outputs are compared."""
        act_dev = None if active is None else dev(np.asarray(active, np.uint8), torch.uint8)
        y = self.st.decode(self.to_dev(tok), self.params, active=act_dev)
        yo = self.orc.decode(tok, active=None if active is None else np.asarray(active, bool))
        if self.fp8:                 # a fold's rounding reaches this step's outputs: check it first
            self.check_state(what)
        yg, yr = y[0], yo
        if active is not None:
            sel = np.flatnonzero(np.asarray(active, bool))
            self._check_rows(y, yo[None], sel, [tok], what)
        else:
            self.check_outputs(yg, yr, what, tokens=[tok])
        if check_state and not self.fp8:
            self.check_state(what)
        return y

    def _check_rows(self, y, yo, sel, tokens, what):
        """Outputs of the sequences `sel` only (masked steps leave the others' rows alone)."""
        if sel.size == 0:
            return
        if self.dS is not None and self.dS.any():
            full = np.zeros_like(self.dS)
            full[sel] = self.dS[sel]
            saved, self.dS = self.dS, full
            try:
                g = y.float().cpu().numpy()
                r = np.array(g, np.float64)
                r[:, sel] = yo[:, sel]
                self.check_outputs(y, r, what, tokens=tokens)
            finally:
                self.dS = saved
            return
        got = y[:, sel.tolist()]
        self.check_outputs(got, yo[:, sel], what, tokens=None)

    def flush(self, what="flush"):
        self.st.flush(self.params)
        self.orc.flush()
        self.check_state(what)

    def spec(self, drafts, what="spec", active=None):
        """drafts: dict of [k, B, ...] arrays."""
        k = next(iter(drafts.values())).shape[0]
        act_dev = None if active is None else dev(np.asarray(active, np.uint8), torch.uint8)
        y = self.st.spec_append(k, self.to_dev(drafts), self.params, active=act_dev)
        toks = [{n: v[j] for n, v in drafts.items()} for j in range(k)]
        yo = self.orc.spec_append(toks, active=None if active is None else np.asarray(active, bool))
        if self.fp8:
            self.check_state(what)
        if active is not None:
            self._check_rows(y, np.stack(yo), np.flatnonzero(np.asarray(active, bool)), toks, what)
        else:
            self.check_outputs(y, np.stack(yo), what, tokens=toks)
        if not self.fp8:
            self.check_state(what)
        return y

    def commit(self, accepted, what="commit"):
        self.st.commit(torch.tensor(np.asarray(accepted, np.int32), device="cuda"))
        self.orc.commit(accepted)
        self.check_state(what)

    def rollback(self, what="rollback"):
        self.st.rollback()
        self.orc.rollback()
        self.check_state(what)

    def load_slots(self, slots, S, what="load_slots"):
        """Sequences `slots` take the fp32 checkpoints S [n, H, rows, cols]."""
        S = np.ascontiguousarray(S, np.float32)
        self.st.load_slots(list(slots), torch.from_numpy(S).cuda())
        self.orc.load_slots(list(slots), S)
        if self.fp8:
            self.fc_seen = self.orc.fc.copy()
            self.fp8b.bound[list(slots)] = 0.0       # both sides round the same fp32 values
        self.check_state(what)


def check_book(book, orc, what):
    """GPU bookkeeping (len, pend, fc, err device tensors) against an oracle session or stack:
    bit-exact."""
    L, P, F, E = book
    got = (L.cpu().numpy(), P.cpu().numpy(), F.cpu().numpy(), int(E.cpu().numpy()[0]))
    oL, oP, oF = orc.trace()
    assert np.array_equal(got[0], oL), f"{what}: len {got[0]} != {oL}"
    assert np.array_equal(got[1], oP), f"{what}: pend {got[1]} != {oP}"
    assert np.array_equal(got[2], oF), f"{what}: fc {got[2]} != {oF}"
    assert got[3] == orc.err, f"{what}: error word {got[3]} != {orc.err}"
