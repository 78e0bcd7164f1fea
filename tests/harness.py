"""Drive the HIP library and the fp64 oracle side by side on identical seeded inputs.

Test-side helper.  Inputs come from the seeded generators (synth); the oracle
never sees a value produced by the HIP path.  Each operation is applied to both
sides and the outputs, the checkpoint (read back in logical layout) and the
bookkeeping are compared:
  outputs      normwise relative error per output vector <= tol
  checkpoint   normwise relative error per (b, h) matrix <= tol
  bookkeeping  len, pend, fc and the error word bit-exact

With an fp16 checkpoint both sides round every fold to binary16 on their own
(the GPU from its fp32 fold, the oracle from fp64).  The two fold results differ
by fp32 rounding only, so they round to the same binary16 value except within
that distance of a rounding boundary, where they land one ulp apart (at most
2^-10 relative).  A test runs at most four folds, and a difference left by one
fold is carried (scaled by decays <= 1) into the next, so 4 x 2^-10 ~ 3.9e-3
bounds outputs and checkpoints: TOL_F16.

With an FP8 (E4M3) checkpoint the same holds with one E4M3 step (up to 2^-3
relative) in place of one binary16 ulp, which is too coarse for a norm bound to
say much.  The checkpoint is therefore compared element by element: an element
may differ only by one step of the E4M3 grid (a fold result that the two sides'
roundings put on either side of a midpoint), and such elements must be rare:
the fp32 fold is within ~1e-6 relative of the fp64 one and E4M3 steps are at
least 2^-4 relative, so about 3e-5 of the elements per fold land there;
FP8_FLIP_FRAC = 1e-3 bounds a test's folds with a wide margin.  A (b, h) matrix
that ever differed is marked; outputs of unmarked matrices keep the io dtype's
tolerance, outputs of marked ones only a loose bound of one E4M3 step
(FP8_TOL_MARKED).  Pair(..., tol=0.0) asks for bit-exact outputs and
checkpoints (inputs chosen so that every result is exact in fp32).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import replay_oracle as ro
from hybrid_decode_replay_amd import binding as rb

TOL = {rb.F32: 1e-4, rb.BF16: 2e-2}
TOL_F16 = 4 * 2.0 ** -10
FP8_FLIP_FRAC = 1e-3
FP8_TOL_MARKED = 2.0 ** -3


def e4m3_grid_index(v):
    """Position of E4M3 values on the sorted grid of finite E4M3 values (+0 and -0 merged)."""
    grid = ro.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    v = np.asarray(v, np.float64)
    idx = np.searchsorted(grid, v)
    assert np.array_equal(grid[np.minimum(idx, grid.size - 1)], v), "value off the E4M3 grid"
    return idx


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
        if tol is not None:
            self.tol = tol
        self.fp8 = ckpt == rb.FP8_E4M3
        self.B, self.H, self.G, self.C, self.R = B, H, G, C, R
        if S0 is None:
            S0 = np.zeros((B, H, C, R), np.float32)
        # both sides start from the checkpoint dtype's values
        if ckpt == rb.F16:
            S0 = np.asarray(S0, np.float32).astype(np.float16)
        elif self.fp8:
            S0 = ro.e4m3_decode(ro.e4m3_encode(S0)).reshape(np.shape(S0)).astype(np.float32)
        self.st = rb.ReplayState(self.cfg)
        self.st.load_checkpoint(torch.from_numpy(np.ascontiguousarray(S0)).cuda())
        rc = {rb.NONE: None, rb.FP8_E4M3: "fp8", rb.MXFP4: "mxfp4"}[read_copy]
        cd = {rb.F16: "f16", rb.FP8_E4M3: "fp8"}.get(ckpt, "f32")
        self.marked = np.zeros((B, H), bool)      # FP8: matrices whose checkpoint ever differed
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
        self.max_err = {"y": 0.0, "ckpt": 0.0}

    # -- conversions
    def to_dev(self, tok):
        """np token dict (one token [B,...] or k tokens [k,B,...]) -> device tensors in io dtype."""
        out = {}
        for k, v in tok.items():
            dt = torch.float32 if k in ("alpha", "beta") else self.iot
            out[k] = dev(v, dt)
        return out

    # -- comparisons
    def check_outputs(self, y_gpu, y_orc, what):
        got = y_gpu.float().cpu().numpy().reshape(np.shape(y_orc))
        assert np.all(np.isfinite(got)), f"{what}: non-finite GPU outputs"
        if self.fp8 and self.marked.any():
            g = np.asarray(got, np.float64)
            r = np.asarray(y_orc, np.float64)
            err = np.max(np.abs(g - r), axis=-1) / np.maximum(np.max(np.abs(r), axis=-1), 1e-30)
            marked = np.broadcast_to(self.marked, err.shape)
            clean = float(np.max(err[~marked], initial=0.0))
            loose = float(np.max(err[marked], initial=0.0))
            self.max_err["y"] = max(self.max_err["y"], clean)
            self.max_err["y_marked"] = max(self.max_err.get("y_marked", 0.0), loose)
            assert clean <= self.tol, f"{what}: output error {clean:.3e} > {self.tol:.1e}"
            assert loose <= FP8_TOL_MARKED, f"{what}: output error {loose:.3e} (marked matrices)"
            return
        err = ro.normwise_error(got, y_orc)
        self.max_err["y"] = max(self.max_err["y"], err)
        assert err <= self.tol, f"{what}: output error {err:.3e} > {self.tol:.1e}"

    def _check_fp8_state(self, what):
        codes = self.st.read_checkpoint().view(torch.uint8).cpu().numpy()
        got = ro.e4m3_decode(codes).reshape(codes.shape)
        ref = self.orc.ckpt
        diff = got != ref
        if diff.any():
            step = np.abs(e4m3_grid_index(got[diff]) - e4m3_grid_index(ref[diff]))
            assert step.max() <= 1, f"{what}: checkpoint differs by {step.max()} E4M3 steps"
        frac = float(diff.mean())
        self.max_flip_frac = max(self.max_flip_frac, frac)
        limit = 0.0 if self.tol == 0.0 else FP8_FLIP_FRAC
        assert frac <= limit, f"{what}: {frac:.2e} of the checkpoint one E4M3 step off (> {limit:.0e})"
        self.marked |= diff.any(axis=(2, 3))

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
        assert err <= self.tol, f"{what}: checkpoint error {err:.3e} > {self.tol:.1e}"

    def _check_book(self, what):
        check_book(self.st.read_book(), self.orc, what)


    # -- operations
    def decode(self, tok, what="decode", check_state=True):
        y = self.st.decode(self.to_dev(tok), self.params)
        yo = self.orc.decode(tok)
        if self.fp8:                 # a fold's rounding reaches this step's outputs: mark first
            self.check_state(what)
        self.check_outputs(y[0], yo, what)
        if check_state and not self.fp8:
            self.check_state(what)
        return y

    def flush(self, what="flush"):
        self.st.flush(self.params)
        self.orc.flush()
        self.check_state(what)

    def spec(self, drafts, what="spec"):
        """drafts: dict of [k, B, ...] arrays."""
        k = next(iter(drafts.values())).shape[0]
        y = self.st.spec_append(k, self.to_dev(drafts), self.params)
        yo = self.orc.spec_append([{n: v[j] for n, v in drafts.items()} for j in range(k)])
        if self.fp8:
            self.check_state(what)
        self.check_outputs(y, np.stack(yo), what)
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
