"""CPU pins of the oracle's read-copy outputs (decode and speculative drafts), off the copy's grid.

The recurrence is linear in the state it starts from, so an output computed from
the dequantized copy Q(S0) of a checkpoint S0 differs from the full-precision
output by the read-out of Q(S0) - S0 carried through the same tokens:
  Mamba-2   y_copy - y_full = e^{A sum dt} (Q(S0) - S0) C_t      (per head, row p)
            with the sum over every token since the checkpoint (history, then
            drafts 0..j for draft j);
  GDN       o_copy - o_full = scale (Q(S0) - S0) M_1 ... M_t q_t,
            M_i = alpha_i (I - beta_i k_i k_i^T), written out as dense matrices.
A sequence whose committed prefix was folded before the drafts reads the folded
full-precision state, so its outputs equal the no-copy outputs exactly.  These
closed forms share nothing with the op runner's replay loops; Q comes from the
oracle's quantizers, pinned on their own by OCP tables in test_oracle_pins.py.
([TR] "NVIDIA ve Dao AI Lab ...", section "Kuantizasyon hatasinin
sinirlandirilmasi": reads from the low-precision copy; section "Durum trafigini
azaltma ve rollback'in basitlestirilmesi": output-only draft evaluation.)

Planted mistakes in a copy of the op runner's source (the copy is loaded as a
separate module; the real oracle is untouched) must each fail the pin.
"""
import importlib.util
import os
import sys

import numpy as np
import pytest

from hybrid_decode_replay_amd import synth
from oracle import replay_oracle as ro

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "replay_oracle.py")


def _scenario(mod, kind, fmt, seed=80):
    """Decode to a flush, decode more, spec 2 drafts, commit a ragged prefix, then spec 2 drafts
    again so that one sequence pre-flushes and two read the copy with histories of 1 and 2.
    Returns per-op lists (copy outputs, full outputs, closed-form differences, pre-flush mask)."""
    B, cap = 3, 4
    if kind == "mamba2":
        H, G, P, N = 2, 1, 3, 32
        A, D = synth.mamba2_params(seed, H)
        S0 = synth.checkpoint(seed, (B, H, P, N), std=1.0)
        toks = synth.mamba2_tokens(seed, 40, B, H, G, P, N)
        rc = mod.Mamba2Session(A, D, S0, cap=cap, read_copy=fmt)
        fp = mod.Mamba2Session(A, D, S0, cap=cap)
    else:
        H, DK, DV = 2, 32, 3
        S0 = synth.checkpoint(seed, (B, H, DV, DK), std=1.0)
        toks = synth.gdn_tokens(seed, 40, B, H, H, DK, DV)
        rc = mod.GDNSession(S0, cap=cap, read_copy=fmt, scale=0.5)
        fp = mod.GDNSession(S0, cap=cap, scale=0.5)
        A = None
    seen = [[] for _ in range(B)]       # tokens since each sequence's last fold, in order
    ck = [np.array(S0[b], np.float64) for b in range(B)]

    def closed(b, extra):
        """Output difference predicted by linearity for sequence b after seen[b] + extra."""
        d0 = ro.read_copy_values(ck[b][None], fmt).reshape(ck[b].shape) - ck[b]
        seq = seen[b] + extra
        last = seq[-1]
        if kind == "mamba2":
            Hh = d0.shape[0]
            g = np.arange(Hh) // (Hh // last["Cm"].shape[0])
            dsum = np.sum([t_["dt"] for t_ in seq], axis=0)
            return np.exp(A * dsum)[:, None] * np.einsum("hpn,hn->hp", d0, last["Cm"][g])
        out = []
        for h in range(d0.shape[0]):
            M = np.eye(d0.shape[2])
            for t_ in seq:
                k = t_["k"][h]
                M = M @ (t_["alpha"][h] * (np.eye(k.size) - t_["beta"][h] * np.outer(k, k)))
            out.append(0.5 * (d0[h] @ M) @ last["q"][h])
        return np.stack(out)

    def one(tok, b):
        return {k: np.asarray(v[b], np.float64) for k, v in tok.items()}

    log = []
    t = 0
    # decode to the first flush and two more tokens
    for _ in range(cap + 2):
        tok = synth.token(toks, t); t += 1
        fc0 = rc.fc.copy()
        yc, yf = rc.decode(tok), fp.decode(tok)
        for b in range(B):
            if rc.fc[b] != fc0[b]:
                seen[b] = []
                ck[b] = np.array(fp.S[b])
                log.append(("decode-fold", b, yc[b], yf[b], None))
            else:
                log.append(("decode", b, yc[b], yf[b], closed(b, [one(tok, b)])))
                seen[b].append(one(tok, b))
    drafts = [synth.token(toks, t + j) for j in range(2)]; t += 2
    ycs, yfs = rc.spec_append(drafts), fp.spec_append(drafts)
    for j in range(2):
        for b in range(B):
            log.append(("spec", b, ycs[j][b], yfs[j][b], closed(b, [one(drafts[i], b) for i in range(j + 1)])))
    acc = [0, 1, 2]
    rc.commit(acc); fp.commit(acc)
    for b in range(B):
        seen[b] += [one(drafts[i], b) for i in range(acc[b])]
    # len is now 2, 3, 4: drafts of 2 pre-flush sequences 1 and 2
    drafts = [synth.token(toks, t + j) for j in range(2)]; t += 2
    pre = rc.len + 2 > cap
    ycs, yfs = rc.spec_append(drafts), fp.spec_append(drafts)
    for j in range(2):
        for b in range(B):
            if pre[b]:
                log.append(("spec-preflush", b, ycs[j][b], yfs[j][b], None))
            else:
                log.append(("spec", b, ycs[j][b], yfs[j][b],
                            closed(b, [one(drafts[i], b) for i in range(j + 1)])))
    return log, pre


def _pin(mod, kind, fmt):
    log, pre = _scenario(mod, kind, fmt)
    assert pre.tolist() == [False, True, True]
    nonzero = 0
    for what, b, yc, yf, want in log:
        if want is None:
            np.testing.assert_array_equal(yc, yf, err_msg=f"{what} b={b}")
            continue
        got = yc - yf
        scale = max(np.max(np.abs(yf)), 1.0)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * scale, err_msg=f"{what} b={b}")
        nonzero += int(np.max(np.abs(want)) > 1e-6)
    assert nonzero >= 10, "the scenario must read copies that differ from the checkpoint"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_read_copy_outputs_closed_form(kind, fmt):
    _pin(ro, kind, fmt)


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, old
    spec = importlib.util.spec_from_loader("replay_oracle_mutant", loader=None, origin=SRC)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = SRC
    exec(compile(text.replace(old, new), SRC + " (mutant)", "exec"), mod.__dict__)
    mod.use_library(ro.lib())
    return mod


MUTANTS = {
    "draft_prefix_short": ("for jj in range(j + 1):", "for jj in range(max(j, 1)):"),
    "history_after_drafts": (
        "                    for past in self.hist[b]:\n                        self._token(Sq, past)\n"
        "                    for jj in range(j + 1):\n                        yq = self._token(Sq, self._slice(drafts[jj], b))\n",
        "                    for jj in range(j + 1):\n                        yq = self._token(Sq, self._slice(drafts[jj], b))\n"
        "                    for past in self.hist[b]:\n                        self._token(Sq, past)\n"),
    "copy_on_preflushed_rows": ("for b in np.flatnonzero(act & ~pre):", "for b in np.flatnonzero(act):"),
    "spec_reads_full_precision": (
        "                    Sq = read_copy_values(self.ckpt[b:b + 1], self.read_copy).copy()\n"
        "                    for past in self.hist[b]:",
        "                    Sq = self.ckpt[b:b + 1].copy()\n                    for past in self.hist[b]:"),
    "decode_reads_full_precision": (
        "        S = read_copy_values(self.ckpt[b:b + 1], self.read_copy).copy()\n        for past in self.hist[b]:",
        "        S = self.ckpt[b:b + 1].copy()\n        for past in self.hist[b]:"),
    "decode_skips_history": (
        "        for past in self.hist[b]:\n            self._token(S, past)\n        return self._token(S, self._slice(inp, b))[0]",
        "        return self._token(S, self._slice(inp, b))[0]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_the_pin(name):
    mod = _mutant(*MUTANTS[name])
    caught = 0
    for kind in ("mamba2", "gdn"):
        for fmt in ("fp8", "mxfp4"):
            try:
                _pin(mod, kind, fmt)
            except AssertionError:
                caught += 1
    assert caught == 4, f"mutant {name} passed the read-copy pin in {4 - caught} of 4 cases"
