"""CPU pins of the oracle's ragged-batch operations: masked steps and per-slot loads.

Pinned by
  * hand-derived bookkeeping traces (tests/golden/bookkeeping_ragged_cap4.txt,
    tests/golden/bookkeeping_stagger_slots_cap4.txt), compared bit for bit;
  * invariants that do not go through the masking code: a sequence left out of a
    step keeps its state bit for bit, and the sequences that step get exactly
    the outputs and states of a session holding only them; after a per-slot
    load the arriving sequence decodes exactly as a fresh session loaded with
    the same checkpoint, and the other sequences exactly as if no load happened.
Sources: every sequence flushes its own buffer ([TR] "NVIDIA ve Dao AI Lab ...",
section "ReplaySSM nasil calisir?"); the gain comes from many concurrent
sequences ([DE] "ReplaySSM beschleunigt ...", section "Warum es wichtig ist").
"""
import os

import numpy as np
import pytest

from hybrid_decode_replay_amd import synth
from oracle import replay_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                tok = line.split()
                out.append((tok[0], tok[1], list(map(int, tok[2:]))))
    return out


def _mask(s):
    return np.array([c == "1" for c in s])


@pytest.mark.parametrize("name,stagger", [("bookkeeping_ragged_cap4.txt", False),
                                          ("bookkeeping_stagger_slots_cap4.txt", True)])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_ragged_golden_trace(name, stagger, kind):
    B, H, cap = 3, 1, 4
    if kind == "mamba2":
        P, N = 2, 2
        A, D = synth.mamba2_params(70, H)
        sess = ro.Mamba2Session(A, D, np.zeros((B, H, P, N)), cap=cap, stagger=stagger)
        toks = synth.mamba2_tokens(70, 64, B, H, 1, P, N)
        shape = (H, P, N)
    else:
        DK = DV = 2
        sess = ro.GDNSession(np.zeros((B, H, DV, DK)), cap=cap, stagger=stagger)
        toks = synth.gdn_tokens(70, 64, B, H, H, DK, DV)
        shape = (H, DV, DK)
    t = 0
    for op, arg, want in _rows(name):
        if op == "decode":
            sess.decode(synth.token(toks, t), active=_mask(arg)); t += 1
        elif op == "spec":
            k, m = arg.split(":")
            sess.spec_append([synth.token(toks, t + j) for j in range(int(k))], active=_mask(m)); t += int(k)
        elif op == "commit":
            sess.commit([int(a) for a in arg.split(",")])
        elif op == "load":
            slots = [int(a) for a in arg.split(",")]
            sess.load_slots(slots, synth.checkpoint(71, (len(slots),) + shape))
        elif op == "flush":
            sess.flush()
        L, Pd, F = sess.trace()
        got = list(L) + list(Pd) + list(F) + [sess.err]
        assert got == want, (op, arg, got, want)


def _layer(kind, B, seed, cap=4, read_copy=None, ckpt_dtype="f32"):
    if kind == "mamba2":
        H, G, P, N = 2, 1, 3, 32
        A, D = synth.mamba2_params(seed, H)
        S0 = synth.checkpoint(seed, (B, H, P, N), std=0.5)
        toks = synth.mamba2_tokens(seed, 60, B, H, G, P, N)

        def mk(S, rc=read_copy):
            return ro.Mamba2Session(A, D, S, cap=cap, read_copy=rc, ckpt_dtype=ckpt_dtype)
        return mk, S0, toks
    H, DK, DV = 2, 32, 3
    S0 = synth.checkpoint(seed, (B, H, DV, DK), std=0.5)
    toks = synth.gdn_tokens(seed, 60, B, H, H, DK, DV)

    def mk(S, rc=read_copy):
        return ro.GDNSession(S, cap=cap, read_copy=rc, ckpt_dtype=ckpt_dtype)
    return mk, S0, toks


def _sub(tok, rows):
    return {k: v[rows] for k, v in tok.items()}


@pytest.mark.parametrize("rc,ckd", [(None, "f32"), ("mxfp4", "f32"), (None, "fp8")])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_masked_decode_equals_sub_batch(kind, rc, ckd):
    """Masked decoding of a batch equals decoding only the active sequences in a session of
    their own, step by step (outputs and checkpoints bit for bit); a left-out sequence keeps
    its state, checkpoint and bookkeeping bit for bit."""
    B = 4
    mk, S0, toks = _layer(kind, B, 72, read_copy=rc, ckpt_dtype=ckd)
    full = mk(S0)
    masks = [_mask(m) for m in ("1111", "1010", "0111", "1101", "1010", "0000", "1111", "0101", "1011", "1110")]
    rows = [np.flatnonzero(m) for m in masks]
    # one private session per sequence, fed exactly that sequence's steps
    solo = [mk(S0[b:b + 1]) for b in range(B)]
    for t, (m, r) in enumerate(zip(masks, rows)):
        before = (full.S.copy(), full.len.copy(), full.fc.copy())
        y = full.decode(synth.token(toks, t), active=m)
        for b in range(B):
            if m[b]:
                yb = solo[b].decode(_sub(synth.token(toks, t), [b]))
                np.testing.assert_array_equal(y[b], yb[0])
                np.testing.assert_array_equal(full.S[b], solo[b].S[0])
                np.testing.assert_array_equal(full.ckpt[b], solo[b].ckpt[0])
                assert (full.len[b], full.fc[b]) == (solo[b].len[0], solo[b].fc[0])
            else:
                np.testing.assert_array_equal(full.S[b], before[0][b])
                assert (full.len[b], full.fc[b]) == (before[1][b], before[2][b])
                assert not y[b].any()


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_masked_spec_equals_sub_batch(kind):
    B = 3
    mk, S0, toks = _layer(kind, B, 73, read_copy="fp8")
    full = mk(S0)
    solo = [mk(S0[b:b + 1]) for b in range(B)]
    for t in range(2):
        full.decode(synth.token(toks, t))
        for b in range(B):
            solo[b].decode(_sub(synth.token(toks, t), [b]))
    m = _mask("101")
    drafts = [synth.token(toks, 2 + j) for j in range(3)]
    ys = full.spec_append(drafts, active=m)
    for b in (0, 2):
        yb = solo[b].spec_append([_sub(d, [b]) for d in drafts])
        for j in range(3):
            np.testing.assert_array_equal(ys[j][b], yb[j][0])
    assert not any(ys[j][1].any() for j in range(3))
    assert list(full.pend) == [3, 0, 3]
    full.commit([2, 0, 3])
    solo[0].commit([2]); solo[2].commit([3])
    for b in (0, 2):
        np.testing.assert_array_equal(full.S[b], solo[b].S[0])
        assert full.len[b] == solo[b].len[0]
    np.testing.assert_array_equal(full.S[1], solo[1].S[0])


@pytest.mark.parametrize("ckd", ["f32", "f16", "fp8"])
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_load_slots_is_a_fresh_sequence(kind, ckd):
    """After load_slots, an arriving sequence decodes exactly as a fresh session loaded with
    its checkpoint (rounded the same way) and fed the same tokens; the others decode exactly
    as in a session where the load never happened."""
    B = 4
    mk, S0, toks = _layer(kind, B, 74, ckpt_dtype=ckd)
    a, ref = mk(S0), mk(S0)
    for t in range(6):
        a.decode(synth.token(toks, t))
        ref.decode(synth.token(toks, t))
    S_new = synth.checkpoint(75, (2,) + S0.shape[1:], std=0.7)
    slots = [3, 1]
    a.load_slots(slots, S_new)
    fresh = [mk(S_new[i:i + 1]) for i in range(2)]
    for i, b in enumerate(slots):
        np.testing.assert_array_equal(a.ckpt[b], fresh[i].ckpt[0])
        assert (a.len[b], a.pend[b], a.fc[b], a.lim[b]) == (0, 0, 0, a.cap)
    for t in range(6, 17):
        tok = synth.token(toks, t)
        y = a.decode(tok)
        yr = ref.decode(tok)
        for b in (0, 2):
            np.testing.assert_array_equal(y[b], yr[b])
        for i, b in enumerate(slots):
            np.testing.assert_array_equal(y[b], fresh[i].decode(_sub(tok, [b]))[0])
    for b in (0, 2):
        np.testing.assert_array_equal(a.S[b], ref.S[b])


def test_ragged_phase_rules():
    mk, S0, toks = _layer("mamba2", 2, 76)
    s = mk(S0)
    s.spec_append([synth.token(toks, 0)], active=np.array([False, False]))
    assert not s.pend.any()
    for bad in (lambda: s.decode(synth.token(toks, 1)), lambda: s.load_slots([0], S0[:1]),
                lambda: s.spec_append([synth.token(toks, 1)])):
        with pytest.raises(ro.PhaseError):
            bad()
    s.rollback()
    with pytest.raises(ValueError):
        s.load_slots([1, 1], S0)
    with pytest.raises(ValueError):
        s.load_slots([2], S0[:1])
