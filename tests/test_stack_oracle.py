"""CPU pins of the layer-stack oracle (oracle.replay_oracle.StackSession).

A stack is the SSM layers of one model stepped together ([TR] "NVIDIA ve Dao AI
Lab ...", section "ReplaySSM nasil calisir?": hybrid models interleave several
SSM layers).  Pinned here: a one-layer stack is the bare session; each layer of
a mixed stack gives exactly what the same layer gives alone under the same
operations; the step protocol (layer order, one operation and draft count per
step, commit / rollback / flush / load only between steps); and the lockstep of
the layers' bookkeeping against the closed form of lockstep decoding.
"""
import numpy as np
import pytest

from oracle import replay_oracle as ro
from hybrid_decode_replay_amd import synth

B, H, G, P, N = 3, 2, 1, 8, 16


def _mamba2(seed, cap, **kw):
    A, D = synth.mamba2_params(seed, H)
    return ro.Mamba2Session(A, D, synth.checkpoint(seed, (B, H, P, N)), cap=cap, **kw)


def _gdn(seed, cap, **kw):
    return ro.GDNSession(synth.checkpoint(seed, (B, H, P, N)), cap=cap, **kw)


def _toks(kind, seed, T):
    if kind == "mamba2":
        return synth.mamba2_tokens(seed, T, B, H, G, P, N)
    return synth.gdn_tokens(seed, T, B, H, H, N, P)


def _cut(toks, a, b):
    return [synth.token(toks, t) for t in range(a, b)]


def test_one_layer_stack_is_the_session():
    cap = 4
    bare, inner = _mamba2(70, cap), _mamba2(70, cap)
    stk = ro.StackSession([inner])
    toks = _toks("mamba2", 70, 20)
    for t in range(6):
        np.testing.assert_array_equal(stk.decode_layer(0, synth.token(toks, t)), bare.decode(synth.token(toks, t)))
    for a, b in zip(stk.spec_layer(0, _cut(toks, 6, 9)), bare.spec_append(_cut(toks, 6, 9))):
        np.testing.assert_array_equal(a, b)
    stk.commit([3, 0, 1])
    bare.commit([3, 0, 1])
    stk.flush()
    bare.flush()
    for x, y in zip(stk.trace(), bare.trace()):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(inner.ckpt, bare.ckpt)


def test_mixed_stack_layers_match_lone_layers():
    """Mamba-2, GDN and an fp16-checkpoint Mamba-2 layer in one stack: each layer's outputs
    and checkpoint equal those of the same layer driven alone through the same operations."""
    cap = 5
    mk = [lambda: _mamba2(71, cap), lambda: _gdn(72, cap), lambda: _mamba2(73, cap, ckpt_dtype="f16")]
    kinds = ["mamba2", "gdn", "mamba2"]
    stk = ro.StackSession([m() for m in mk])
    alone = [m() for m in mk]
    toks = [_toks(k, 74 + i, 30) for i, k in enumerate(kinds)]
    for t in range(7):
        for l in range(3):
            np.testing.assert_array_equal(stk.decode_layer(l, synth.token(toks[l], t)),
                                          alone[l].decode(synth.token(toks[l], t)))
    for l in range(3):
        for a, b in zip(stk.spec_layer(l, _cut(toks[l], 7, 11)), alone[l].spec_append(_cut(toks[l], 7, 11))):
            np.testing.assert_array_equal(a, b)
    stk.commit([4, 2, 0])
    for s in alone:
        s.commit([4, 2, 0])
    for t in range(11, 16):
        for l in range(3):
            np.testing.assert_array_equal(stk.decode_layer(l, synth.token(toks[l], t)),
                                          alone[l].decode(synth.token(toks[l], t)))
    for l in range(3):
        np.testing.assert_array_equal(stk.layers[l].ckpt, alone[l].ckpt)
    stk.trace()


def test_step_protocol():
    cap = 4
    stk = ro.StackSession([_mamba2(75, cap), _gdn(76, cap)])
    tm, tg = _toks("mamba2", 75, 12), _toks("gdn", 76, 12)
    with pytest.raises(ro.PhaseError):
        stk.decode_layer(1, synth.token(tg, 0))            # layer 0 comes first
    stk.decode_layer(0, synth.token(tm, 0))
    with pytest.raises(ro.PhaseError):
        stk.spec_layer(1, _cut(tg, 0, 2))                   # the step is a decode step
    with pytest.raises(ro.PhaseError):
        stk.flush()                                         # not between steps
    with pytest.raises(ro.PhaseError):
        stk.trace()
    stk.decode_layer(1, synth.token(tg, 0))
    stk.spec_layer(0, _cut(tm, 1, 4))
    with pytest.raises(ro.PhaseError):
        stk.spec_layer(1, _cut(tg, 1, 3))                   # k = 2 after k = 3
    with pytest.raises(ro.PhaseError):
        stk.commit([1, 1, 1])
    stk.spec_layer(1, _cut(tg, 1, 4))
    with pytest.raises(ro.PhaseError):
        stk.decode_layer(0, synth.token(tm, 4))             # drafts pending for the stack
    stk.commit([3, 1, 0])
    np.testing.assert_array_equal(stk.trace()[0], [4, 2, 1])
    with pytest.raises(ValueError):
        ro.StackSession([_mamba2(75, 4), _gdn(76, 5)])     # capacities differ
    with pytest.raises(ValueError):
        ro.StackSession([])


def test_lockstep_closed_form():
    """T lockstep decode steps through a three-layer stack: len = T mod cap and fc = T div cap
    in every layer (no layer drifts), with the stagger flag: fc = number of window ends
    1 + (b mod cap) + j cap <= T."""
    cap, T = 3, 11
    for stagger in (False, True):
        stk = ro.StackSession([_mamba2(77, cap, stagger=stagger), _gdn(78, cap, stagger=stagger),
                               _mamba2(79, cap, stagger=stagger)])
        toks = [_toks(k, 80 + i, T) for i, k in enumerate(["mamba2", "gdn", "mamba2"])]
        for t in range(T):
            for l in range(3):
                stk.decode_layer(l, synth.token(toks[l], t))
        L, pend, fc = stk.trace()
        first = 1 + np.arange(B) % cap if stagger else np.full(B, cap)
        want_fc = np.where(T >= first, 1 + (T - first) // cap, 0)
        want_len = np.where(T >= first, (T - first) % cap, T)
        np.testing.assert_array_equal(fc, want_fc)
        np.testing.assert_array_equal(L, want_len)
        np.testing.assert_array_equal(pend, 0)
