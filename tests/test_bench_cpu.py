"""CPU checks of the benchmark's speculative byte count.

bench.spec_bytes counts the bytes of seeded speculative rounds from the accepted
counts alone, simulating the per-sequence bookkeeping it implies (a round whose
committed entries plus k drafts exceed the buffer folds the committed prefix
first; the accepted prefix then advances the pointer).  Here that simulation is
checked against the oracle's own bookkeeping machine on the same counts, and the
byte total against a count made from the oracle's lengths before every round
([TR] "NVIDIA ve Dao AI Lab ...", section "Durum trafigini azaltma ve
rollback'in basitlestirilmesi": drafts appended, the accepted prefix advances
the buffer pointer).
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hybrid_decode_replay_amd import synth  # noqa: E402
from oracle import replay_oracle as ro  # noqa: E402


@pytest.mark.parametrize("kind,cap,k", [("mamba2", 4, 3), ("gdn", 5, 2), ("mamba2", 16, 4)])
def test_spec_bytes_bookkeeping_matches_oracle(kind, cap, k):
    B, rounds, seed = 6, 14, 21
    rng = np.random.default_rng(seed)
    acc = np.minimum(rng.geometric(0.35, size=(rounds, B)) - 1, k).astype(np.int32)
    if kind == "mamba2":
        H, G, C, R = 2, 1, 4, 16
        A, D = synth.mamba2_params(seed, H)
        sess = ro.Mamba2Session(A, D, synth.checkpoint(seed, (B, H, C, R)), cap=cap)
        toks = synth.mamba2_tokens(seed, rounds * k, B, H, G, C, R)
    else:
        H, G, C, R = 2, 2, 8, 16
        sess = ro.GDNSession(synth.checkpoint(seed, (B, H, C, R)), cap=cap)
        toks = synth.gdn_tokens(seed, rounds * k, B, H, G, R, C)
    lens_before = []
    for r in range(rounds):
        lens_before.append(sess.trace()[0].copy())
        sess.spec_append([synth.token(toks, r * k + j) for j in range(k)])
        sess.commit(acc[r])
    total, lens, folds = bench.spec_bytes(kind, H, G, C, R, cap, k, acc)
    ln, pend, fc = sess.trace()
    assert np.array_equal(lens, ln) and np.array_equal(folds, fc) and not pend.any()
    # the byte total from the oracle's own lengths: checkpoint and drafts every round,
    # the committed entries read, a checkpoint write per folded prefix
    entry, inp, out = bench.token_sizes(kind, H, G, C, R)
    S = H * C * R * 4
    hist = int(sum(l.sum() for l in lens_before))
    expect = rounds * B * (S + k * (inp + entry + out)) + hist * entry + int(fc.sum()) * S
    assert total == expect


def test_spec_bytes_full_acceptance_closed_form():
    """Every draft accepted, cap 16, k 4: lengths 0, 4, 8, 12 before the rounds of each
    cycle, then 16 + 4 > 16 folds; so one fold per four rounds after the first cycle."""
    rounds, B, k, cap = 13, 3, 4, 16
    acc = np.full((rounds, B), k, np.int32)
    total, lens, folds = bench.spec_bytes("gdn", 2, 2, 8, 16, cap, k, acc)
    # rounds 0..3 reach 16; rounds 4, 8, 12 fold (len 16 + 4 > 16), each restarting at 0
    assert folds.tolist() == [3] * B
    assert lens.tolist() == [4] * B
