"""GPU parity of long speculative drafts (k up to the full 16-entry buffer) for both layers.

Drafts are appended unverified and evaluated output-only from one checkpoint read
([TR] "NVIDIA ve Dao AI Lab ...", section "Durum trafigini azaltma ve rollback'in
basitlestirilmesi"); with k = 16 every append that follows a committed prefix
pre-flushes it (the overflow reading).  Covers the 16-token kernels (up to 32
virtual entries), one-wave workgroups (head dim 16, where a GDN wave runs four
draft chains at a time), bf16 and fp32 io, and ragged commits.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from hybrid_decode_replay_amd import synth  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_decode_replay_amd import binding  # noqa: F401
    yield


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("C,R,io", [(64, 64, "f32"), (16, 32, "bf16"), (128, 128, "bf16")])
def test_drafts_up_to_buffer_capacity(kind, C, R, io):
    from harness import Pair
    from hybrid_decode_replay_amd import binding as b
    B, H, cap = 3, 2, 16
    G = 1 if kind == "mamba2" else H
    S0 = synth.checkpoint(91, (B, H, C, R))
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap,
                io=b.BF16 if io == "bf16" else b.F32, seed=91, S0=S0)
    if kind == "mamba2":
        toks = synth.mamba2_tokens(91, 120, B, H, G, C, R, dtype=io)
    else:
        toks = synth.gdn_tokens(91, 120, B, H, G, R, C, dtype=io)
    print(f"[long drafts] {kind} C={C} R={R} io={io}", flush=True)
    t = 0
    for _ in range(5):
        pair.decode(synth.token(toks, t)); t += 1
    plan = [(16, [16, 3, 0]), (16, None), (16, [0, 16, 9]), (13, [13, 1, 7]), (16, [2, 16, 16]), (5, None)]
    for k, acc in plan:
        pair.spec({n: v[t:t + k] for n, v in toks.items()}, what=f"spec k={k} at token {t}")
        t += k
        if acc is None:
            pair.rollback(what="rollback")
        else:
            pair.commit(acc, what=f"commit {acc}")
    for _ in range(20):
        pair.decode(synth.token(toks, t)); t += 1
    print("max errors", pair.max_err)
