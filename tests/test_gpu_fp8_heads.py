"""Mamba-2 steps on an FP8 checkpoint with four heads of a group per workgroup (the form
the batch-256 layer takes) at a few hundred sequences: parity with the oracle through
folds, masked steps, per-slot arrivals, a speculative round and its commit, bf16 and fp32
io, buffer capacities 16, 5 and 1 (with one entry, a decode after a committed draft folds
the draft and the token in one pass and rounds the checkpoint once), tests/harness.py
FP8 element-wise bound."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from hybrid_decode_replay_amd import synth  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_decode_replay_amd import binding  # noqa: F401  (fails loudly if not built)
    yield


@pytest.mark.parametrize("io,cap,B", [("bf16", 16, 208), ("f32", 5, 200), ("bf16", 1, 196)])
def test_fp8_four_head_steps(io, cap, B):
    from harness import Pair
    from hybrid_decode_replay_amd import binding as b
    H, G, C, R = 16, 4, 64, 128                   # 4 heads per group: B * 4 work items
    seed = 500 + cap
    S0 = synth.checkpoint(seed, (B, H, C, R))
    pair = Pair(b.MAMBA2, B, H, G, C, R, cap=cap, io=b.BF16 if io == "bf16" else b.F32, seed=seed, S0=S0,
                ckpt=b.FP8_E4M3)
    toks = synth.mamba2_tokens(seed, 3 * cap + 24, B, H, G, C, R, dtype=io)
    rng = np.random.default_rng(seed)
    print(f"[fp8 four-head] B {B} cap {cap} io {io}", flush=True)
    t = 0
    for step in range(cap + 3):                  # a full window (fold) and a partial one
        pair.decode(synth.token(toks, t), what=f"decode {step}"); t += 1
    for step in range(4):                         # sequences leaving and joining
        active = rng.random(B) < 0.6
        pair.decode(synth.token(toks, t), what=f"masked decode {step}", active=active); t += 1
    slots = rng.choice(B, size=7, replace=False)
    pair.load_slots(slots, synth.checkpoint(seed + 1, (7, H, C, R)), what="arrivals")
    k = min(3, cap)
    pair.spec({n: v[t:t + k] for n, v in toks.items()}, what="spec round"); t += k
    pair.commit(rng.integers(0, k + 1, size=B), what="commit")
    for step in range(cap + 2):
        pair.decode(synth.token(toks, t), what=f"decode after spec {step}"); t += 1
