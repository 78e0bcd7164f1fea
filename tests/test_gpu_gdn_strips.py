"""Gated DeltaNet steps whose waves own two 16-column strips each (d_k = 128, d_v a
multiple of 128, an fp16 or FP8 checkpoint or a read copy): parity with the oracle
through decode, flushes, speculative appends (with and without a pre-flush),
commits, rollbacks and masked steps, at small batch (tests/harness.py)."""
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


CASES = [  # (d_v, io, checkpoint, read copy)
    (128, "f32", "f16", None), (128, "bf16", "fp8", None), (256, "f32", "fp8", None),
    (128, "f32", "f32", "fp8"), (128, "bf16", "f32", "mxfp4"), (256, "bf16", "f32", "fp8"),
    (128, "f32", "fp8", "mxfp4"), (128, "bf16", "f16", "mxfp4"),
]


@pytest.mark.parametrize("DV,io,ck,rc", CASES)
def test_two_strip_waves(DV, io, ck, rc):
    from harness import Pair
    from hybrid_decode_replay_amd import binding as b
    B, H, DK, cap = 3, 2, 128, 8
    seed = 300 + DV + len(io) + len(ck) + (len(rc) if rc else 0)
    S0 = synth.checkpoint(seed, (B, H, DV, DK))
    pair = Pair(b.GDN, B, H, H, DV, DK, cap=cap, io=b.BF16 if io == "bf16" else b.F32, seed=seed, S0=S0,
                scale=0.5, ckpt={"f32": b.F32, "f16": b.F16, "fp8": b.FP8_E4M3}[ck],
                read_copy={None: b.NONE, "fp8": b.FP8_E4M3, "mxfp4": b.MXFP4}[rc])
    toks = synth.gdn_tokens(seed, 80, B, H, H, DK, DV, dtype=io)
    rng = np.random.default_rng(seed)
    t = 0
    print(f"[gdn two-strip] d_v {DV} io {io} ckpt {ck} copy {rc}", flush=True)
    for step in range(11):                                 # one fold, then a partial window
        pair.decode(synth.token(toks, t), what=f"decode {step}"); t += 1
    pair.spec({n: v[t:t + 3] for n, v in toks.items()}, what="spec k=3"); t += 3
    pair.commit(np.array([3, 1, 0]), what="commit")
    pair.spec({n: v[t:t + 6] for n, v in toks.items()}, what="spec k=6 with a pre-flush"); t += 6
    pair.rollback(what="rollback")
    active = np.array([1, 0, 1], bool)
    for step in range(5):
        pair.decode(synth.token(toks, t), what=f"masked decode {step}", active=active); t += 1
        active = rng.random(B) < 0.7
    pair.spec({n: v[t:t + 4] for n, v in toks.items()}, what="masked spec", active=np.array([0, 1, 1], bool)); t += 4
    pair.commit(np.array([2, 4, 1]), what="commit after masked spec")
    pair.flush("flush")
    for step in range(cap + 2):
        pair.decode(synth.token(toks, t), what=f"decode after flush {step}"); t += 1
