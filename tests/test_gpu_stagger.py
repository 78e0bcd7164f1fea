"""GPU parity of staggered flush phases and of the full-buffer decode at capacity 1.

Staggered flushes (REPLAY_FLAG_STAGGER_FLUSH): after a load, sequence b's first
window ends after 1 + (b mod cap) tokens, so lockstep decoding folds about
batch/cap sequences per step.  The pages leave the flush schedule open (values
do not depend on it, [TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM nasil
calisir?": outputs equal ordinary decoding up to rounding); the oracle applies
the same window rule, and bookkeeping must match bit for bit.
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


def _toks(kind, seed, T, B, H, G, C, R, io="f32"):
    if kind == "mamba2":
        return synth.mamba2_tokens(seed, T, B, H, G, C, R, dtype=io)
    return synth.gdn_tokens(seed, T, B, H, G, R, C, dtype=io)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_staggered_windows_against_oracle(kind):
    from harness import Pair
    from hybrid_decode_replay_amd import binding as b
    B, H, C, R, cap = 5, 2, 32, 32, 4
    G = 1 if kind == "mamba2" else H
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap, io=b.F32, seed=97,
                S0=synth.checkpoint(97, (B, H, C, R)), flags=b.FLAG_STAGGER_FLUSH)
    toks = _toks(kind, 97, 200, B, H, G, C, R)
    t = 0
    for _ in range(9):                       # lockstep decoding: staggered folds
        pair.decode(synth.token(toks, t), what=f"decode {t}"); t += 1
    rng = np.random.default_rng(97)
    for rnd in range(16):
        op = int(rng.integers(0, 5))
        if op <= 1:
            pair.decode(synth.token(toks, t), what=f"round {rnd} decode"); t += 1
        elif op == 4:
            pair.flush(what=f"round {rnd} flush")
        else:
            k = int(rng.integers(1, cap + 1))
            pair.spec({n: v[t:t + k] for n, v in toks.items()}, what=f"round {rnd} spec k={k}"); t += k
            if op == 2:
                pair.rollback()
            else:
                pair.commit(rng.integers(0, k + 1, size=B))
    # reload restores the stagger
    pair.st.load_checkpoint(torch.from_numpy(synth.checkpoint(98, (B, H, C, R))).cuda())
    pair.orc.load(synth.checkpoint(98, (B, H, C, R)))
    for _ in range(6):
        pair.decode(synth.token(toks, t), what=f"after reload {t}"); t += 1


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_full_buffer_decode_at_capacity_one(kind):
    from harness import Pair
    from hybrid_decode_replay_amd import binding as b
    B, H, C, R = 3, 2, 16, 32
    G = 1 if kind == "mamba2" else H
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=1, io=b.F32, seed=99,
                S0=synth.checkpoint(99, (B, H, C, R)))
    toks = _toks(kind, 99, 20, B, H, G, C, R)
    pair.spec({n: v[0:1] for n, v in toks.items()})
    pair.commit([1, 0, 1])                   # rows 0 and 2 now hold a full buffer
    pair.decode(synth.token(toks, 1), what="decode on a full buffer (two folds)")
    for t in range(2, 8):
        pair.decode(synth.token(toks, t))


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_staggered_folds_refresh_the_read_copy(kind):
    """With an FP8 read copy, after every staggered step the copy is the quantization of
    the GPU's own checkpoint (bit-exact), and the checkpoints are bitwise those of the run
    without a copy: the copy is refreshed by exactly the rows that fold.  (Outputs after a
    fold are not compared with the oracle here: both sides round their own fold results
    to FP8, and values on a code boundary may land one code apart.)"""
    from oracle import replay_oracle as ro
    from hybrid_decode_replay_amd import binding as b
    B, H, C, R, cap = 5, 2, 32, 32, 4
    G = 1 if kind == "mamba2" else H
    kk = b.MAMBA2 if kind == "mamba2" else b.GDN
    S0 = torch.from_numpy(synth.checkpoint(96, (B, H, C, R))).cuda()
    states = {}
    for name, rc in (("plain", b.NONE), ("copy", b.FP8_E4M3)):
        st = b.ReplayState(b.make_config(kk, B, H, G, C, R, cap, b.F32, read_copy=rc, flags=b.FLAG_STAGGER_FLUSH))
        st.load_checkpoint(S0)
        states[name] = st
    toks = _toks(kind, 96, 12, B, H, G, C, R)
    params = {}
    if kind == "mamba2":
        A, D = synth.mamba2_params(96, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
    for t in range(12):
        tok = {k: torch.from_numpy(v[t]).cuda() for k, v in toks.items()}
        for st in states.values():
            st.decode(tok, params)
        ck = states["copy"].read_checkpoint()
        assert torch.equal(ck, states["plain"].read_checkpoint()), f"step {t}"
        codes, _ = states["copy"].read_copy()
        torch.cuda.synchronize()
        ck64 = ck.cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(codes.cpu().numpy(), ro.e4m3_encode(ck64).reshape(ck64.shape))
