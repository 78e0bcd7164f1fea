"""Bit-exact parity on inputs whose every result is exact in fp32.

Test inputs are multiples of 1/4 with a few significant bits, Mamba-2 runs with
A = 0 (every decay factor is exactly 1) and Gated DeltaNet with alpha = 1,
beta = 1/2 and one-hot keys (a token halves one column of the state and adds
v/2 to it).  Every sum and product the method forms -- the fold, the replayed
buffer terms, the readout -- then needs fewer than 24 significant bits, so the
GPU's fp32 arithmetic and the oracle's fp64 arithmetic reach the same numbers in
any order.  What is left to compare is the rounding that the method itself
prescribes: the checkpoint dtype's rounding at a fold (binary16 or E4M3, ties
to even), and the read copy's quantization (E4M3, or MXFP4 with its E8M0
scales).  Fold results here often sit exactly on a rounding midpoint, so the
ties-to-even rule is exercised too.  Outputs, checkpoints and bookkeeping must
be identical, through decode windows, spec append, commit, rollback and flush.
The inputs are checked on the host to be exact (every oracle output and state
equals its fp32 rounding) before the GPU runs.
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
    from hybrid_decode_replay_amd import binding  # noqa: F401  (fails loudly if not built)
    yield


def rb():
    from hybrid_decode_replay_amd import binding
    return binding


def _quarters(rng, shape, m):
    """Multiples of 1/4 in [-m/4, m/4]."""
    return rng.integers(-m, m + 1, shape).astype(np.float64) / 4.0


def _state(rng, shape):
    """E4M3 values with magnitudes in [1/8, 4) (exponents -3..1, any 3-bit mantissa), a
    tenth of them zero: on every checkpoint dtype's grid, with steps no finer than 2^-6."""
    e = rng.integers(-3, 2, shape)
    m = rng.integers(0, 8, shape)
    s = rng.choice([-1.0, 1.0], shape)
    v = s * (1.0 + m / 8.0) * np.exp2(e)
    v[rng.random(shape) < 0.1] = 0.0
    return v.astype(np.float32)


def _inputs(kind, seed, T, B, H, G, C, R):
    rng = np.random.default_rng([seed, 909])
    if kind == "mamba2":
        return {"x": _quarters(rng, (T, B, H, C), 4).astype(np.float32),
                "Bm": _quarters(rng, (T, B, G, R), 4).astype(np.float32),
                "Cm": _quarters(rng, (T, B, G, R), 2).astype(np.float32),
                "dt": rng.choice([0.25, 0.5, 1.0], (T, B, H)).astype(np.float32)}
    k = np.zeros((T, B, G, R), np.float32)
    idx = rng.integers(0, R, (T, B, G))
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    return {"q": _quarters(rng, (T, B, G, R), 2).astype(np.float32), "k": k,
            "v": _quarters(rng, (T, B, H, C), 4).astype(np.float32),
            "alpha": np.ones((T, B, H), np.float32), "beta": np.full((T, B, H), 0.5, np.float32)}


def _script(kind, pair, toks):
    """decode x5, spec 3 + partial commit, decode x2, spec 4 + rollback, flush, decode x3."""
    cut = lambda a, b: {n: v[a:b] for n, v in toks.items()}  # noqa: E731
    for t in range(5):
        pair.decode(synth.token(toks, t), what=f"decode {t}")
    pair.spec(cut(5, 8), what="spec 3")
    pair.commit([3, 1, 0, 2], what="commit")
    for t in range(8, 10):
        pair.decode(synth.token(toks, t), what=f"decode {t}")
    pair.spec(cut(10, 14), what="spec 4")
    pair.rollback()
    pair.flush()
    for t in range(14, 17):
        pair.decode(synth.token(toks, t), what=f"decode {t}")


def _host_exact(kind, S0, toks, H):
    """The script on the fp64 oracle (fp32 checkpoint, no copy): every output and every
    state it passes through must equal its fp32 rounding, or the inputs are not exact."""
    from oracle import replay_oracle as ro

    S = np.array(S0, np.float64)
    if kind == "mamba2":
        A, D = np.zeros(H), np.ones(H)
        for t in range(17):
            tok = synth.token(toks, t)
            y = ro.mamba2_token(S, tok["x"], tok["Bm"], tok["Cm"], tok["dt"], A, D)
            assert np.array_equal(y, y.astype(np.float32)) and np.array_equal(S, S.astype(np.float32))
    else:
        for t in range(17):
            tok = synth.token(toks, t)
            o = ro.gdn_token(S, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"])
            assert np.array_equal(o, o.astype(np.float32)) and np.array_equal(S, S.astype(np.float32))


CASES = [("f32", "none"), ("f32", "fp8"), ("f32", "mxfp4"), ("f16", "none"), ("f16", "fp8"),
         ("f16", "mxfp4"), ("fp8", "none"), ("fp8", "mxfp4")]


@pytest.mark.parametrize("ckpt,copy", CASES)
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_bit_exact_on_dyadic_inputs(kind, ckpt, copy):
    from harness import Pair
    b = rb()
    B, H, G, C, R, cap = 4, 4, 2, 64, 128, 4
    if kind == "gdn":
        G = H
    rng = np.random.default_rng([H, C, R, 808])
    S0 = _state(rng, (B, H, C, R))
    toks = _inputs(kind, 17, 17, B, H, G, C, R)
    _host_exact(kind, S0, toks, H)
    ck = {"f32": b.F32, "f16": b.F16, "fp8": b.FP8_E4M3}[ckpt]
    rc = {"none": b.NONE, "fp8": b.FP8_E4M3, "mxfp4": b.MXFP4}[copy]
    print(f"[exact] {kind} ckpt={ckpt} copy={copy}", flush=True)
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap, io=b.F32, seed=17, S0=S0,
                ckpt=ck, read_copy=rc, tol=0.0)
    if kind == "mamba2":        # A = 0 (decays of exactly 1), D = 1
        pair.params = {"A": torch.zeros(H, device="cuda"), "D": torch.ones(H, device="cuda")}
        pair.orc.A = np.zeros(H)
        pair.orc.D = np.ones(H)
    _script(kind, pair, toks)
    assert pair.max_err["y"] == 0.0 and pair.max_err["ckpt"] == 0.0
    if rc != b.NONE:
        from oracle import replay_oracle as ro
        codes, scales = pair.st.read_copy()
        torch.cuda.synchronize()
        ref = pair.orc.ckpt.astype(np.float32).astype(np.float64)
        if rc == b.FP8_E4M3:
            np.testing.assert_array_equal(codes.cpu().numpy(), ro.e4m3_encode(ref).reshape(ref.shape))
        else:
            wc, ws = ro.mxfp4_quantize(ref)
            np.testing.assert_array_equal(codes.cpu().numpy(), wc)
            np.testing.assert_array_equal(scales.cpu().numpy(), ws)


BF16_CASES = [("f32", "none"), ("f32", "fp8"), ("f32", "mxfp4"), ("f16", "none"), ("fp8", "none"),
              ("fp8", "mxfp4")]


@pytest.mark.parametrize("ckpt,copy", BF16_CASES)
@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_bit_exact_fold_with_bf16_io(kind, ckpt, copy):
    """The same dyadic script with bf16 io, where the folds take the 16x16x32 bf16 product
    (the four-head Mamba-2 kernels, every GDN kernel).  This pins those products' operand
    layouts and the rounding after them bit for bit: checkpoints and bookkeeping must match
    exactly.  Mamba-2's dt takes 8-bit values in [1/2, 2), so a fold weight dt x carries up
    to 10 bits and its second bf16 term is not zero (with A = 0 nothing needs the third,
    which the other parity tests hold, fp32 checkpoints to 1e-4).  Outputs are written in
    bf16, so they are held to its rounding (relative 2^-9 per element).  Mamba-2 runs with
    one B/C group, so that its four-head kernels fold."""
    from harness import Pair
    b = rb()
    B, H, G, C, R, cap = 4, 4, 1, 64, 128, 4
    if kind == "gdn":
        G = H
    rng = np.random.default_rng([H, C, R, 818])
    S0 = _state(rng, (B, H, C, R))
    toks = _inputs(kind, 19, 17, B, H, G, C, R)
    if kind == "mamba2":
        toks["dt"] = (np.random.default_rng([19, 707]).integers(64, 256, toks["dt"].shape) / 128.0).astype(np.float32)
    for n, v in toks.items():
        if n not in ("alpha", "beta"):
            assert np.array_equal(torch.from_numpy(v).to(torch.bfloat16).float().numpy(), v), n
    _host_exact(kind, S0, toks, H)
    ck = {"f32": b.F32, "f16": b.F16, "fp8": b.FP8_E4M3}[ckpt]
    rc = {"none": b.NONE, "fp8": b.FP8_E4M3, "mxfp4": b.MXFP4}[copy]
    print(f"[exact bf16] {kind} ckpt={ckpt} copy={copy}", flush=True)
    pair = Pair(b.MAMBA2 if kind == "mamba2" else b.GDN, B, H, G, C, R, cap=cap, io=b.BF16, seed=19, S0=S0,
                ckpt=ck, read_copy=rc, tol=0.0)
    pair.tol = 2.0 ** -8          # outputs only; checkpoints stay bit-exact (ckpt_tol = 0)
    if kind == "mamba2":
        pair.params = {"A": torch.zeros(H, device="cuda"), "D": torch.ones(H, device="cuda")}
        pair.orc.A = np.zeros(H)
        pair.orc.D = np.ones(H)
    _script(kind, pair, toks)
    assert pair.max_err["ckpt"] == 0.0
    assert pair.max_err["y"] <= 2.0 ** -8
