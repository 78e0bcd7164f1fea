"""GPU parity of the FP8 (E4M3) recurrence checkpoint (Mamba-2 and Gated DeltaNet).

The checkpoint is stored as OCP E4M3 codes in the read copy's strip layout: a
fold decodes it, folds in fp32 and rounds the result to the nearest E4M3 value
(ties to even, saturating) at once; non-flush steps read one byte per element,
or an MXFP4 copy of the FP8 values ([TR] "NVIDIA ve Dao AI Lab ...", section
"Kuantizasyon hatasinin sinirlandirilmasi", pairs low-precision reads with an
FP8 recurrence).  The oracle rounds its fp64 state the same way at load and at
every flush.  Checked here:
  * load / read of the checkpoint: bit-exact round trip of every finite code;
  * the first window (both sides read the same FP8 values): outputs within the
    io dtype's tolerance;
  * the first fold: every code equal to the oracle's, except where the oracle's
    exact fold result lies within fp32 rounding of an E4M3 midpoint -- there the
    two codes are neighbours;
  * longer runs with spec, commit, rollback and flush: checkpoints within the
    element-wise bound derived in tests/harness.py (Fp8Bound) and rarely
    different at all, outputs within the io tolerance plus the read-out of the
    measured checkpoint difference; bookkeeping bit-exact;
  * an MXFP4 copy is the quantization of exactly the stored FP8 values;
  * the conventional baseline with an FP8 state.
Bit-exact agreement on inputs that make all arithmetic exact is in
test_gpu_exact_dyadic.py.
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


def _kind(name):
    b = rb()
    return b.MAMBA2 if name == "mamba2" else b.GDN


def _tokens(kind, seed, T, B, H, G, C, R, io="f32"):
    if kind == "mamba2":
        return synth.mamba2_tokens(seed, T, B, H, G, C, R, dtype=io)
    return synth.gdn_tokens(seed, T, B, H, G, R, C, dtype=io)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("C,R", [(16, 16), (48, 32), (64, 128), (32, 256)])
def test_checkpoint_round_trip_bit_exact(kind, C, R):
    b = rb()
    B, H = 3, 2
    st = b.ReplayState(b.make_config(_kind(kind), B, H, H, C, R, 16, b.F32, ckpt_dtype=b.FP8_E4M3))
    g = torch.Generator().manual_seed(C * 1000 + R)
    codes = torch.randint(0, 256, (B, H, C, R), generator=g, dtype=torch.int32)
    codes[(codes & 0x7F) == 0x7F] = 0x7E                 # NaN codes -> largest finite
    S = codes.to(torch.uint8).view(torch.float8_e4m3fn).cuda()
    st.load_checkpoint(S)
    back = st.read_checkpoint()
    torch.cuda.synchronize()
    assert back.dtype == torch.float8_e4m3fn
    assert torch.equal(back.view(torch.uint8), S.view(torch.uint8))
    assert st.layout().ckpt_bytes == B * H * C * R


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("B,H,G,C,R,cap,io,std", [
    (3, 4, 2, 64, 128, 16, "f32", 0.1),
    (2, 2, 1, 32, 16, 5, "bf16", 1.0),     # one-block strips
    (5, 3, 3, 48, 64, 7, "f32", 1.0),      # ragged windows, three waves
    (2, 2, 2, 128, 256, 4, "bf16", 0.1),
])
def test_decode_windows(kind, B, H, G, C, R, cap, io, std):
    from harness import Pair
    b = rb()
    if kind == "gdn":
        G = H
    S0 = synth.checkpoint(12, (B, H, C, R), std=std)
    pair = Pair(_kind(kind), B, H, G, C, R, cap=cap, io=b.BF16 if io == "bf16" else b.F32, seed=12, S0=S0,
                ckpt=b.FP8_E4M3)
    T = 3 * cap + 2
    toks = _tokens(kind, 12, T, B, H, G, C, R, io)
    print(f"[fp8 decode] {kind} B={B} H={H} C={C} R={R} cap={cap} io={io}", flush=True)
    for t in range(T):
        pair.decode(synth.token(toks, t), what=f"step {t}")
    print("max errors", pair.max_err, "flip fraction", pair.max_flip_frac)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_first_fold_codes(kind):
    """At the first fold the two sides round fold results that differ by fp32 rounding
    only.  A code may differ only where the oracle's exact fold result (an fp32-checkpoint
    oracle session from the same FP8 start, which has not rounded yet) lies within that
    distance of the midpoint between the two codes' values."""
    from oracle import replay_oracle as ro
    b = rb()
    B, H, C, R, cap = 8, 4, 64, 128, 6
    G = H
    S0 = synth.checkpoint(13, (B, H, C, R), std=1.0)
    S0 = ro.e4m3_decode(ro.e4m3_encode(S0)).reshape(S0.shape).astype(np.float32)
    cfg = b.make_config(_kind(kind), B, H, G, C, R, cap, b.F32, ckpt_dtype=b.FP8_E4M3)
    st = b.ReplayState(cfg)
    st.load_checkpoint(torch.from_numpy(S0).cuda())
    toks = _tokens(kind, 13, cap, B, H, G, C, R)
    params = {}
    if kind == "mamba2":
        A, D = synth.mamba2_params(13, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        exact = ro.Mamba2Session(A, D, S0, cap=cap)
    else:
        exact = ro.GDNSession(S0, cap=cap)
    for t in range(cap):
        tok = synth.token(toks, t)
        st.decode({k: torch.from_numpy(v).cuda() for k, v in tok.items()}, params)
        exact.decode(tok)
    codes = st.read_checkpoint().view(torch.uint8).cpu().numpy()
    got = ro.e4m3_decode(codes).reshape(codes.shape)
    x = exact.ckpt                                          # unrounded fold (fp64)
    want = ro.e4m3_decode(ro.e4m3_encode(x)).reshape(x.shape)
    diff = got != want
    print(f"[fp8 first fold] {kind}: {int(diff.sum())} of {diff.size} codes differ", flush=True)
    if diff.any():
        from harness import e4m3_grid_index
        assert np.all(np.abs(e4m3_grid_index(got[diff]) - e4m3_grid_index(want[diff])) == 1)
        mid = 0.5 * (got[diff] + want[diff])
        scale = np.max(np.abs(x), axis=(2, 3), keepdims=True)
        tol = 1e-5 * np.broadcast_to(scale, x.shape)[diff]
        assert np.all(np.abs(x[diff] - mid) <= tol), "a differing code away from a rounding midpoint"
    assert diff.mean() <= 1e-3


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_spec_commit_rollback_and_flush(kind):
    from harness import Pair
    b = rb()
    B, H, C, R, cap = 4, 2, 32, 64, 8
    pair = Pair(_kind(kind), B, H, H, C, R, cap=cap, io=b.F32, seed=22,
                S0=synth.checkpoint(22, (B, H, C, R), std=0.5), ckpt=b.FP8_E4M3)
    toks = _tokens(kind, 22, 40, B, H, H, C, R)
    for t in range(3):
        pair.decode(synth.token(toks, t))
    pair.spec({n: v[3:7] for n, v in toks.items()}, what="spec 4")
    pair.commit([4, 2, 0, 1])
    pair.spec({n: v[7:13] for n, v in toks.items()}, what="spec 6 with pre-flush rows")
    pair.rollback()
    pair.decode(synth.token(toks, 13))
    pair.flush()
    pair.spec({n: v[14:22] for n, v in toks.items()}, what="spec 8 from an empty buffer")
    pair.commit([8, 8, 3, 0])
    for t in range(22, 30):
        pair.decode(synth.token(toks, t))
    print("max errors", pair.max_err, "flip fraction", pair.max_flip_frac)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_mxfp4_copy_of_fp8_checkpoint(kind):
    """Non-flush steps read an MXFP4 copy of the FP8 checkpoint; after every fold the copy
    is the MXFP4 quantization of exactly the stored FP8 values."""
    from harness import Pair
    from oracle import replay_oracle as ro
    b = rb()
    B, H, C, R, cap = 2, 2, 32, 64, 4
    pair = Pair(_kind(kind), B, H, H, C, R, cap=cap, io=b.F32, seed=32,
                S0=synth.checkpoint(32, (B, H, C, R), std=0.5), ckpt=b.FP8_E4M3, read_copy=b.MXFP4)
    toks = _tokens(kind, 32, 3 * cap, B, H, H, C, R)
    for t in range(3 * cap):
        pair.decode(synth.token(toks, t), what=f"step {t}")
        ck = pair.st.read_checkpoint()
        codes, scales = pair.st.read_copy()
        torch.cuda.synchronize()
        ck64 = ck.float().cpu().numpy().astype(np.float64)
        wc, ws = ro.mxfp4_quantize(ck64)
        np.testing.assert_array_equal(codes.cpu().numpy(), wc)
        np.testing.assert_array_equal(scales.cpu().numpy(), ws)


def test_fp8_flags_rejected():
    b = rb()
    bad = [dict(read_copy=b.FP8_E4M3), dict(read_copy=b.MXFP4, flags=b.FLAG_QUANTIZED_CKPT),
           dict(flags=b.FLAG_VALU_FOLD)]
    for kw in bad:
        cfg = b.make_config(b.MAMBA2, 2, 2, 1, 32, 32, 8, b.F32, ckpt_dtype=b.FP8_E4M3, **kw)
        assert b.config_check(cfg) == b.ERR_UNSUPPORTED, kw
    cfg = b.make_config(b.GDN, 2, 2, 2, 32, 32, 8, b.F32, ckpt_dtype=b.FP8_E4M3, read_copy=b.MXFP4)
    assert b.config_check(cfg) == b.OK


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
@pytest.mark.parametrize("C,R", [(32, 64), (160, 64), (160, 128)])   # 1 row pass; 3-5 with a ragged last
def test_conventional_fp8_state(kind, C, R):
    """Conventional decoding on an FP8 state vs the oracle's replay session with a one-entry
    buffer (every token folds: the fp64 state is updated, rounded to E4M3 and the output read
    from the rounded values, the order the conventional kernel uses).  Both start from the
    same E4M3 values.  Every token rounds the state on both sides, so the element-wise bound
    of tests/harness.py (Fp8Bound) is advanced once per token: a difference is carried by
    the update (Mamba-2 decay <= 1 per element; GDN a product of factors of 2-norm <= 1 per
    row) and each rounding may add about one E4M3 step.  The outputs may differ by the
    read-out of the measured state difference (readout_bound) beyond 1e-4 of the vector's
    norm; at most 1e-3 of the codes may differ."""
    from harness import Fp8Bound, readout_bound
    from oracle import replay_oracle as ro
    b = rb()
    B, H, T = 3, 2, 6
    cfg = b.make_config(_kind(kind), B, H, H, C, R, 16, b.F32, ckpt_dtype=b.FP8_E4M3)
    S0 = synth.checkpoint(42, (B, H, C, R), std=0.5)
    # the conventional state in the checkpoint dtype, made by the library's own load rounding
    st = b.ReplayState(b.make_config(_kind(kind), B, H, H, C, R, 16, b.F32, ckpt_dtype=b.FP8_E4M3))
    st.load_checkpoint(torch.from_numpy(S0).cuda())
    S = st.read_checkpoint()
    torch.cuda.synchronize()
    toks = _tokens(kind, 42, T, B, H, H, C, R)
    params = {}
    if kind == "mamba2":
        A, D = synth.mamba2_params(42, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        sess = ro.Mamba2Session(A, D, S0, cap=1, ckpt_dtype="fp8")
    else:
        sess = ro.GDNSession(S0, cap=1, ckpt_dtype="fp8")
    assert np.array_equal(ro.e4m3_decode(S.view(torch.uint8).cpu().numpy()).reshape(S0.shape), sess.S)
    bound = Fp8Bound(kind, (B, H, C, R))
    for t in range(T):
        tok = synth.token(toks, t)
        y = b.conv_decode_step(cfg, S, {k: torch.from_numpy(v).cuda() for k, v in tok.items()}, params)
        yr = sess.decode(tok)
        torch.cuda.synchronize()
        bound.advance(np.ones(B, bool), sess.S)
        Sg = ro.e4m3_decode(S.view(torch.uint8).cpu().numpy()).reshape(S0.shape)
        dS, _ = bound.check(Sg, sess.S, f"token {t}")
        yg = y[0].float().cpu().numpy().astype(np.float64)
        allow = 1e-4 * np.max(np.abs(yr), axis=-1, keepdims=True) + readout_bound(kind, dS, [tok])[0]
        over = np.abs(yg - yr) > allow
        assert not over.any(), (t, int(over.sum()))
