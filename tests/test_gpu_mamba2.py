"""GPU parity of the replayed Mamba-2 decode path against the fp64 oracle (through the C ABI).

Outputs within 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs and outputs) normwise
relative error, checkpoints likewise after every operation, bookkeeping
bit-exact.  Sizes span several tiles and ragged buffer fills; the full-size
case samples sequences of the batch-256 hybrid-serving layer.
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


def _run_decode(B, H, G, P, N, cap, io, steps, seed, flags=0, zero=False, std=0.1):
    from harness import Pair
    b = rb()
    S0 = synth.checkpoint(seed, (B, H, P, N), std=std, zero=zero)
    pair = Pair(b.MAMBA2, B, H, G, P, N, cap=cap, io=io, seed=seed, S0=S0, flags=flags)
    toks = synth.mamba2_tokens(seed, steps, B, H, G, P, N, dtype="bf16" if io == b.BF16 else "f32")
    for t in range(steps):
        print(f"[mamba2 decode] B={B} H={H} G={G} P={P} N={N} cap={cap} step={t}", flush=True) if t == 0 else None
        pair.decode(synth.token(toks, t), what=f"step {t}")
    return pair


def test_config0_small_fp32_layer():
    """Mamba-2 single layer, fp32 everything: B=2, H=4, P=N=64, G=1, buffer 16, 64 steps from zero."""
    b = rb()
    pair = _run_decode(2, 4, 1, 64, 64, 16, b.F32, 64, seed=0, zero=True)
    assert pair.orc.flush_events and [e[0] for e in pair.orc.flush_events[::2]][:4] == [15, 31, 47, 63]
    print("max errors", pair.max_err)


def test_config0_valu_fold_cross_check():
    b = rb()
    _run_decode(2, 4, 1, 64, 64, 16, b.F32, 40, seed=0, zero=True, flags=b.FLAG_VALU_FOLD)


@pytest.mark.parametrize("B,H,G,P,N,cap,io", [
    (3, 4, 2, 16, 16, 1, "f32"),      # buffer of one entry: every step flushes
    (2, 2, 1, 32, 32, 5, "bf16"),
    (1, 2, 2, 128, 256, 16, "f32"),   # largest state dim
    (2, 2, 1, 256, 128, 3, "bf16"),   # largest head dim (16 waves)
    (5, 3, 3, 48, 64, 7, "f32"),      # odd wave count, ragged windows
    (4, 8, 8, 64, 128, 16, "bf16"),
])
def test_shapes_and_buffer_sizes(B, H, G, P, N, cap, io):
    b = rb()
    io = b.BF16 if io == "bf16" else b.F32
    _run_decode(B, H, G, P, N, cap, io, 2 * cap + 3, seed=7 + cap)


def test_explicit_flush_and_reload():
    from harness import Pair
    b = rb()
    B, H, G, P, N = 2, 2, 1, 32, 64
    S0 = synth.checkpoint(3, (B, H, P, N))
    pair = Pair(b.MAMBA2, B, H, G, P, N, cap=8, io=b.F32, seed=3, S0=S0)
    toks = synth.mamba2_tokens(3, 40, B, H, G, P, N)
    for t in range(5):
        pair.decode(synth.token(toks, t))
    pair.flush("flush after 5")
    pair.flush("flush of an empty buffer")
    for t in range(5, 20):
        pair.decode(synth.token(toks, t))
    # reload a checkpoint: len, pend, fc reset; decoding continues from it
    S1 = synth.checkpoint(4, (B, H, P, N))
    pair.st.load_checkpoint(torch.from_numpy(S1).cuda())
    pair.orc.load(S1)
    pair.check_state("after load")
    for t in range(20, 40):
        pair.decode(synth.token(toks, t))


def test_spec_rounds_against_oracle():
    """Draft append with output-only verification, commit of a seeded accepted prefix, rollback."""
    from harness import Pair
    b = rb()
    B, H, G, P, N, cap = 4, 2, 1, 32, 32, 8
    S0 = synth.checkpoint(5, (B, H, P, N))
    pair = Pair(b.MAMBA2, B, H, G, P, N, cap=cap, io=b.F32, seed=5, S0=S0)
    toks = synth.mamba2_tokens(5, 400, B, H, G, P, N)
    rng = np.random.default_rng(5)
    t = 0
    for rnd in range(30):
        op = rng.integers(0, 4)
        if op == 0:
            pair.decode(synth.token(toks, t), what=f"round {rnd} decode"); t += 1
            continue
        k = int(rng.integers(1, cap + 1))
        drafts = {n: v[t:t + k] for n, v in toks.items()}
        t += k
        pair.spec(drafts, what=f"round {rnd} spec k={k}")
        if op == 1:
            pair.rollback(what=f"round {rnd} rollback")
        else:
            acc = rng.integers(-1, k + 2, size=B)      # includes out-of-range counts (clamped, flagged)
            pair.commit(acc, what=f"round {rnd} commit {acc}")


def test_phase_rules_and_capacity():
    b = rb()
    cfg = b.make_config(b.MAMBA2, 2, 2, 1, 16, 16, 4, b.F32)
    st = b.ReplayState(cfg)
    A = torch.full((2,), -1.0, device="cuda")
    D = torch.ones(2, device="cuda")
    tok = {n: torch.zeros(s, device="cuda") for n, s in
           (("x", (1, 2, 2, 16)), ("Bm", (1, 2, 1, 16)), ("Cm", (1, 2, 1, 16)), ("dt", (1, 2, 2)))}
    params = {"A": A, "D": D}
    with pytest.raises(b.ReplayError) as e:
        st.spec_append(5, tok, params)
    assert e.value.status == b.ERR_CAPACITY
    with pytest.raises(b.ReplayError) as e:
        st.rollback()
    assert e.value.status == b.ERR_STATE
    st.spec_append(1, tok, params)
    assert st.phase() == 1
    for fn in (lambda: st.decode(tok, params), lambda: st.flush(params), lambda: st.spec_append(1, tok, params),
               lambda: st.load_checkpoint(torch.zeros(st.ckpt_shape, device="cuda"))):
        with pytest.raises(b.ReplayError) as e:
            fn()
        assert e.value.status == b.ERR_STATE
    st.rollback()
    assert st.phase() == 0
    with pytest.raises(b.ReplayError) as e:
        st.decode({**tok, "x": None}, params)
    assert e.value.status == b.ERR_ARG


def test_determinism_bitwise():
    b = rb()
    outs = []
    for _ in range(2):
        cfg = b.make_config(b.MAMBA2, 3, 4, 2, 64, 128, 16, b.BF16)
        st = b.ReplayState(cfg)
        S0 = synth.checkpoint(9, (3, 4, 64, 128))
        st.load_checkpoint(torch.from_numpy(S0).cuda())
        A, D = synth.mamba2_params(9, 4)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        toks = synth.mamba2_tokens(9, 35, 3, 4, 2, 64, 128, dtype="bf16")
        ys = []
        for t in range(35):
            tok = {k: torch.from_numpy(v[t]).cuda().to(torch.bfloat16) for k, v in toks.items()}
            ys.append(st.decode(tok, params).clone())
        outs.append((torch.stack(ys), st.read_checkpoint()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


def _conv_run(B, H, G, P, N, io, steps, seed):
    from oracle import replay_oracle as ro
    b = rb()
    cfg = b.make_config(b.MAMBA2, B, H, G, P, N, 16, io)
    iot = torch.bfloat16 if io == b.BF16 else torch.float32
    S0 = synth.checkpoint(seed, (B, H, P, N))
    A, D = synth.mamba2_params(seed, H)
    params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
    toks = synth.mamba2_tokens(seed, steps, B, H, G, P, N, dtype="bf16" if io == b.BF16 else "f32")
    S = torch.from_numpy(S0).cuda()
    So = S0.astype(np.float64)
    tol = 2e-2 if io == b.BF16 else 1e-4
    for t in range(steps):
        tok = synth.token(toks, t)
        y = b.conv_decode_step(cfg, S, {k: torch.from_numpy(v).cuda().to(iot) for k, v in tok.items()}, params)
        yo = ro.mamba2_token(So, tok["x"], tok["Bm"], tok["Cm"], tok["dt"], A, D)
        assert ro.normwise_error(y[0].float().cpu().numpy(), yo) <= tol
    torch.cuda.synchronize()
    assert ro.normwise_error(S.cpu().numpy(), So, axis=(2, 3)) <= 1e-4


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conventional_decode_baseline(io):
    b = rb()
    _conv_run(3, 4, 2, 64, 128, b.BF16 if io == "bf16" else b.F32, 20, seed=11)
    _conv_run(2, 3, 1, 48, 16, b.F32, 5, seed=12)


def test_conventional_spec_snapshots_and_restore():
    from oracle import replay_oracle as ro
    b = rb()
    B, H, G, P, N, k = 3, 2, 1, 32, 64, 4
    cfg = b.make_config(b.MAMBA2, B, H, G, P, N, 16, b.F32)
    S0 = synth.checkpoint(13, (B, H, P, N))
    A, D = synth.mamba2_params(13, H)
    params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
    toks = synth.mamba2_tokens(13, k, B, H, G, P, N)
    S = torch.from_numpy(S0).cuda()
    snaps = torch.empty((k, B, H, P, N), device="cuda")
    y = b.conv_spec_step(cfg, S, snaps, k, {n: torch.from_numpy(v).cuda() for n, v in toks.items()}, params)
    So = S0.astype(np.float64)
    states = []
    for j in range(k):
        yo = ro.mamba2_token(So, toks["x"][j], toks["Bm"][j], toks["Cm"][j], toks["dt"][j], A, D)
        assert ro.normwise_error(y[j].cpu().numpy(), yo) <= 1e-4
        states.append(So.copy())
        assert ro.normwise_error(snaps[j].cpu().numpy(), So, axis=(2, 3)) <= 1e-4
    assert torch.equal(S.cpu(), torch.from_numpy(S0))            # read-only during the drafts
    acc = torch.tensor([0, 2, 4], dtype=torch.int32, device="cuda")
    b.conv_spec_restore(cfg, S, snaps, k, acc)
    torch.cuda.synchronize()
    Sh = S.cpu().numpy()
    np.testing.assert_array_equal(Sh[0], S0[0])
    np.testing.assert_array_equal(Sh[1], snaps[1, 1].cpu().numpy())
    np.testing.assert_array_equal(Sh[2], snaps[3, 2].cpu().numpy())


def test_full_size_layer_sampled_sequences():
    """Batch-256 hybrid-serving Mamba-2 layer (H=128, P=64, N=128, G=8, bf16 inputs, fp32
    checkpoint ~ N(0, 0.1)), 48 decode steps (three flush windows); the oracle replays
    three sampled sequences (all 128 heads) from copies of exactly the device-drawn inputs."""
    from oracle import replay_oracle as ro
    b = rb()
    B, H, G, P, N, T = 256, 128, 8, 64, 128, 48
    cfg = b.make_config(b.MAMBA2, B, H, G, P, N, 16, b.BF16)
    st = b.ReplayState(cfg)
    S0 = synth.checkpoint_device(1, (B, H, P, N), "cuda")
    st.load_checkpoint(S0)
    A, D = synth.mamba2_params(1, H)
    params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
    toks = synth.mamba2_tokens_device(1, T, B, H, G, P, N, "cuda")
    ys = torch.empty((T, B, H, P), dtype=torch.bfloat16, device="cuda")
    print("[full-size mamba2] launching", flush=True)
    for t in range(T):
        st.decode({k: v[t:t + 1] for k, v in toks.items()}, params, y=ys[t:t + 1])
    ck = st.read_checkpoint()
    L, Pd, F, E = st.read_book()
    torch.cuda.synchronize()
    assert torch.all(L == 0) and torch.all(F == 3) and torch.all(Pd == 0) and int(E[0]) == 0
    sample = [0, 131, 255]
    sess = ro.Mamba2Session(A, D, S0[sample].cpu().numpy())
    host = {k: v[:, sample].float().cpu().numpy() for k, v in toks.items()}
    yg = ys[:, sample].float().cpu().numpy()
    for t in range(T):
        yo = sess.decode(synth.token(host, t))
        err = ro.normwise_error(yg[t], yo)
        assert err <= 2e-2, (t, err)
    err_ck = ro.normwise_error(ck[sample].cpu().numpy(), sess.ckpt, axis=(2, 3))
    assert err_ck <= 1e-4, err_ck
