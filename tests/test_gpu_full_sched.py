"""Full-size parity of the flush schedules and of the layer stack the benchmark times.

* Staggered flush phases on the batch-256 Mamba-2 and GDN layers (buffer 16): after
  the load sequence b's first window holds 1 + (b mod 16) entries, so every step
  folds about 1/16 of the sequences.  40 steps; sampled sequences from every part of
  the stagger cycle (first windows of 1, 8, 16, ...) are replayed by the oracle with
  their own batch indices.
* The hybrid stack the benchmark times: Mamba-2, GDN, Mamba-2, GDN at batch 256
  (bf16 io, fp32 checkpoints), one bookkeeping set, lockstep and staggered; 40 model
  steps, three sampled sequences per layer against the oracle's StackSession.
The pages leave the flush schedule open and fix that values do not depend on it
([TR] "NVIDIA ve Dao AI Lab ...", section "ReplaySSM nasil calisir?").
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from hybrid_decode_replay_amd import synth  # noqa: E402

SHAPES = {"mamba2": (128, 8, 64, 128), "gdn": (32, 32, 128, 128)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_decode_replay_amd import binding  # noqa: F401  (fails loudly if not built)
    yield


def _layer(kind, B, T, seed, flags):
    from hybrid_decode_replay_amd import binding as b
    H, G, C, R = SHAPES[kind]
    if kind == "mamba2":
        A, D = synth.mamba2_params(seed, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        toks = synth.mamba2_tokens_device(seed, T, B, H, G, C, R, "cuda")
        cfg = b.make_config(b.MAMBA2, B, H, G, C, R, 16, b.BF16, flags=flags)
    else:
        A = D = None
        params = None
        toks = synth.gdn_tokens_device(seed, T, B, H, G, R, C, "cuda")
        cfg = b.make_config(b.GDN, B, H, G, C, R, 16, b.BF16, flags=flags)
    S0 = synth.checkpoint_device(seed, (B, H, C, R), "cuda")
    return cfg, params, toks, S0, (A, D)


def _session(kind, AD, S0s, sample, stagger):
    from oracle import replay_oracle as ro
    if kind == "mamba2":
        return ro.Mamba2Session(AD[0], AD[1], S0s, stagger=stagger, seq_ids=sample)
    return ro.GDNSession(S0s, stagger=stagger, seq_ids=sample)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_full_size_staggered_flushes(kind):
    from hybrid_decode_replay_amd import binding as b
    from oracle import replay_oracle as ro
    B, T = 256, 40
    cfg, params, toks, S0, AD = _layer(kind, B, T, 21, b.FLAG_STAGGER_FLUSH)
    st = b.ReplayState(cfg)
    st.load_checkpoint(S0)
    H, G, C, R = SHAPES[kind]
    ys = torch.empty((T, B, H, C), dtype=torch.bfloat16, device="cuda")
    print(f"[full-size stagger {kind}] launching", flush=True)
    for t in range(T):
        st.decode({k: v[t:t + 1] for k, v in toks.items()}, params, y=ys[t:t + 1])
    ck = st.read_checkpoint()
    L, Pd, F, E = st.read_book()
    torch.cuda.synchronize()
    Lh, Fh = L.cpu().numpy(), F.cpu().numpy()
    # the schedule itself, for every sequence: first window 1 + (b mod 16), then 16
    first = 1 + np.arange(B) % 16
    want_fc = np.where(T >= first, 1 + (T - first) // 16, 0)
    want_len = np.where(T >= first, (T - first) % 16, T)
    assert np.array_equal(Fh, want_fc) and np.array_equal(Lh, want_len)
    assert int(E[0]) == 0 and torch.all(Pd == 0)
    sample = [0, 7, 15, 130, 255]
    sess = _session(kind, AD, S0[sample].cpu().numpy(), sample, True)
    host = {k: v[:, sample].float().cpu().numpy() for k, v in toks.items()}
    yg = ys[:, sample].float().cpu().numpy()
    for t in range(T):
        err = ro.normwise_error(yg[t], sess.decode(synth.token(host, t)))
        assert err <= 2e-2, (t, err)
    assert list(Lh[sample]) == list(sess.len) and list(Fh[sample]) == list(sess.fc)
    err_ck = ro.normwise_error(ck[sample].cpu().numpy(), sess.ckpt, axis=(2, 3))
    assert err_ck <= 1e-4, err_ck


@pytest.mark.parametrize("stagger", [False, True])
def test_full_size_hybrid_stack(stagger):
    from hybrid_decode_replay_amd import binding as b
    from oracle import replay_oracle as ro
    B, T = 256, 40
    kinds = ("mamba2", "gdn", "mamba2", "gdn")
    flags = b.FLAG_STAGGER_FLUSH if stagger else 0
    layers = [_layer(kind, B, T, 40 + i, flags) for i, kind in enumerate(kinds)]
    states = [b.ReplayState(cfg) for cfg, *_ in layers]
    stk = b.ReplayStack(states)
    stk.load([S0 for _, _, _, S0, _ in layers])
    ys = [torch.empty((T, B, SHAPES[k][0], SHAPES[k][2]), dtype=torch.bfloat16, device="cuda") for k in kinds]
    print(f"[full-size stack, stagger={stagger}] launching", flush=True)
    for t in range(T):
        for l, (cfg, params, toks, S0, AD) in enumerate(layers):
            stk.decode_layer(l, {k: v[t:t + 1] for k, v in toks.items()}, params, y=ys[l][t:t + 1])
    cks = [st.read_checkpoint() for st in states]
    book = stk.read_book()
    torch.cuda.synchronize()
    sample = [1, 128, 254]
    sessions = [_session(kind, AD, S0[sample].cpu().numpy(), sample, stagger)
                for kind, (cfg, params, toks, S0, AD) in zip(kinds, layers)]
    so = ro.StackSession(sessions)
    hosts = [{k: v[:, sample].float().cpu().numpy() for k, v in toks.items()} for _, _, toks, _, _ in layers]
    ygs = [y[:, sample].float().cpu().numpy() for y in ys]
    for t in range(T):
        for l in range(len(kinds)):
            err = ro.normwise_error(ygs[l][t], so.decode_layer(l, synth.token(hosts[l], t)))
            assert err <= 2e-2, (t, l, err)
    Lh, Pdh, Fh, E = (x.cpu().numpy() for x in book)
    oL, oP, oF = so.trace()
    assert list(Lh[sample]) == list(oL) and list(Fh[sample]) == list(oF) and not Pdh.any() and int(E[0]) == 0
    for l, s in enumerate(sessions):
        err_ck = ro.normwise_error(cks[l][sample].cpu().numpy(), s.ckpt, axis=(2, 3))
        assert err_ck <= 1e-4, (l, err_ck)
