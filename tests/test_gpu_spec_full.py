"""GPU parity of speculative rounds at the full batch-512 shapes, in the launch
configuration the benchmark times (k = 4 drafts per round, one spec-append launch
over all 512 sequences, then one commit).

Each round appends 4 draft-token inputs without verification, evaluates their
outputs from one checkpoint read, and commits the accepted prefix by advancing the
buffer pointer ([TR] "NVIDIA ve Dao AI Lab ...", section "Durum trafigini azaltma ve
rollback'in basitlestirilmesi").  Accepted counts are min(Geometric(0.35) - 1, 4),
seeded; over 10 rounds the committed prefixes fill the 16-entry buffer, so forced
flushes of the committed prefix happen mid-run.  The oracle replays three sampled
sequences from copies of exactly the device-drawn inputs: every draft output within
the bf16 tolerance, the final checkpoint within 1e-4, len and fc bit-exact; for the
whole batch, nothing pending, no error bit and 0 <= len <= 16.
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


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_full_size_spec_rounds_sampled_sequences(kind):
    from hybrid_decode_replay_amd import binding as b
    from oracle import replay_oracle as ro
    B, K, ROUNDS = 512, 4, 10
    T = K * ROUNDS
    if kind == "mamba2":
        H, G, C, R = 128, 8, 64, 128
        cfg = b.make_config(b.MAMBA2, B, H, G, C, R, 16, b.BF16)
        A, D = synth.mamba2_params(3, H)
        params = {"A": torch.from_numpy(A).cuda(), "D": torch.from_numpy(D).cuda()}
        toks = synth.mamba2_tokens_device(3, T, B, H, G, C, R, "cuda")
    else:
        H, G, C, R = 32, 32, 128, 128
        cfg = b.make_config(b.GDN, B, H, G, C, R, 16, b.BF16)
        params = None
        toks = synth.gdn_tokens_device(3, T, B, H, G, R, C, "cuda")
    st = b.ReplayState(cfg)
    S0 = synth.checkpoint_device(3, (B, H, C, R), "cuda")
    st.load_checkpoint(S0)
    rng = np.random.default_rng(3)
    acc = np.minimum(rng.geometric(0.35, size=(ROUNDS, B)) - 1, K).astype(np.int32)

    sample = [0, 200, 511]
    S0s = S0[sample].cpu().numpy()
    sess = ro.Mamba2Session(A, D, S0s) if kind == "mamba2" else ro.GDNSession(S0s)
    host = {k: v[:, sample].float().cpu().numpy() for k, v in toks.items()}
    ys = torch.empty((ROUNDS, K, B, H, C), dtype=torch.bfloat16, device="cuda")
    print(f"[full-size spec {kind}] launching {ROUNDS} rounds at batch {B}", flush=True)
    for r in range(ROUNDS):
        st.spec_append(K, {k: v[K * r:K * r + K] for k, v in toks.items()}, params, y=ys[r])
        st.commit(torch.from_numpy(acc[r]).cuda())
    ck = st.read_checkpoint()
    L, Pd, F, E = st.read_book()
    torch.cuda.synchronize()
    yg = ys[:, :, sample].float().cpu().numpy()
    for r in range(ROUNDS):
        outs = sess.spec_append([synth.token(host, K * r + j) for j in range(K)])
        for j in range(K):
            err = ro.normwise_error(yg[r, j], outs[j])
            assert err <= 2e-2, (r, j, err)
        sess.commit(acc[r][sample])
    assert int(E[0]) == 0 and torch.all(Pd == 0)
    Lh, Fh = L.cpu().numpy(), F.cpu().numpy()
    assert np.all((Lh >= 0) & (Lh <= 16))
    assert list(Lh[sample]) == list(sess.len) and list(Fh[sample]) == list(sess.fc)
    assert np.any(Fh > 0), "no sequence flushed: the run did not reach a forced flush"
    err_ck = ro.normwise_error(ck[sample].cpu().numpy(), sess.ckpt, axis=(2, 3))
    assert err_ck <= 1e-4, err_ck
