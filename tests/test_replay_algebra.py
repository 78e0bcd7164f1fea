"""The replay formulas the GPU kernels implement, checked in fp64 against the oracle.

This is not the oracle and the GPU code does not use it: it is a numpy
statement of the unrolled recurrence (the pages describe unrolling the
recurrence over a small window of buffered tokens, [DE] "ReplaySSM beschleunigt
das Decoding ...", section "Wie es funktioniert"; building intermediate states
with two small matrix products, [TR] "NVIDIA ve Dao AI Lab ...", section "Durum
trafigini azaltma ve rollback'in basitlestirilmesi") so that the algebra is
known to be right before any kernel relies on it.

Mamba-2 (per head; entries i = 1..m, entry m is the newest; l_i = dt_i A,
L_i = l_1 + ... + l_i):
  output   y_m   = e^{L_m} (S0 C) + sum_i e^{L_m - L_i} dt_i (B_i . C) x_i + D x_m
  fold     S_new = e^{L_m} S0 + sum_i e^{L_m - L_i} dt_i x_i B_i^T
Gated DeltaNet (per head; g_i = log alpha_i, Gam_i = g_1 + ... + g_i):
  adjoint chain (one output from one checkpoint product): r_m = q;
      for i = m..1: c_i = beta_i (k_i . r_i); r_{i-1} = alpha_i (r_i - c_i k_i)
      o = scale (S0 r_0 + sum_i c_i v_i)
  WY fold: W = K S0^T (row i = S0 k_i); Ahat_ij = beta_i e^{Gam_i - Gam_j} (k_i . k_j), j < i;
      U = (I + Ahat)^{-1} diag(beta) (V - diag(e^{Gam}) W)
      S_new = e^{Gam_m} S0 + sum_i e^{Gam_m - Gam_i} u_i k_i^T
Only exponentials of differences that are <= 0 appear.
"""
import numpy as np
import pytest

from oracle import replay_oracle as ro
from hybrid_decode_replay_amd import synth


def mamba2_replay(S0, A, D, xs, Bs, C, dts):
    """S0 [P,N]; xs [m,P]; Bs [m,N]; C [N]; dts [m] -> (y_m, S_new)."""
    L = np.cumsum(dts * A)
    w = np.exp(L[-1] - L) * dts
    y = np.exp(L[-1]) * (S0 @ C) + ((Bs @ C) * w) @ xs + D * xs[-1]
    S_new = np.exp(L[-1]) * S0 + xs.T @ (w[:, None] * Bs)
    return y, S_new


def gdn_adjoint_output(S0, qs, ks, vs, alphas, betas, scale=1.0):
    r = qs.copy()
    acc = np.zeros(S0.shape[0])
    for i in range(len(ks) - 1, -1, -1):
        c = betas[i] * (ks[i] @ r)
        acc += c * vs[i]
        r = alphas[i] * (r - c * ks[i])
    return scale * (S0 @ r + acc)


def gdn_wy_fold(S0, ks, vs, alphas, betas):
    m = len(ks)
    Gam = np.cumsum(np.log(alphas))
    W = ks @ S0.T                                           # [m, DV]
    Ahat = np.zeros((m, m))
    for i in range(m):
        for j in range(i):
            Ahat[i, j] = betas[i] * np.exp(Gam[i] - Gam[j]) * (ks[i] @ ks[j])
    rhs = betas[:, None] * (vs - np.exp(Gam)[:, None] * W)
    U = np.linalg.solve(np.eye(m) + Ahat, rhs)
    return np.exp(Gam[-1]) * S0 + (np.exp(Gam[-1] - Gam)[:, None] * U).T @ ks


@pytest.mark.parametrize("m", [1, 2, 7, 16])
def test_mamba2_replay_output_and_fold(m):
    H, P, N = 1, 5, 6
    A, D = (np.asarray(a, np.float64) for a in synth.mamba2_params(40 + m, H))
    toks = {k: np.asarray(v, np.float64) for k, v in synth.mamba2_tokens(40 + m, m, 1, H, 1, P, N).items()}
    S0 = synth.checkpoint(40 + m, (1, H, P, N), std=0.3).astype(np.float64)
    S = S0.copy()
    for t in range(m):
        y_seq = ro.mamba2_token(S, toks["x"][t], toks["Bm"][t], toks["Cm"][t], toks["dt"][t], A, D)
    y, S_new = mamba2_replay(S0[0, 0], A[0], D[0], toks["x"][:, 0, 0], toks["Bm"][:, 0, 0],
                             toks["Cm"][m - 1, 0, 0], toks["dt"][:, 0, 0])
    np.testing.assert_allclose(y, y_seq[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_new, S[0, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("m", [1, 3, 16])
def test_gdn_adjoint_chain_and_wy_fold(m):
    H, DK, DV = 1, 8, 6
    toks = {k: np.asarray(v, np.float64) for k, v in synth.gdn_tokens(50 + m, m, 1, H, H, DK, DV).items()}
    S0 = synth.checkpoint(50 + m, (1, H, DV, DK), std=0.3).astype(np.float64)
    S = S0.copy()
    for t in range(m):
        o_seq = ro.gdn_token(S, *(toks[k][t] for k in ("q", "k", "v", "alpha", "beta")), 0.8)
    sl = {k: v[:, 0, 0] for k, v in toks.items()}
    o = gdn_adjoint_output(S0[0, 0], sl["q"][-1], sl["k"], sl["v"], sl["alpha"], sl["beta"], 0.8)
    np.testing.assert_allclose(o, o_seq[0, 0], rtol=1e-12, atol=1e-12)
    S_new = gdn_wy_fold(S0[0, 0], sl["k"], sl["v"], sl["alpha"], sl["beta"])
    np.testing.assert_allclose(S_new, S[0, 0], rtol=1e-11, atol=1e-12)
