"""Pins of the fp64 CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against one of: a brute-force unrolled sum written
as a closed form (not a loop over the recurrence), a special case with a known
closed form, a library routine (torch's fp8 cast), the OCP MX format tables, or
a hand-derived bookkeeping trace.  Together they are chosen so that a dropped
term, a wrong sign, a wrong index or a transposed operand in the oracle fails
at least one test (see test_planted_mistakes_are_caught).
"""
import os

import numpy as np
import pytest

from oracle import replay_oracle as ro
from hybrid_decode_replay_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(d):
    """fp64 copies of a dict of input arrays (keeps test-side arithmetic in fp64)."""
    return {k: np.asarray(v, np.float64) for k, v in d.items()}


# --------------------------------------------------------------------------
# Brute-force references (closed forms, numpy only)
# --------------------------------------------------------------------------

def brute_mamba2(S0, A, D, toks, T):
    """S_t = (prod_{j<=t} a_j) S0 + sum_{s<=t} (prod_{s<j<=t} a_j) dt_s x_s B_s^T,  y_t = S_t C_t + D x_t."""
    B, H, P, N = S0.shape
    G = toks["Bm"].shape[2]
    hpg = H // G
    toks = {k: v.astype(np.float64) for k, v in toks.items()}
    A = np.asarray(A, np.float64)
    D = np.asarray(D, np.float64)
    ys = np.zeros((T, B, H, P))
    S_final = np.zeros_like(S0, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = h // hpg
            a = np.exp(toks["dt"][:, b, h].astype(np.float64) * A[h])
            for t in range(T):
                S = np.prod(a[: t + 1]) * S0[b, h].astype(np.float64)
                for s in range(t + 1):
                    w = np.prod(a[s + 1: t + 1]) * toks["dt"][s, b, h]
                    S = S + w * np.outer(toks["x"][s, b, h], toks["Bm"][s, b, g])
                ys[t, b, h] = S @ toks["Cm"][t, b, g] + D[h] * toks["x"][t, b, h]
                if t == T - 1:
                    S_final[b, h] = S
    return ys, S_final


def brute_gdn(S0, toks, T, scale=1.0):
    """Dense transition matrices M_j = alpha_j (I - beta_j k_j k_j^T):
    S_t = S0 M_1..M_t + sum_s beta_s v_s k_s^T M_{s+1}..M_t,  o_t = scale S_t q_t."""
    B, H, DV, DK = S0.shape
    G = toks["k"].shape[2]
    hpg = H // G
    toks = {k: v.astype(np.float64) for k, v in toks.items()}
    I = np.eye(DK)
    ys = np.zeros((T, B, H, DV))
    S_final = np.zeros_like(S0, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = h // hpg
            k = toks["k"][:, b, g].astype(np.float64)
            M = [toks["alpha"][t, b, h] * (I - toks["beta"][t, b, h] * np.outer(k[t], k[t])) for t in range(T)]
            for t in range(T):
                prod_all = I.copy()
                for j in range(t + 1):
                    prod_all = prod_all @ M[j]
                S = S0[b, h].astype(np.float64) @ prod_all
                for s in range(t + 1):
                    tail = I.copy()
                    for j in range(s + 1, t + 1):
                        tail = tail @ M[j]
                    S = S + toks["beta"][s, b, h] * np.outer(toks["v"][s, b, h], k[s]) @ tail
                ys[t, b, h] = scale * S @ toks["q"][t, b, g]
                if t == T - 1:
                    S_final[b, h] = S
    return ys, S_final


def run_mamba2_oracle(S0, A, D, toks, T):
    S = S0.astype(np.float64).copy()
    ys = np.stack([ro.mamba2_token(S, *(toks[k][t] for k in ("x", "Bm", "Cm", "dt")), A, D) for t in range(T)])
    return ys, S


def run_gdn_oracle(S0, toks, T, scale=1.0):
    S = S0.astype(np.float64).copy()
    ys = np.stack([ro.gdn_token(S, *(toks[k][t] for k in ("q", "k", "v", "alpha", "beta")), scale) for t in range(T)])
    return ys, S


# --------------------------------------------------------------------------
# Recurrences vs brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("G", [1, 2])
def test_mamba2_matches_unrolled_sum(G):
    B, H, P, N, T = 2, 4, 3, 5, 40
    A, D = synth.mamba2_params(11, H)
    toks = synth.mamba2_tokens(11, T, B, H, G, P, N)
    S0 = synth.checkpoint(11, (B, H, P, N), std=0.5)
    y_o, S_o = run_mamba2_oracle(S0, A, D, toks, T)
    y_b, S_b = brute_mamba2(S0, A, D, toks, T)
    assert np.max(np.abs(y_o - y_b)) <= 1e-12 * max(1.0, np.max(np.abs(y_b)))
    assert np.max(np.abs(S_o - S_b)) <= 1e-12 * max(1.0, np.max(np.abs(S_b)))


@pytest.mark.parametrize("G", [1, 2])
def test_gdn_matches_transition_products(G):
    B, H, DK, DV, T = 1, 2, 4, 3, 30
    toks = synth.gdn_tokens(12, T, B, H, G, DK, DV)
    S0 = synth.checkpoint(12, (B, H, DV, DK), std=0.5)
    y_o, S_o = run_gdn_oracle(S0, toks, T, scale=0.7)
    y_b, S_b = brute_gdn(S0, toks, T, scale=0.7)
    assert np.max(np.abs(y_o - y_b)) <= 1e-12 * max(1.0, np.max(np.abs(y_b)))
    assert np.max(np.abs(S_o - S_b)) <= 1e-12 * max(1.0, np.max(np.abs(S_b)))


def test_gdn_rectangular_state_orientation():
    """d_v != d_k: the state is d_v x d_k, o has d_v entries (a transposed state fails)."""
    B, H, DK, DV, T = 1, 1, 5, 2, 6
    toks = synth.gdn_tokens(13, T, B, H, H, DK, DV)
    S0 = synth.checkpoint(13, (B, H, DV, DK), std=0.5)
    y_o, _ = run_gdn_oracle(S0, toks, T)
    y_b, _ = brute_gdn(S0, toks, T)
    assert y_o.shape == (T, B, H, DV)
    np.testing.assert_allclose(y_o, y_b, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Special cases with closed forms
# --------------------------------------------------------------------------

def test_mamba2_single_step_from_zero():
    B, H, G, P, N = 2, 3, 1, 4, 6
    A, D = (np.asarray(a, np.float64) for a in synth.mamba2_params(1, H))
    tok = f64(synth.token(synth.mamba2_tokens(1, 1, B, H, G, P, N), 0))
    S = np.zeros((B, H, P, N))
    y = ro.mamba2_token(S, tok["x"], tok["Bm"], tok["Cm"], tok["dt"], A, D)
    for b in range(B):
        for h in range(H):
            bc = float(np.dot(tok["Bm"][b, 0].astype(np.float64), tok["Cm"][b, 0]))
            want = (tok["dt"][b, h] * bc + D[h]) * tok["x"][b, h].astype(np.float64)
            np.testing.assert_allclose(y[b, h], want, rtol=1e-13, atol=1e-13)


def test_mamba2_zero_decay_is_running_sum():
    B, H, G, P, N, T = 1, 2, 1, 3, 4, 12
    toks = f64(synth.mamba2_tokens(2, T, B, H, G, P, N))
    A = np.zeros(H)
    D = np.zeros(H)
    S0 = synth.checkpoint(2, (B, H, P, N), std=1.0).astype(np.float64)
    S = S0.copy()
    for t in range(T):
        ro.mamba2_token(S, *(toks[k][t] for k in ("x", "Bm", "Cm", "dt")), A, D)
    want = S0 + sum(toks["dt"][t][:, :, None, None] * toks["x"][t][:, :, :, None] * toks["Bm"][t][:, :1, None, :]
                    for t in range(T))
    np.testing.assert_allclose(S, want, rtol=1e-13, atol=1e-13)


def test_mamba2_zero_dt_keeps_state():
    B, H, G, P, N = 1, 2, 1, 3, 4
    A, D = (np.asarray(a, np.float64) for a in synth.mamba2_params(3, H))
    tok = f64(synth.token(synth.mamba2_tokens(3, 1, B, H, G, P, N), 0))
    tok["dt"] = np.zeros_like(tok["dt"])
    S0 = synth.checkpoint(3, (B, H, P, N), std=1.0).astype(np.float64)
    S = S0.copy()
    y = ro.mamba2_token(S, tok["x"], tok["Bm"], tok["Cm"], tok["dt"], A, D)
    np.testing.assert_array_equal(S, S0)
    want = np.einsum("bhpn,bn->bhp", S0, tok["Cm"][:, 0].astype(np.float64)) + D[None, :, None] * tok["x"]
    np.testing.assert_allclose(y, want, rtol=1e-13, atol=1e-13)


def test_mamba2_group_mapping():
    """Heads h use B/C of group h // (H/G): changing group 1's B alters only heads 2,3."""
    B, H, G, P, N = 1, 4, 2, 2, 3
    A, D = synth.mamba2_params(4, H)
    tok = synth.token(synth.mamba2_tokens(4, 1, B, H, G, P, N), 0)
    S1 = np.zeros((B, H, P, N))
    y1 = ro.mamba2_token(S1, tok["x"], tok["Bm"], tok["Cm"], tok["dt"], A, D)
    Bm2 = tok["Bm"].copy()
    Bm2[0, 1] += 1.0
    S2 = np.zeros((B, H, P, N))
    y2 = ro.mamba2_token(S2, tok["x"], Bm2, tok["Cm"], tok["dt"], A, D)
    np.testing.assert_array_equal(y1[0, :2], y2[0, :2])
    assert np.all(y1[0, 2:] != y2[0, 2:])


def test_gdn_zero_beta_is_pure_decay():
    B, H, DK, DV, T = 1, 2, 4, 4, 7
    toks = f64(synth.gdn_tokens(5, T, B, H, H, DK, DV))
    toks["beta"] = np.zeros_like(toks["beta"])
    S0 = synth.checkpoint(5, (B, H, DV, DK), std=1.0).astype(np.float64)
    S = S0.copy()
    for t in range(T):
        o = ro.gdn_token(S, *(toks[k][t] for k in ("q", "k", "v", "alpha", "beta")))
    decay = np.prod(toks["alpha"].astype(np.float64), axis=0)[0]
    np.testing.assert_allclose(S[0], decay[:, None, None] * S0[0], rtol=1e-13)
    np.testing.assert_allclose(o[0], np.einsum("hij,hj->hi", S[0], toks["q"][T - 1, 0]), rtol=1e-13)


def test_gdn_unit_beta_overwrites_key_direction():
    """beta = 1 and |k| = 1: after the update S k = v for any alpha (delta-rule overwrite)."""
    B, H, DK, DV = 2, 3, 8, 5
    tok = f64(synth.token(synth.gdn_tokens(6, 1, B, H, H, DK, DV), 0))
    k = tok["k"].astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    tok["beta"] = np.ones_like(tok["beta"])
    S = synth.checkpoint(6, (B, H, DV, DK), std=1.0).astype(np.float64)
    ro.gdn_token(S, tok["q"], k, tok["v"], tok["alpha"], tok["beta"])
    Sk = np.einsum("bhij,bhj->bhi", S, k)
    np.testing.assert_allclose(Sk, tok["v"], rtol=1e-12, atol=1e-12)


def test_gdn_single_step_from_zero():
    B, H, DK, DV = 2, 2, 6, 3
    tok = f64(synth.token(synth.gdn_tokens(7, 1, B, H, H, DK, DV), 0))
    S = np.zeros((B, H, DV, DK))
    o = ro.gdn_token(S, tok["q"], tok["k"], tok["v"], tok["alpha"], tok["beta"], 0.5)
    kq = np.einsum("bhj,bhj->bh", tok["k"].astype(np.float64), tok["q"])
    want = 0.5 * (tok["beta"] * kq)[:, :, None] * tok["v"]
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)


def test_gdn_orthonormal_keys_projection():
    """alpha = beta = 1 with orthonormal keys: S_T = S0 (I - K^T K) + V^T K."""
    DK, DV, T = 6, 3, 4
    rng = np.random.default_rng(8)
    Q, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    K = Q[:T]                                          # T orthonormal rows
    V = rng.standard_normal((T, DV))
    S0 = rng.standard_normal((1, 1, DV, DK))
    S = S0.copy()
    for t in range(T):
        ro.gdn_token(S, K[t][None, None], K[t][None, None], V[t][None, None], np.ones((1, 1)), np.ones((1, 1)))
    want = S0[0, 0] @ (np.eye(DK) - K.T @ K) + V.T @ K
    np.testing.assert_allclose(S[0, 0], want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Quantizers: OCP MX v1.0 tables, a library cast, hand-derived block scales
# --------------------------------------------------------------------------

def test_e4m3_table_landmarks():
    """OCP FP8 E4M3: max normal 448 (S.1111.110), min normal 2^-6, max subnormal 7*2^-9,
    min subnormal 2^-9, S.1111.111 is NaN, sign bit mirrors."""
    L = ro.lib()
    assert L.oracle_e4m3_decode(0x7E) == 448.0
    assert L.oracle_e4m3_decode(0x08) == 2.0 ** -6
    assert L.oracle_e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert L.oracle_e4m3_decode(0x01) == 2.0 ** -9
    assert L.oracle_e4m3_decode(0x38) == 1.0
    assert L.oracle_e4m3_decode(0x3C) == 1.5
    assert np.isnan(L.oracle_e4m3_decode(0x7F)) and np.isnan(L.oracle_e4m3_decode(0xFF))
    assert L.oracle_e4m3_decode(0xBE) == -448.0 or L.oracle_e4m3_decode(0xFE) == -448.0
    assert L.oracle_e4m3_decode(0xFE) == -448.0


def test_e4m3_encode_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    # every finite code value, every midpoint between neighbours, and random values
    vals = np.array([ro.lib().oracle_e4m3_decode(c) for c in range(0x7F)])
    mids = 0.5 * (vals[1:] + vals[:-1])
    rng = np.random.default_rng(9)
    rand = rng.uniform(-448, 448, 20000) * 2.0 ** rng.integers(-12, 1, 20000)
    x = np.concatenate([vals, -vals, mids, -mids, rand]).astype(np.float32)
    ours = ro.e4m3_encode(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_saturates_beyond_max():
    big = np.array([449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf])
    np.testing.assert_array_equal(ro.e4m3_encode(big), [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    assert ro.e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_e2m1_table_and_ties():
    L = ro.lib()
    table = [L.oracle_e2m1_decode(c) for c in range(16)]
    assert table[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert table[8:] == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    # ties go to the even code (mantissa bit 0)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, code in ties.items():
        assert L.oracle_e2m1_encode(v) == code, v
        assert L.oracle_e2m1_encode(-v) == code | 8, v
    assert L.oracle_e2m1_encode(7.0) == 7 and L.oracle_e2m1_encode(1e9) == 7
    assert L.oracle_e2m1_encode(0.26) == 1 and L.oracle_e2m1_encode(2.6) == 5


def test_mxfp4_block_scale_rule():
    """Shared exponent floor(log2(amax)) - 2 (E2M1's largest exponent), E8M0 bias 127."""
    cases = [(6.0, 127), (4.0, 127), (7.9, 127), (8.0, 128), (0.3, 123), (1.0, 125), (2.0 ** -140, 0)]
    for amax, scale_code in cases:
        v = np.zeros(32)
        v[5] = amax
        v[9] = -amax / 3
        codes, scales = ro.mxfp4_quantize(v)
        assert scales[0] == scale_code, (amax, scales[0])
    codes, scales = ro.mxfp4_quantize(np.zeros(32))
    assert scales[0] == 0 and not codes.any()
    # hand example: amax 5 -> X = 0; 5 ties between 4 and 6 -> 4; 0.3 -> 0.5; -2.6 -> -3
    v = np.zeros(32)
    v[:4] = [5.0, 0.3, -2.6, 1.2]
    codes, scales = ro.mxfp4_quantize(v)
    assert scales[0] == 127
    assert list(codes[:4]) == [6, 1, 8 | 5, 2]
    deq = ro.mxfp4_dequantize(codes, scales)
    assert list(deq[:4]) == [4.0, 0.5, -3.0, 1.0]
    # amax 12 -> X = 1: values are halved before rounding; 12 -> 6 (x2 = 12), 3.1 -> 1.5 (x2 = 3)
    v[:4] = [12.0, 3.1, -0.2, 0.0]
    codes, scales = ro.mxfp4_quantize(v)
    assert scales[0] == 128
    assert list(ro.mxfp4_dequantize(codes, scales)[:4]) == [12.0, 3.0, -0.0, 0.0]


def test_mxfp4_error_bound():
    """|deq - v| <= half an E2M1 step times the block scale (no clipping under the floor rule
    beyond amax*(1 - 6/8) ...): checked as the plain nearest-grid property on random blocks."""
    rng = np.random.default_rng(10)
    v = rng.standard_normal((200, 32)) * 2.0 ** rng.integers(-20, 20, (200, 1))
    codes, scales = ro.mxfp4_quantize(v)
    deq = ro.mxfp4_dequantize(codes, scales)
    scale = 2.0 ** (scales.astype(np.float64) - 127)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for i in range(v.shape[0]):
        r = np.abs(v[i]) / scale[i]
        best = np.min(np.abs(grid[None, :] - np.minimum(r, 6.0)[:, None]), axis=1)
        np.testing.assert_allclose(np.abs(np.abs(deq[i]) / scale[i] - np.minimum(r, 6.0)), best, atol=1e-12)


def test_mxfp4_ceil_scale_rule():
    """Non-clipping rule: X is the smallest exponent with amax <= 6 * 2^X.  Hand cases
    (6 fits X = 0 exactly; 7 and 6(1 + 2^-20) need X = 1 where the default rule clips at
    X = 0; 3 fits X = -1; 12 fits X = 1 like the default rule), the relation to the
    default rule (the same X or one more, one more exactly when the default rule's
    amax / 2^X exceeds 6), and that no element saturates."""
    cases = [(6.0, 127), (7.0, 128), (6.0 * (1 + 2.0 ** -20), 128), (4.0, 127), (8.0, 128), (12.0, 128),
             (12.5, 129), (3.0, 126), (3.1, 127), (0.3, 123), (0.38, 124), (2.0 ** -140, 0)]
    for amax, scale_code in cases:
        v = np.zeros(32)
        v[7] = -amax
        v[20] = amax / 5
        _, scales = ro.mxfp4_quantize(v, "ceil")
        assert scales[0] == scale_code, (amax, scales[0])
    codes, scales = ro.mxfp4_quantize(np.zeros(32), "ceil")
    assert scales[0] == 0 and not codes.any()
    # hand example: amax 7 -> X = 1; 7/2 = 3.5 ties between 3 and 4 -> 4 (even code 6) -> 8;
    # under the default rule (X = 0) the same 7 saturates to 6
    v = np.zeros(32)
    v[:3] = [7.0, -1.3, 0.2]
    codes, scales = ro.mxfp4_quantize(v, "ceil")
    assert scales[0] == 128 and list(codes[:3]) == [6, 8 | 1, 0]
    assert list(ro.mxfp4_dequantize(codes, scales)[:3]) == [8.0, -1.0, 0.0]
    cf, sf = ro.mxfp4_quantize(v)
    assert sf[0] == 127 and ro.mxfp4_dequantize(cf, sf)[0] == 6.0
    rng = np.random.default_rng(12)
    v = rng.standard_normal((400, 32)) * 2.0 ** rng.integers(-30, 30, (400, 1))
    v[:50, 3] = 6.0 * 2.0 ** rng.integers(-20, 20, 50)           # exactly on the boundary
    codes, scales = ro.mxfp4_quantize(v, "ceil")
    _, sfloor = ro.mxfp4_quantize(v)
    amax = np.max(np.abs(v), axis=1)
    X = scales.reshape(-1).astype(np.int64) - 127
    for i in range(v.shape[0]):                                   # brute-force minimality
        fits = [x for x in range(-127, 128) if amax[i] <= 6.0 * 2.0 ** x]
        assert X[i] == fits[0], i
    Xf = sfloor.reshape(-1).astype(np.int64) - 127
    assert np.array_equal(X - Xf, (amax / 2.0 ** Xf > 6.0).astype(np.int64))
    deq = ro.mxfp4_dequantize(codes, scales)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    r = np.abs(v) / 2.0 ** X[:, None]
    assert np.all(r <= 6.0)
    best = np.min(np.abs(grid[None, None, :] - r[:, :, None]), axis=2)
    np.testing.assert_allclose(np.abs(np.abs(deq) / 2.0 ** X[:, None] - r), best, atol=1e-12)


# --------------------------------------------------------------------------
# Bookkeeping: hand-derived golden trace
# --------------------------------------------------------------------------

def _load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            op, arg = tok[0], tok[1]
            nums = list(map(int, tok[2:]))
            rows.append((op, arg, nums))
    return rows


def test_bookkeeping_golden_trace_cap4():
    B, H, G, P, N, cap = 3, 1, 1, 2, 2, 4
    A, D = synth.mamba2_params(20, H)
    sess = ro.Mamba2Session(A, D, np.zeros((B, H, P, N)), cap=cap)
    toks = synth.mamba2_tokens(20, 64, B, H, G, P, N)
    t = 0
    for op, arg, want in _load_golden("bookkeeping_cap4.txt"):
        if op == "decode":
            sess.decode(synth.token(toks, t)); t += 1
        elif op == "spec":
            k = int(arg)
            sess.spec_append([synth.token(toks, t + j) for j in range(k)]); t += k
        elif op == "commit":
            sess.commit([int(a) for a in arg.split(",")])
        elif op == "rollback":
            sess.rollback()
        elif op == "flush":
            sess.flush()
        L, Pd, F = sess.trace()
        got = list(L) + list(Pd) + list(F) + [sess.err]
        assert got == want, (op, arg, got, want)


def test_phase_errors():
    sess = ro.Mamba2Session(np.zeros(1), np.zeros(1), np.zeros((1, 1, 1, 1)), cap=4)
    tok = {"x": np.zeros((1, 1, 1)), "Bm": np.zeros((1, 1, 1)), "Cm": np.zeros((1, 1, 1)), "dt": np.zeros((1, 1))}
    with pytest.raises(ro.PhaseError):
        sess.rollback()
    sess.spec_append([tok, tok])
    for bad in (lambda: sess.decode(tok), sess.flush, lambda: sess.spec_append([tok])):
        with pytest.raises(ro.PhaseError):
            bad()
    with pytest.raises(ValueError):
        ro.Mamba2Session(np.zeros(1), np.zeros(1), np.zeros((1, 1, 1, 1)), cap=17)


def test_decode_flush_cadence_cap16():
    """With the 16-entry buffer, flushes land on steps 16, 32, 48, 64 and len cycles 1..15,0."""
    B, H, G, P, N = 2, 1, 1, 2, 2
    A, D = synth.mamba2_params(21, H)
    sess = ro.Mamba2Session(A, D, np.zeros((B, H, P, N)))
    toks = synth.mamba2_tokens(21, 64, B, H, G, P, N)
    for t in range(64):
        sess.decode(synth.token(toks, t))
        L, Pd, F = sess.trace()
        assert list(L) == [(t + 1) % 16] * B and list(F) == [(t + 1) // 16] * B and not Pd.any()
    assert [e[0] for e in sess.flush_events[::B]] == [15, 31, 47, 63]


# --------------------------------------------------------------------------
# Op-runner semantics: what the pages fix about flush and rollback
# --------------------------------------------------------------------------

def _mk(kind, B=2, cap=4, seed=30, read_copy=None):
    """A session factory (keyword `stagger` passed through) and the tokens of a tiny layer."""
    if kind == "mamba2":
        H, G, P, N = 2, 1, 3, 4
        A, D = synth.mamba2_params(seed, H)
        S0 = synth.checkpoint(seed, (B, H, P, N))
        toks = synth.mamba2_tokens(seed, 80, B, H, G, P, N)
        return (lambda stagger=False: ro.Mamba2Session(A, D, S0, cap=cap, read_copy=read_copy, stagger=stagger)), toks
    H, DK, DV = 2, 4, 3
    S0 = synth.checkpoint(seed, (B, H, DV, DK))
    toks = synth.gdn_tokens(seed, 80, B, H, H, DK, DV)
    return (lambda stagger=False: ro.GDNSession(S0, cap=cap, read_copy=read_copy, stagger=stagger)), toks


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_flush_then_continue_equals_uninterrupted(kind):
    """Folding the buffer into the checkpoint early changes nothing downstream."""
    mk, toks = _mk(kind)
    a, b = mk(), mk()
    ya, yb = [], []
    for t in range(23):
        ya.append(a.decode(synth.token(toks, t)))
        yb.append(b.decode(synth.token(toks, t)))
        if t in (2, 9, 10):
            b.flush()
    np.testing.assert_array_equal(np.stack(ya), np.stack(yb))
    np.testing.assert_array_equal(a.S, b.S)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_rollback_equals_never_appended(kind):
    mk, toks = _mk(kind)
    a, b = mk(), mk()
    for t in range(3):
        a.decode(synth.token(toks, t)); b.decode(synth.token(toks, t))
    a.spec_append([synth.token(toks, 50 + j) for j in range(3)])
    a.rollback()
    for t in range(3, 12):
        np.testing.assert_array_equal(a.decode(synth.token(toks, t)), b.decode(synth.token(toks, t)))
    np.testing.assert_array_equal(a.S, b.S)


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_spec_outputs_and_commit_equal_sequential(kind):
    mk, toks = _mk(kind, cap=16)
    a, b = mk(), mk()
    for t in range(5):
        a.decode(synth.token(toks, t)); b.decode(synth.token(toks, t))
    drafts = [synth.token(toks, 5 + j) for j in range(4)]
    ys = a.spec_append(drafts)
    seq = [b.decode(d) for d in drafts[:2]]
    np.testing.assert_array_equal(ys[0], seq[0])
    np.testing.assert_array_equal(ys[1], seq[1])
    a.commit([2, 2])
    np.testing.assert_array_equal(a.S, b.S)
    assert list(a.len) == list(b.len) == [7, 7]


def test_normwise_error_definition():
    ref = np.array([[1.0, -2.0], [1e-40, 0.0]])
    got = np.array([[1.0, -2.002], [0.0, 0.0]])
    assert abs(ro.normwise_error(got, ref) - max(0.002 / 2.0, 1e-40 / 1e-30)) < 1e-15


# --------------------------------------------------------------------------
# Read-copy and quantized-checkpoint semantics of the op runner
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_readout_equals_identity_token(kind):
    """The readout used after a rounded fold equals a token whose update is the identity
    (Mamba-2 dt = 0; GDN alpha = 1, beta = 0)."""
    mk, toks = _mk(kind)
    sess = mk()
    tok = synth.token(toks, 0)
    S = sess.S.copy()
    if kind == "mamba2":
        ident = dict(tok, dt=np.zeros_like(tok["dt"]))
    else:
        ident = dict(tok, alpha=np.ones_like(tok["alpha"]), beta=np.zeros_like(tok["beta"]))
    y_id = sess._token(S, ident)
    np.testing.assert_array_equal(S, sess.S)
    for b in range(sess.B):
        np.testing.assert_allclose(sess._readout(sess.S[b], sess._slice(tok, b)), y_id[b], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_read_copy_is_identity_on_grid_values(fmt):
    """A checkpoint already on the copy's grid reads back exactly, so read-copy outputs equal
    full-precision outputs; and rounding is idempotent."""
    B, H, G, P, N = 2, 2, 1, 4, 32
    A, D = synth.mamba2_params(60, H)
    S0 = ro.read_copy_values(synth.checkpoint(60, (B, H, P, N)), fmt).reshape(B, H, P, N)
    np.testing.assert_array_equal(ro.read_copy_values(S0, fmt).reshape(S0.shape), S0)
    toks = synth.mamba2_tokens(60, 5, B, H, G, P, N)
    plain = ro.Mamba2Session(A, D, S0, cap=8)
    rc = ro.Mamba2Session(A, D, S0, cap=8, read_copy=fmt)
    for t in range(5):
        np.testing.assert_allclose(rc.decode(synth.token(toks, t)), plain.decode(synth.token(toks, t)),
                                   rtol=1e-13, atol=1e-13)


def test_quantized_checkpoint_rounds_at_every_flush():
    B, H, G, P, N, cap = 2, 2, 1, 4, 32, 3
    A, D = synth.mamba2_params(61, H)
    S0 = synth.checkpoint(61, (B, H, P, N))
    sess = ro.Mamba2Session(A, D, S0, cap=cap, read_copy="fp8", quantized_ckpt=True)
    plain = ro.Mamba2Session(A, D, S0, cap=cap)
    toks = synth.mamba2_tokens(61, 10, B, H, G, P, N)
    assert not np.array_equal(sess.S, plain.S)
    for t in range(10):
        sess.decode(synth.token(toks, t))
        plain.decode(synth.token(toks, t))
        if (t + 1) % cap == 0:
            np.testing.assert_array_equal(ro.read_copy_values(sess.ckpt, "fp8").reshape(sess.ckpt.shape), sess.ckpt)
    assert np.max(np.abs(sess.S - plain.S)) > 0
    with pytest.raises(ValueError):
        ro.Mamba2Session(A, D, S0, quantized_ckpt=True)


# --------------------------------------------------------------------------
# FP16 recurrence checkpoint
# --------------------------------------------------------------------------

def test_binary16_rounding_landmarks():
    """IEEE binary16 (1 sign, 5 exponent bits with bias 15, 10 fraction bits) rounded to
    nearest even, written out from the format: the oracle's fp16 checkpoint rounding."""
    sess = ro.Mamba2Session(np.zeros(1), np.zeros(1), np.zeros((1, 1, 1, 4)), ckpt_dtype="f16")
    u = 2.0 ** -10                           # spacing of binary16 in [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),                  # tie, the even neighbour is 1
        (1.0 + 3 * u / 2, 1.0 + 2 * u),      # tie, the even neighbour is above
        (1.0 + u / 2 + 2.0 ** -30, 1.0 + u), # just above the tie
        (65504.0, 65504.0),                  # largest finite
        (65519.99, 65504.0),                 # below the overflow threshold 65520
        (2.0 ** -24, 2.0 ** -24),            # smallest subnormal
        (2.0 ** -25, 0.0),                   # tie between 0 and 2^-24: even is 0
        (3 * 2.0 ** -26, 2.0 ** -24),        # above that tie
        (2.0 ** -14 - 2.0 ** -24, 2.0 ** -14 - 2.0 ** -24),   # largest subnormal
        (-(1.0 + 3 * u / 2), -(1.0 + 2 * u)),
    ]
    S = np.array([[[[v for v, _ in cases]]]], np.float64).reshape(1, 1, 1, -1)
    got = sess._round(S).ravel()
    np.testing.assert_array_equal(got, [w for _, w in cases])
    with np.errstate(over="ignore"):
        assert np.isinf(sess._round(np.array([65520.0]))[0])   # the overflow threshold rounds up


def test_f16_checkpoint_rounds_at_load_and_every_flush():
    """The fp16 session equals the fp32 session until a flush; at a flush its checkpoint is
    the binary16 rounding of the state the fp32 recurrence reaches from the same start."""
    B, H, G, P, N, cap = 2, 2, 1, 4, 32, 3
    A, D = synth.mamba2_params(62, H)
    S0 = synth.checkpoint(62, (B, H, P, N)).astype(np.float16).astype(np.float64)
    toks = synth.mamba2_tokens(62, 7, B, H, G, P, N)
    f16 = ro.Mamba2Session(A, D, S0, cap=cap, ckpt_dtype="f16")
    f32 = ro.Mamba2Session(A, D, S0, cap=cap)
    np.testing.assert_array_equal(f16.S, S0)
    for t in range(cap - 1):
        np.testing.assert_array_equal(f16.decode(synth.token(toks, t)), f32.decode(synth.token(toks, t)))
    f16.decode(synth.token(toks, cap - 1))
    f32.decode(synth.token(toks, cap - 1))
    np.testing.assert_array_equal(f16.ckpt, f32.ckpt.astype(np.float16).astype(np.float64))
    assert np.max(np.abs(f16.ckpt - f32.ckpt)) > 0
    with pytest.raises(ValueError):
        ro.Mamba2Session(A, D, S0, ckpt_dtype="bf16")
    with pytest.raises(ValueError):
        ro.Mamba2Session(A, D, S0, read_copy="fp8", quantized_ckpt=True, ckpt_dtype="f16")


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_f16_checkpoint_exact_on_dyadic_inputs(kind):
    """With inputs whose recurrence stays on the binary16 grid (A = 0 and dt a power of two
    for Mamba-2; alpha = 1, beta = 0 for GDN, so the state only decays by exactly 1 or
    accumulates exactly), the fp16 and fp32 sessions agree bit for bit through flushes."""
    B, H, G, P, N, cap = 1, 2, 1, 4, 16, 2
    S0 = (np.arange(B * H * P * N).reshape(B, H, P, N) % 7 - 3) * 0.25
    if kind == "mamba2":
        A, D = np.zeros(H), np.ones(H)
        toks = {"x": np.full((6, B, H, P), 0.5), "Bm": np.full((6, B, G, N), 0.25),
                "Cm": np.full((6, B, G, N), 1.0), "dt": np.full((6, B, H), 0.125)}
        a, b = (ro.Mamba2Session(A, D, S0, cap=cap, ckpt_dtype=c) for c in ("f16", "f32"))
    else:
        toks = {"q": np.full((6, B, G, N), 0.5), "k": np.full((6, B, G, N), 0.25),
                "v": np.full((6, B, H, P), 1.0), "alpha": np.ones((6, B, H)), "beta": np.zeros((6, B, H))}
        a, b = (ro.GDNSession(S0, cap=cap, ckpt_dtype=c) for c in ("f16", "f32"))
    for t in range(6):
        np.testing.assert_array_equal(a.decode(synth.token(toks, t)), b.decode(synth.token(toks, t)))
        np.testing.assert_array_equal(a.ckpt, b.ckpt)
    assert a.fc[0] == 3


# --------------------------------------------------------------------------
# Staggered flush phases and the full-buffer decode at capacity 1
# --------------------------------------------------------------------------

def test_stagger_schedule_closed_form():
    """Sequence b folds after 1 + (b mod cap) tokens, then every cap tokens."""
    B, H, G, P, N, cap, T = 5, 1, 1, 4, 8, 3, 11
    A, D = synth.mamba2_params(63, H)
    sess = ro.Mamba2Session(A, D, synth.checkpoint(63, (B, H, P, N)), cap=cap, stagger=True)
    toks = synth.mamba2_tokens(63, T, B, H, G, P, N)
    for t in range(T):
        sess.decode(synth.token(toks, t))
    got = sorted((op, b) for op, b in sess.flush_events)
    want = sorted((s, b) for b in range(B) for s in range(T)
                  if s + 1 >= 1 + b % cap and (s + 1 - (1 + b % cap)) % cap == 0)
    assert got == want


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_stagger_leaves_values_unchanged(kind):
    """The flush schedule changes only where the state is cut, not the values (fp64)."""
    mk, toks = _mk(kind, B=4)
    plain, stag = mk(), mk(stagger=True)
    for t in range(30):
        np.testing.assert_allclose(stag.decode(synth.token(toks, t)), plain.decode(synth.token(toks, t)),
                                   rtol=1e-12, atol=1e-12)
    assert stag.flush_events != plain.flush_events
    np.testing.assert_array_equal(plain.lim, 4)


def test_full_buffer_decode_at_capacity_one():
    """cap = 1, len = 1 after a commit: the decode folds the committed entry, appends the
    token, and the one-entry window is full again -- two flushes on one step."""
    B, H, G, P, N = 2, 1, 1, 4, 8
    A, D = synth.mamba2_params(64, H)
    sess = ro.Mamba2Session(A, D, synth.checkpoint(64, (B, H, P, N)), cap=1)
    toks = synth.mamba2_tokens(64, 3, B, H, G, P, N)
    sess.spec_append([synth.token(toks, 0)])
    sess.commit([1, 0])
    fc0 = sess.fc.copy()
    sess.decode(synth.token(toks, 1))
    np.testing.assert_array_equal(sess.len, [0, 0])
    np.testing.assert_array_equal(sess.fc - fc0, [2, 1])


def test_capacity_one_double_fold_rounds_once():
    """cap = 1 with a committed draft: the decode folds the draft and the token in one pass,
    so an FP8 checkpoint is rounded once.  A = 0, dt = x = 1 (each fold adds B): from 1 the
    two entries add 1/16 each; one rounding gives 1 + 1/8 = 1.125 (on the grid), where
    rounding after each fold would give round(1.0625) = 1 (tie to even), then again 1."""
    S0 = np.ones((1, 1, 1, 1))
    sess = ro.Mamba2Session(np.zeros(1), np.zeros(1), S0, cap=1, ckpt_dtype="fp8")
    tok = {"x": np.ones((1, 1, 1)), "Bm": np.full((1, 1, 1), 1 / 16), "Cm": np.ones((1, 1, 1)),
           "dt": np.ones((1, 1))}
    sess.spec_append([tok])
    sess.commit([1])
    y = sess.decode(tok)
    assert sess.ckpt.ravel()[0] == 1.125
    assert y.ravel()[0] == 1.125 and sess.fc[0] == 2


# --------------------------------------------------------------------------
# FP8 (E4M3) recurrence checkpoint
# --------------------------------------------------------------------------

def test_fp8_checkpoint_fold_rounds_by_hand():
    """One Mamba-2 token folded at cap = 1 (A = 0, dt = x = 1, so the fold adds B to the
    state).  Each element's E4M3 rounding worked by hand from the format (1.m x 2^(e-7),
    3 mantissa bits, subnormal step 2^-9, largest finite 448):
      1 + 1/16     -> 1        tie between 1 and 1.125, even mantissa wins
      1 + 3/32     -> 1.125    nearest
      1.125 + 1/16 -> 1.25     tie between 1.125 and 1.25, even mantissa wins
      416 + 64     -> 448      saturates (step 32 in [256, 448])
      0 + 0.001    -> 2^-9     nearest subnormal (half step is 2^-10 < 0.001)
      0 - 0.3      -> -0.3125  step 2^-5 in [0.25, 0.5)
    The step's output is read from the rounded state: y = S' . C (D = 0)."""
    S0 = np.array([1.0, 1.0, 1.125, 416.0, 0.0, 0.0]).reshape(1, 1, 1, 6)
    Bv = np.array([1 / 16, 3 / 32, 1 / 16, 64.0, 0.001, -0.3])
    C = np.array([1.0, 1.0, 1.0, 2.0 ** -7, 512.0, 1.0])
    sess = ro.Mamba2Session(np.zeros(1), np.zeros(1), S0, cap=1, ckpt_dtype="fp8")
    np.testing.assert_array_equal(sess.S, S0)         # already on the grid: load keeps it
    tok = {"x": np.ones((1, 1, 1)), "Bm": Bv.reshape(1, 1, 6), "Cm": C.reshape(1, 1, 6), "dt": np.ones((1, 1))}
    y = sess.decode(tok)
    want = np.array([1.0, 1.125, 1.25, 448.0, 2.0 ** -9, -0.3125])
    np.testing.assert_array_equal(sess.ckpt.ravel(), want)
    assert y.ravel()[0] == 1.0 + 1.125 + 1.25 + 3.5 + 1.0 - 0.3125
    assert sess.fc[0] == 1


def test_fp8_checkpoint_gdn_column_replaced_by_hand():
    """GDN with alpha = beta = 1 and k = e_0 replaces column 0 of the state with v; the FP8
    checkpoint then holds v rounded to E4M3 and leaves the other columns as loaded."""
    S0 = np.full((1, 1, 3, 4), 0.5)
    tok = {"q": np.array([[[1.0, 0, 0, 0]]]), "k": np.array([[[1.0, 0, 0, 0]]]),
           "v": np.array([[[1.0625, 0.3, -17.0]]]), "alpha": np.ones((1, 1)), "beta": np.ones((1, 1))}
    sess = ro.GDNSession(S0, cap=1, ckpt_dtype="fp8")
    o = sess.decode(tok)
    want = S0.copy()
    want[0, 0, :, 0] = [1.0, 0.3125, -16.0]           # tie to even; nearest; step 2 in [16, 32)
    np.testing.assert_array_equal(sess.ckpt, want)
    np.testing.assert_array_equal(o.ravel(), [1.0, 0.3125, -16.0])    # o = S' q, q = e_0


def test_fp8_checkpoint_rounds_at_load_and_every_flush():
    """The FP8 session equals the fp32 session until a flush; at a flush its checkpoint is
    the E4M3 rounding of the state the fp32 recurrence reaches from the same start."""
    B, H, G, P, N, cap = 2, 2, 1, 4, 32, 3
    A, D = synth.mamba2_params(65, H)
    S0 = synth.checkpoint(65, (B, H, P, N), std=1.0)
    fp8 = ro.Mamba2Session(A, D, S0, cap=cap, ckpt_dtype="fp8")
    grid = ro.e4m3_decode(ro.e4m3_encode(S0)).reshape(S0.shape)
    np.testing.assert_array_equal(fp8.S, grid)
    assert np.max(np.abs(grid - S0)) > 0
    f32 = ro.Mamba2Session(A, D, grid, cap=cap)
    toks = synth.mamba2_tokens(65, 7, B, H, G, P, N)
    for t in range(cap - 1):
        np.testing.assert_array_equal(fp8.decode(synth.token(toks, t)), f32.decode(synth.token(toks, t)))
    fp8.decode(synth.token(toks, cap - 1))
    f32.decode(synth.token(toks, cap - 1))
    np.testing.assert_array_equal(fp8.ckpt, ro.e4m3_decode(ro.e4m3_encode(f32.ckpt)).reshape(S0.shape))
    # E4M3 keeps 3 mantissa bits: the rounding moves the state by at most 2^-4 relative
    # per normal element, and by at most half the subnormal step 2^-10 below 2^-6
    bound = np.maximum(np.abs(f32.ckpt) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(fp8.ckpt - f32.ckpt) <= bound * (1 + 1e-12))
    with pytest.raises(ValueError):
        ro.Mamba2Session(A, D, S0, read_copy="fp8", ckpt_dtype="fp8")
    with pytest.raises(ValueError):
        ro.Mamba2Session(A, D, S0, read_copy="mxfp4", quantized_ckpt=True, ckpt_dtype="fp8")
    ro.Mamba2Session(A, D, S0, read_copy="mxfp4", ckpt_dtype="fp8")     # allowed


@pytest.mark.parametrize("kind", ["mamba2", "gdn"])
def test_fp8_checkpoint_exact_on_grid_inputs(kind):
    """Inputs whose folds land on the E4M3 grid (increments of 1/4 on states below 4 in
    magnitude): the FP8 and fp32 sessions agree bit for bit through flushes."""
    B, H, G, P, N, cap = 1, 2, 1, 4, 16, 2
    S0 = (np.arange(B * H * P * N).reshape(B, H, P, N) % 7 - 3) * 0.25
    if kind == "mamba2":
        A, D = np.zeros(H), np.ones(H)
        toks = {"x": np.full((6, B, H, P), 0.5), "Bm": np.full((6, B, G, N), 0.25),
                "Cm": np.full((6, B, G, N), 1.0), "dt": np.full((6, B, H), 1.0)}
        a, b = (ro.Mamba2Session(A, D, S0, cap=cap, ckpt_dtype=c) for c in ("fp8", "f32"))
    else:
        toks = {"q": np.full((6, B, G, N), 0.5), "k": np.full((6, B, G, N), 0.25),
                "v": np.full((6, B, H, P), 1.0), "alpha": np.ones((6, B, H)), "beta": np.zeros((6, B, H))}
        a, b = (ro.GDNSession(S0, cap=cap, ckpt_dtype=c) for c in ("fp8", "f32"))
    for t in range(6):
        np.testing.assert_array_equal(a.decode(synth.token(toks, t)), b.decode(synth.token(toks, t)))
        np.testing.assert_array_equal(a.ckpt, b.ckpt)
    assert a.fc[0] == 3
