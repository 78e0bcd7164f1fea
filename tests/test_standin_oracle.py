"""CPU pins of the stand-in layers' references (oracle/standin_oracle.py).

Pinned by closed forms and by brute force, not by retyping the definition:
  linear     identity weights return the input; one-hot inputs pick weight
             columns; a product against hand-computed integers.
  attention  one cached token returns its value row; a zero query averages the
             values; a query far along one key picks that key's value; swapping
             cached (key, value) pairs changes nothing; grouped-query heads read
             their group's cache; scalar-loop brute force on tiny inputs.
"""
import numpy as np

from oracle import standin_oracle as so


def test_linear_identity_and_one_hot():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((5, 8))
    np.testing.assert_array_equal(so.linear(X, np.eye(8)), X)
    W = rng.standard_normal((3, 8))
    e = np.zeros((1, 8))
    e[0, 5] = 1.0
    np.testing.assert_array_equal(so.linear(e, W)[0], W[:, 5])


def test_linear_hand_computed():
    X = np.array([[1.0, 2.0, 3.0], [-1.0, 0.0, 2.0]])
    W = np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.5]])
    np.testing.assert_array_equal(so.linear(X, W), np.array([[-2.0, 5.5], [-3.0, -1.0]]))


def _cache(seed, B=2, Hq=4, Hkv=2, L=5, D=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, D)), rng.standard_normal((B, Hkv, L, D)),
            rng.standard_normal((B, Hkv, L, D)))


def test_attention_single_token_and_zero_query():
    q, K, V = _cache(1, L=1)
    o = so.attention(q, K, V, 0.3)
    for h in range(4):
        np.testing.assert_allclose(o[:, h], V[:, h // 2, 0], rtol=0, atol=1e-15)
    q, K, V = _cache(2, L=7)
    o = so.attention(np.zeros_like(q), K, V, 1.0)
    for h in range(4):
        np.testing.assert_allclose(o[:, h], V[:, h // 2].mean(axis=1), rtol=1e-14, atol=1e-15)


def test_attention_dominant_key_and_permutation():
    q, K, V = _cache(3, L=6)
    K = K / np.linalg.norm(K, axis=-1, keepdims=True)
    q2 = np.zeros_like(q)
    for b in range(2):
        for h in range(4):
            q2[b, h] = 400.0 * K[b, h // 2, 3]                # far along key 3
    o = so.attention(q2, K, V, 1.0)
    for h in range(4):
        np.testing.assert_allclose(o[:, h], V[:, h // 2, 3], rtol=0, atol=1e-6)
    perm = np.array([4, 0, 5, 2, 1, 3])
    np.testing.assert_allclose(so.attention(q, K[:, :, perm], V[:, :, perm], 0.7), so.attention(q, K, V, 0.7),
                               rtol=1e-13, atol=1e-14)


def test_attention_matches_scalar_loops():
    q, K, V = _cache(4, B=2, Hq=4, Hkv=1, L=4, D=3)
    np.testing.assert_allclose(so.attention(q, K, V, 0.5), so.attention_loops(q.tolist(), K.tolist(), V.tolist(), 0.5),
                               rtol=1e-13, atol=1e-14)
