"""Plain fp64 CPU references of the stand-in non-SSM layers of a hybrid decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module.  It shares
no code with the GPU library and never imports it.

A hybrid model's decode step runs, besides its SSM layers, dense projections of
every mixer and a few attention layers ([TR] "NVIDIA ve Dao AI Lab, hibrit model
cozumlemesini hizlandirmak icin ReplaySSM'i sundu", section "ReplaySSM nasil
calisir?"); the pages' decode-step speedups are measured on such models
(section "Durum trafigini azaltma ve rollback'in basitlestirilmesi").  The
library's stand-ins compute the plain definitions below; the pages give no
formula for them, so these are the textbook ones:

  linear     Y = X W^T              (W stored [out][in])
  attention  o[b, h] = sum_t softmax_t(scale q[b, h] . K[b, g, t]) V[b, g, t],
             g = h // (Hq // Hkv)   (grouped-query heads)

Inputs are the bf16 values the device sees, upcast exactly to fp64.
"""
from __future__ import annotations

import numpy as np


def linear(X, W):
    """Y[m][n] = sum_k X[m][k] W[n][k] in fp64 (a library matrix product)."""
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64).T


def attention(q, K, V, scale):
    """q [B][Hq][D], K and V [B][Hkv][L][D] -> o [B][Hq][D], softmax over the L tokens in
    fp64 with the maximum subtracted (the same value, computed without overflow)."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, D = q.shape
    Hkv = K.shape[1]
    qpk = Hq // Hkv
    o = np.empty((B, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // qpk
            s = scale * (K[b, g] @ q[b, h])
            p = np.exp(s - s.max())
            o[b, h] = (p @ V[b, g]) / p.sum()
    return o


def attention_loops(q, K, V, scale):
    """The same definition written out with scalar loops (for tiny inputs): the exponentials
    of the raw scores, their sum, and the weighted sum of values."""
    import math
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, L = len(K[0]), len(K[0][0])
    qpk = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // qpk
            e = []
            for t in range(L):
                s = 0.0
                for d in range(D):
                    s += float(q[b][h][d]) * float(K[b][g][t][d])
                e.append(math.exp(scale * s))
            z = sum(e)
            for d in range(D):
                acc = 0.0
                for t in range(L):
                    acc += e[t] * float(V[b][g][t][d])
                out[b][h][d] = acc / z
    return np.array(out)
