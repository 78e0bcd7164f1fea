"""Seeded synthetic inputs for the SSM decode layers.

This module only draws random numbers and shapes them into the value
distributions of the workloads; it holds none of the layer arithmetic.  It is
the one piece shared by the GPU tests, the benchmark and the CPU oracle runs,
so both sides see bit-identical inputs.

Recipes (all seeded):
  Mamba-2   x, B, C ~ N(0, 1); dt = softplus(N(0, 1) - 2) per (token, b, h);
            A_h = -exp(U(0, 1.5)); D_h ~ N(0, 1); checkpoint zero or N(0, 0.1)
            (0.1 is the standard deviation).
  GDN       q, k = L2-normalised N(0, 1) rows; v ~ N(0, 1);
            alpha = sigmoid(N(3, 1)); beta = sigmoid(N(0, 1)); checkpoint
            N(0, 0.1).
Reduced-precision inputs are drawn in fp32 and rounded to bf16 (round to
nearest even); the fp32 copies returned to the oracle hold exactly the bf16
values.
"""
from __future__ import annotations

import numpy as np

try:  # torch is plumbing for device tensors and the bf16 rounding
    import torch
except Exception:  # pragma: no cover
    torch = None


def _softplus(z):
    return np.logaddexp(0.0, z)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32."""
    a = np.ascontiguousarray(a, np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


# --------------------------------------------------------------------------
# Host (numpy) generators: small shapes, oracle-sized runs
# --------------------------------------------------------------------------

def mamba2_params(seed: int, H: int):
    rng = np.random.default_rng([seed, 101])
    A = (-np.exp(rng.uniform(0.0, 1.5, H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    return A, D


def mamba2_tokens(seed: int, T: int, B: int, H: int, G: int, P: int, N: int,
                  dtype: str = "f32"):
    """Per-token Mamba-2 inputs for T steps: dict of fp32 arrays with leading T axis."""
    rng = np.random.default_rng([seed, 102])
    x = rng.standard_normal((T, B, H, P), dtype=np.float32)
    Bm = rng.standard_normal((T, B, G, N), dtype=np.float32)
    Cm = rng.standard_normal((T, B, G, N), dtype=np.float32)
    dt = _softplus(rng.standard_normal((T, B, H)) - 2.0).astype(np.float32)
    out = {"x": x, "Bm": Bm, "Cm": Cm, "dt": dt}
    if dtype == "bf16":
        out = {k: round_bf16(v) for k, v in out.items()}
    return out


def gdn_tokens(seed: int, T: int, B: int, H: int, G: int, DK: int, DV: int,
               dtype: str = "f32"):
    """Per-token Gated DeltaNet inputs: q, k [T,B,G,DK], v [T,B,H,DV], alpha/beta [T,B,H]."""
    rng = np.random.default_rng([seed, 202])
    q = rng.standard_normal((T, B, G, DK))
    k = rng.standard_normal((T, B, G, DK))
    q = (q / np.linalg.norm(q, axis=-1, keepdims=True)).astype(np.float32)
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((T, B, H, DV), dtype=np.float32)
    alpha = _sigmoid(rng.normal(3.0, 1.0, (T, B, H))).astype(np.float32)
    beta = _sigmoid(rng.standard_normal((T, B, H))).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}


def checkpoint(seed: int, shape, std: float = 0.1, zero: bool = False):
    """Initial fp32 checkpoint in logical layout ([B,H,P,N] or [B,H,DV,DK])."""
    if zero:
        return np.zeros(shape, np.float32)
    rng = np.random.default_rng([seed, 303])
    return (std * rng.standard_normal(shape)).astype(np.float32)


def token(inputs: dict, t: int) -> dict:
    """Slice step t out of a dict of [T, ...] arrays."""
    return {k: v[t] for k, v in inputs.items()}


# --------------------------------------------------------------------------
# Device (torch) generators: full-size runs; values are drawn on the GPU
# --------------------------------------------------------------------------

def _gen(device, seed, stream_id):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream_id))
    return g


def mamba2_tokens_device(seed, T, B, H, G, P, N, device, dtype=None):
    """Mamba-2 inputs for T steps on `device` (bf16 by default): x, Bm, Cm, dt."""
    dtype = dtype or torch.bfloat16
    g = _gen(device, seed, 1)
    x = torch.randn((T, B, H, P), generator=g, device=device, dtype=torch.float32).to(dtype)
    Bm = torch.randn((T, B, G, N), generator=g, device=device, dtype=torch.float32).to(dtype)
    Cm = torch.randn((T, B, G, N), generator=g, device=device, dtype=torch.float32).to(dtype)
    z = torch.randn((T, B, H), generator=g, device=device, dtype=torch.float32)
    dt = torch.nn.functional.softplus(z - 2.0).to(dtype)
    return {"x": x, "Bm": Bm, "Cm": Cm, "dt": dt}


def gdn_tokens_device(seed, T, B, H, G, DK, DV, device, dtype=None):
    dtype = dtype or torch.bfloat16
    g = _gen(device, seed, 2)
    q = torch.randn((T, B, G, DK), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((T, B, G, DK), generator=g, device=device, dtype=torch.float32)
    q = (q / q.norm(dim=-1, keepdim=True)).to(dtype)
    k = (k / k.norm(dim=-1, keepdim=True)).to(dtype)
    v = torch.randn((T, B, H, DV), generator=g, device=device, dtype=torch.float32).to(dtype)
    alpha = torch.sigmoid(3.0 + torch.randn((T, B, H), generator=g, device=device))
    beta = torch.sigmoid(torch.randn((T, B, H), generator=g, device=device))
    return {"q": q, "k": k, "v": v, "alpha": alpha.float(), "beta": beta.float()}


def checkpoint_device(seed, shape, device, std=0.1):
    g = _gen(device, seed, 3)
    return std * torch.randn(shape, generator=g, device=device, dtype=torch.float32)
