"""Seeded synthetic inputs for the BitLinear workloads.

Shapes and random draws only: this module holds none of the method's arithmetic, so
both the CPU oracle and the HIP path can take their inputs from it. Weights follow the
nn.Linear convention, W [N out, K in]; activations are X [T tokens, K].

Workloads (the pages name the models, not a dataset: "Llama3-8B-1.58-100B-tokens" in
the bitnet.cpp article's list of supported models, and the 70B model of the b1.58
paper review's "Main findings"; synthetic tensors of those layer shapes stand in):
  tiny      W [256, 1024] ~ 0.02 N(0,1), X [8, 1024] ~ N(0,1)
  decode8b  one Llama-3-8B layer at T = 1: q, o [4096, 4096]; k, v [1024, 4096];
            gate, up [14336, 4096]; down [4096, 14336]
  prefill   T = 2048 with (N, K) = (14336, 4096) and (4096, 14336); X is Student-t
            with 3 degrees of freedom scaled to unit variance (variance of t_3 is 3)
  sweep70b  W (N, K) = (8192, 28672) and (28672, 8192); T in {1, 8, 32, 64}
  fullpass  32 layers x the seven decode8b projections at T = 16
"""
from __future__ import annotations

import numpy as np

WEIGHT_SIGMA = 0.02

# Llama-3-8B projection shapes (N out, K in); q/k/v and gate/up share an input.
LLAMA3_8B = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (14336, 4096),
    "up": (14336, 4096),
    "down": (4096, 14336),
}
LLAMA3_8B_LAYERS = 32
# projections grouped by the activation they read (attention excluded: the inputs of
# o and down are fresh synthetic tensors)
LLAMA3_8B_INPUTS = {"attn_in": ("q", "k", "v"), "attn_out": ("o",),
                    "mlp_in": ("gate", "up"), "mlp_mid": ("down",)}

LLAMA_70B_SWEEP = {"down": (8192, 28672), "gate": (28672, 8192)}
SWEEP_TOKENS = (1, 8, 32, 64)

TINY_W = (256, 1024)
TINY_T = 8
PREFILL_T = 2048
PREFILL_SHAPES = ((14336, 4096), (4096, 14336))
FULLPASS_T = 16


def _rng(seed):
    return np.random.default_rng(seed)


def weights(N: int, K: int, seed: int, sigma: float = WEIGHT_SIGMA) -> np.ndarray:
    """W [N, K] fp32 with entries sigma * N(0, 1)."""
    w = _rng(seed).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def acts_normal(T: int, K: int, seed: int) -> np.ndarray:
    """X [T, K] fp32 with entries N(0, 1)."""
    return _rng(seed).standard_normal((T, K), dtype=np.float32)


def acts_student_t(T: int, K: int, seed: int, df: int = 3) -> np.ndarray:
    """X [T, K] fp32, Student-t(df) scaled to unit variance (Var t_df = df/(df-2))."""
    x = _rng(seed).standard_t(df, size=(T, K))
    return (x / np.sqrt(df / (df - 2.0))).astype(np.float32)


def wide_range(n: int, seed: int, lo_exp: int = -149, hi_exp: int = 100) -> np.ndarray:
    """fp32 values whose magnitudes spread over many binades (denormals included):
    random sign, random 24-bit significand, exponent uniform in [lo_exp, hi_exp]."""
    r = _rng(seed)
    mant = r.integers(1 << 23, 1 << 24, size=n).astype(np.float64)
    e = r.integers(lo_exp, hi_exp + 1, size=n)
    v = np.ldexp(mant, e - 23)
    sign = np.where(r.random(n) < 0.5, -1.0, 1.0)
    return (sign * v).astype(np.float32)


def decode8b_layer(seed: int = 0):
    """{proj: W [N, K]} of one Llama-3-8B layer, one seed per projection."""
    return {p: weights(N, K, seed * 16 + i)
            for i, (p, (N, K)) in enumerate(LLAMA3_8B.items())}


def decode8b_inputs(T: int = 1, seed: int = 100):
    """{input name: X [T, K]} for the four distinct activations of a layer."""
    out = {}
    for i, (name, projs) in enumerate(LLAMA3_8B_INPUTS.items()):
        K = LLAMA3_8B[projs[0]][1]
        out[name] = acts_normal(T, K, seed + i)
    return out
