"""Seeded synthetic workloads for biased-attention forward runs.

This module only draws random numbers and lays them out in the shapes of the
five attention-with-bias workloads; it holds none of the attention or bias
decomposition arithmetic.  Both the fp64 CPU oracle (``oracle/``) and the GPU
path (tests, bench) take their inputs from here, so that the two sides see
bit-identical values.

Workloads (shapes ``[B, H, N, D]``, factor rank ``R``):

* ``tiny_alibi_f32``   B1 H2 N128 D32 R2, fp32, non-causal, Q,K,V ~ N(0,1)
* ``gpt2_alibi_causal`` B8 H12 N2048 D64 R2, bf16, causal, Q,K,V ~ N(0,1)*0.5
* ``sandwich``         B4 H8 N4096 D64 R64 (C=64), bf16, Q,K,V ~ N(0,1)*0.5
* ``vision_svd``       B2 H8 N4096 (64x64 token grid) D16 R8, bf16
* ``pairformer_svd``   B512 H4 N512 D32 R16, bf16, pair rep 512x512x128
* ``mulbias_cos``      B4 H8 N4096 D64 R2, bf16, multiplicative bias cos(i - j)

The language-model workloads stand in for GPT-2 with ALiBi / Sandwich bias,
the vision one for Swin-style relative-position bias (128 channels over 8
heads, R=8), the pairformer one for an AlphaFold 3 Pairformer pair bias, and
``mulbias_cos`` uses the Sandwich shapes for the multiplicative-bias example; none of
their datasets or weights are used.  Draw order per workload: Q, K, V, then
the bias-source parameters, from ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "rng_for", "round_to", "draw_qkv",
    "draw_vision_params", "vision_bias_head", "vision_bias",
    "draw_pairformer_params", "pairformer_bias", "make_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    R: int
    causal: bool
    dtype: str            # "f32" | "bf16"
    bias: str             # "alibi" | "sandwich" | "vision" | "pairformer" | "mulbias_cos"
    qkv_std: float
    seed: int
    C: int = 0            # Sandwich channel count
    grid: int = 0         # vision token grid side (N = grid**2)
    c_z: int = 0          # pair-representation channels
    cp_rank: int = 0      # rank of the outer-product sum forming the pair rep

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_alibi_f32", 1, 2, 128, 32, 2, False, "f32", "alibi", 1.0, 20260001),
        Workload("gpt2_alibi_causal", 8, 12, 2048, 64, 2, True, "bf16", "alibi", 0.5, 20260002),
        Workload("sandwich", 4, 8, 4096, 64, 64, False, "bf16", "sandwich", 0.5, 20260003, C=64),
        Workload("vision_svd", 2, 8, 4096, 16, 8, False, "bf16", "vision", 0.5, 20260004, grid=64),
        Workload("pairformer_svd", 512, 4, 512, 32, 16, False, "bf16", "pairformer", 0.5, 20260005,
                 c_z=128, cp_rank=16),
        # multiplicative rank-2 bias of the rebuttal's example (closed form, each side builds it)
        Workload("mulbias_cos", 4, 8, 4096, 64, 2, False, "bf16", "mulbias_cos", 0.5, 20260006),
    ]
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with some fields replaced (smaller test variants)."""
    w = WORKLOADS[name]
    if overrides:
        w = w.replace(**overrides)
        if w.bias == "vision" and "grid" in overrides and "N" not in overrides:
            w = w.replace(N=w.grid * w.grid)
    if w.bias == "vision" and w.N != w.grid * w.grid:
        raise ValueError("vision workload needs N == grid**2")
    return w


def rng_for(w: Workload, salt: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(w.seed + 1_000_003 * salt))


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 copy of ``x`` after round-to-nearest-even into ``dtype`` (torch's cast)."""
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(tdt).to(torch.float64).numpy()


def draw_qkv(w: Workload, rng: np.random.Generator, rounded: bool = True):
    """Q, K, V as fp64 arrays ``[B,H,N,D]``; values representable in ``w.dtype`` if ``rounded``."""
    shape = (w.B, w.H, w.N, w.D)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape) * w.qkv_std
        out.append(round_to(x, w.dtype) if rounded else x)
    return tuple(out)


# ---------------------------------------------------------------- vision ----
def draw_vision_params(w: Workload, rng: np.random.Generator):
    """Per-head width sigma_h ~ U[4,16] and one N(0,1) draw per table entry t_h[dy,dx]."""
    G = w.grid
    sigma = rng.uniform(4.0, 16.0, size=w.H)
    noise = rng.standard_normal((w.H, 2 * G - 1, 2 * G - 1))
    return {"sigma": sigma, "noise": noise, "grid": G}


def vision_bias_head(params, h: int) -> np.ndarray:
    """Head ``h`` of the spatial relative-position bias, ``[N,N]`` fp64, tokens row-major (i = G*y + x).

    t_h[dy,dx] = 4*exp(-(dy^2+dx^2)/(2 sigma_h^2)) + 0.05*noise, b_ij = t_h[y_i-y_j, x_i-x_j].
    """
    G = params["grid"]
    off = np.arange(-(G - 1), G, dtype=np.float64)
    dy2 = off[:, None] ** 2
    dx2 = off[None, :] ** 2
    table = 4.0 * np.exp(-(dy2 + dx2) / (2.0 * params["sigma"][h] ** 2)) + 0.05 * params["noise"][h]
    y = np.repeat(np.arange(G), G)
    x = np.tile(np.arange(G), G)
    return table[(y[:, None] - y[None, :]) + G - 1, (x[:, None] - x[None, :]) + G - 1]


def vision_bias(params, H: int) -> np.ndarray:
    return np.stack([vision_bias_head(params, h) for h in range(H)])


# ------------------------------------------------------------ pairformer ----
def draw_pairformer_params(w: Workload, rng: np.random.Generator):
    """Pair rep z = sum_r U[i,r] V[j,r] W[r,c] + 0.01 N(0,1); projection P ~ N(0, 1/c_z)."""
    N, r, c = w.N, w.cp_rank, w.c_z
    U = rng.standard_normal((N, r))
    V = rng.standard_normal((N, r))
    W = rng.standard_normal((r, c))
    noise = rng.standard_normal((N, N, c)) * 0.01
    P = rng.standard_normal((c, w.H)) * np.sqrt(1.0 / c)
    return {"U": U, "V": V, "W": W, "noise": noise, "P": P}


def pairformer_bias(params) -> np.ndarray:
    """Per-head pair bias ``[H,N,N]``: z (N x N x c_z) projected to heads; shared by every batch row."""
    z = np.einsum("ir,jr,rc->ijc", params["U"], params["V"], params["W"], optimize=True) + params["noise"]
    return np.ascontiguousarray(np.moveaxis(z @ params["P"], 2, 0))


# ------------------------------------------------------------------ all ----
def make_inputs(w: Workload, with_bias_source: bool = True) -> dict:
    """Q, K, V (fp64, rounded to ``w.dtype``) and, for the vision / pairformer workloads,
    the dense bias-source tensor ``bias_src`` ``[H,N,N]`` fp64 (it is input data there, like a
    learned bias).  ALiBi and Sandwich biases are closed forms that each side builds itself."""
    rng = rng_for(w)
    q, k, v = draw_qkv(w, rng)
    out = {"q": q, "k": k, "v": v}
    if with_bias_source and w.bias == "vision":
        out["bias_params"] = draw_vision_params(w, rng)
        out["bias_src"] = vision_bias(out["bias_params"], w.H)
    elif with_bias_source and w.bias == "pairformer":
        out["bias_params"] = draw_pairformer_params(w, rng)
        out["bias_src"] = pairformer_bias(out["bias_params"])
    return out
