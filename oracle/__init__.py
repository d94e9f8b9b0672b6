"""Plain fp64 CPU oracle for the forward pass of attention with an additive bias.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (``attention_additive_rank_amd``) and does not import it; its
inputs come from ``synth`` (seeded draws) or from the test itself.

What it computes (sources are the FlashBias pages: the paper abstract, "FlashBias:
Fast Computation of Attention with Bias", and the authors' OpenReview rebuttal
of the same title):

* attention with an additive bias, ``o = softmax(s * q k^T + b) v`` -- the
  abstract defines attention with bias as standard attention plus an additive
  bias matrix on the query-key scores; the 1/sqrt(C) scale is the one written
  in the rebuttal's Eq. (1) (answer to Reviewer BRmd, Q1);
* the exact bias decompositions: ALiBi (rebuttal, answer to Reviewer BRmd, Q2:
  slopes of shape #heads, factor tiles Block_q x 2 / Block_k x 2) and Sandwich
  (rebuttal, answer to Reviewer UJUf, Q1 (1)-(2): the bias sum of cosines and
  its cos/sin factor functions with b = phi_q phi_k^T);
* the low-rank product ``b = phi_q phi_k^T`` that FlashBias folds into the
  attention contraction (rebuttal, answer to Reviewer UJUf, Q2; answer to
  Reviewer BRmd, Q3: factors of shape #heads x N x R against a #heads x N x N bias);
* the truncated SVD used for general static biases (abstract: "fast-accurate
  approximation"; rebuttal, answer to Reviewer xU4x, Q6: rank per layer/head,
  computed offline), with the retained-energy figure of the answer to
  Reviewer Bp2x, Q2 (95% energy).

Every function is a direct transcription of the definition with library
primitives (numpy matmul / exp / cos / svd); there is no tiling, no online
softmax and no reordering.  ALiBi slopes follow m_h = 2^(-8(h+1)/H) with h
zero-based, because the pages give only their shape.
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Union

import numpy as np

__all__ = [
    "alibi_slopes", "alibi_bias", "alibi_factors",
    "sandwich_frequencies", "sandwich_bias", "sandwich_factors",
    "lowrank_bias", "cos_mulbias_factors", "attention", "attention_mulbias", "attention_backward",
    "lowrank_factor_grads", "truncated_svd", "bias_energy", "rank_for_energy",
]

BiasLike = Union[None, np.ndarray, Callable[[int, int], np.ndarray]]


# ------------------------------------------------------------------ ALiBi ----
def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes ``m_h = 2^(-8(h+1)/H)``, h = 0..H-1 (shape #heads)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float64)


def alibi_bias(slopes: Sequence[float], N: int) -> np.ndarray:
    """Dense ALiBi bias ``b[h,i,j] = m_h * (j - i)``, ``[H,N,N]`` fp64 (positive for j > i)."""
    m = np.asarray(slopes, dtype=np.float64)
    idx = np.arange(N, dtype=np.float64)
    return m[:, None, None] * (idx[None, None, :] - idx[None, :, None])


def alibi_factors(slopes: Sequence[float], N: int):
    """Exact rank-2 ALiBi factors: ``phi_q(i) = [1, i]``, ``phi_k(j) = [m_h*j, -m_h]``.

    Returns ``(phi_q, phi_k)``, each ``[H,N,2]`` fp64, with phi_q phi_k^T = m_h (j - i).
    """
    m = np.asarray(slopes, dtype=np.float64)
    H = m.shape[0]
    idx = np.arange(N, dtype=np.float64)
    phi_q = np.empty((H, N, 2))
    phi_q[:, :, 0] = 1.0
    phi_q[:, :, 1] = idx[None, :]
    phi_k = np.empty((H, N, 2))
    phi_k[:, :, 0] = m[:, None] * idx[None, :]
    phi_k[:, :, 1] = -m[:, None]
    return phi_q, phi_k


# --------------------------------------------------------------- Sandwich ----
def sandwich_frequencies(C: int) -> np.ndarray:
    """Angular frequencies ``w_k = 10000^(-2k/C)``, k = 1..C/2, in extended precision.

    The factor functions' exponent is read with the same channel count C as the
    bias sum (both are the channel count of the representation)."""
    if C % 2:
        raise ValueError("Sandwich bias needs an even channel count")
    k = np.arange(1, C // 2 + 1, dtype=np.longdouble)
    return np.power(np.longdouble(10000.0), -2.0 * k / np.longdouble(C))


def sandwich_bias(N: int, C: int) -> np.ndarray:
    """Dense Sandwich bias ``b_ij = sum_{k=1}^{C/2} cos((i-j) / 10000^(2k/C))``, ``[N,N]`` fp64.

    b depends on i-j only, so the sum is evaluated once per difference (in
    extended precision) and then laid out as the N x N matrix."""
    w = sandwich_frequencies(C)
    d = np.arange(-(N - 1), N, dtype=np.longdouble)
    t = np.cos(d[:, None] * w[None, :]).sum(axis=1).astype(np.float64)
    i = np.arange(N)
    return t[(i[:, None] - i[None, :]) + N - 1]


def sandwich_factors(N: int, C: int) -> np.ndarray:
    """Sandwich factor functions ``phi(i) = [cos(i w_1), sin(i w_1), ..., cos(i w_{C/2}), sin(i w_{C/2})]``.

    ``[N,C]`` fp64; phi_q = phi_k = phi, and phi phi^T equals :func:`sandwich_bias`
    by cos(a-b) = cos a cos b + sin a sin b."""
    w = sandwich_frequencies(C)
    ang = np.arange(N, dtype=np.longdouble)[:, None] * w[None, :]
    phi = np.empty((N, C), dtype=np.float64)
    phi[:, 0::2] = np.cos(ang).astype(np.float64)
    phi[:, 1::2] = np.sin(ang).astype(np.float64)
    return phi


# --------------------------------------------------------------- low rank ----
def cos_mulbias_factors(N: int) -> np.ndarray:
    """Rank-2 factors of the multiplicative bias b_ij = cos(i - j) from the rebuttal's
    example (answer to Reviewer BRmd, Q1 (2)): phi(i) = [cos i, sin i] for queries and keys
    alike, since cos(i - j) = cos i cos j + sin i sin j.  ``[N, 2]`` fp64."""
    i = np.arange(N, dtype=np.float64)
    return np.stack([np.cos(i), np.sin(i)], axis=1)


def lowrank_bias(phi_q: np.ndarray, phi_k: np.ndarray) -> np.ndarray:
    """``b = phi_q phi_k^T`` over the last two axes (``[..., N, R] x [..., N, R] -> [..., N, N]``)."""
    return np.matmul(phi_q, np.swapaxes(phi_k, -1, -2))


# --------------------------------------------------------------- attention ---
def _bias_slice(bias: BiasLike, b: int, h: int, B: int, H: int) -> Optional[np.ndarray]:
    if bias is None:
        return None
    if callable(bias):
        return bias(b, h)
    bias = np.asarray(bias)
    if bias.ndim == 2:
        return bias
    if bias.ndim == 3:
        return bias[h if bias.shape[0] == H else 0]
    return bias[b if bias.shape[0] == B else 0, h if bias.shape[1] == H else 0]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, bias: BiasLike = None,
              scale: Optional[float] = None, causal: bool = False,
              rows: Optional[np.ndarray] = None):
    """Naive softmax attention with an additive bias, fp64.

    ``q, k, v``: ``[B,H,N,D]``.  ``bias``: None, an array broadcastable over
    batch/head (``[N,N]``, ``[H,N,N]``, ``[B,H,N,N]`` with size-1 axes allowed) or
    a callable ``(b, h) -> [N,N]``.  ``scale`` defaults to 1/sqrt(D).  With
    ``causal`` query i sees keys j <= i.  ``rows`` restricts the output to those
    query rows.  Returns ``(O, LSE)``: ``O`` ``[B,H,len(rows),D]``, ``LSE`` the natural
    log-sum-exp of each row's scores ``[B,H,len(rows)]``.

    Per (b,h): L = s*QK^T + b; L_ij = -inf where masked; m = max_j L_ij;
    p = exp(L - m); l = sum_j p; O = p V / l; LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rows), v.shape[3]))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            L = s * (q[b, h, rows] @ k[b, h].T)
            bb = _bias_slice(bias, b, h, B, H)
            if bb is not None:
                L = L + np.asarray(bb, dtype=np.float64)[rows]
            if causal:
                L = np.where(np.arange(Nk)[None, :] > rows[:, None], -np.inf, L)
            m = L.max(axis=1, keepdims=True)
            p = np.exp(L - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, h] = (p @ v[b, h]) / l
            lse[b, h] = (m + np.log(l))[:, 0]
    return out, lse


def attention_mulbias(q: np.ndarray, k: np.ndarray, v: np.ndarray, bias: BiasLike,
                      scale: Optional[float] = None, causal: bool = False,
                      rows: Optional[np.ndarray] = None):
    """Naive softmax attention with a multiplicative bias, fp64 (rebuttal, answer to
    Reviewer BRmd, Q1, Eq. (1)): the scaled scores are multiplied element-wise by the bias.

    Arguments as :func:`attention`, ``bias`` required.  Per (b,h): L = (s*QK^T) * b;
    L_ij = -inf where masked; m = max_j L_ij; p = exp(L - m); l = sum_j p; O = p V / l;
    LSE = m + ln l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    Nk = k.shape[2]
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rows), v.shape[3]))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            bb = np.asarray(_bias_slice(bias, b, h, B, H), dtype=np.float64)
            L = (s * (q[b, h, rows] @ k[b, h].T)) * bb[rows]
            if causal:
                L = np.where(np.arange(Nk)[None, :] > rows[:, None], -np.inf, L)
            m = L.max(axis=1, keepdims=True)
            p = np.exp(L - m)
            l = p.sum(axis=1, keepdims=True)
            out[b, h] = (p @ v[b, h]) / l
            lse[b, h] = (m + np.log(l))[:, 0]
    return out, lse


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, bias: BiasLike = None,
                       scale: Optional[float] = None, causal: bool = False, o_stored: Optional[np.ndarray] = None):
    """Gradients of ``O = softmax(s Q K^T + b) V`` for an upstream gradient ``dO``, fp64.

    The textbook chain rule, per (b,h), with nothing fused or reordered:
    L = s Q K^T + b (masked entries -inf); P = softmax_rows(L); O = P V;
    dV = P^T dO; dP = dO V^T; dL_ij = P_ij (dP_ij - sum_k P_ik dP_ik) (the softmax
    Jacobian); dQ = s dL K; dK = s dL^T Q; db = dL (the gradient with respect to the
    bias matrix; masked entries get 0).  The training use of the bias factors is the
    rebuttal's (answer to Reviewer UJUf, Q1: Sandwich bias in GPT-2 training).
    ``o_stored``: when given, the row term sum_k P_ik dP_ik is taken as rowsum(dO * O) with
    this O (the two are equal for the exact O, since sum_k P_ik dP_ik = sum_d dO_id O_id);
    a backward that receives the forward's stored output, rounded to the input dtype, uses
    that form.
    Returns ``(dq, dk, dv, db)`` with ``db`` ``[B,H,N,N]``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, D = q.shape
    s = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    db = np.zeros((B, H, N, k.shape[2]))
    for b in range(B):
        for h in range(H):
            L = s * (q[b, h] @ k[b, h].T)
            bb = _bias_slice(bias, b, h, B, H)
            if bb is not None:
                L = L + np.asarray(bb, dtype=np.float64)
            if causal:
                L = np.where(np.arange(k.shape[2])[None, :] > np.arange(N)[:, None], -np.inf, L)
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P = P / P.sum(axis=1, keepdims=True)
            dv[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            if o_stored is None:
                row = np.sum(P * dP, axis=1, keepdims=True)
            else:
                row = np.sum(do[b, h] * np.asarray(o_stored[b, h], dtype=np.float64), axis=1, keepdims=True)
            dL = P * (dP - row)
            dq[b, h] = s * (dL @ k[b, h])
            dk[b, h] = s * (dL.T @ q[b, h])
            db[b, h] = dL
    return dq, dk, dv, db


def lowrank_factor_grads(db: np.ndarray, phi_q: np.ndarray, phi_k: np.ndarray):
    """Gradients of a loss with respect to the factors of ``b = phi_q phi_k^T`` from the
    gradient ``db`` with respect to b: ``dphi_q = db phi_k``, ``dphi_k = db^T phi_q``
    (over the last two axes; factors broadcast like ``db`` allows)."""
    db = np.asarray(db, dtype=np.float64)
    return (np.matmul(db, np.asarray(phi_k, dtype=np.float64)),
            np.matmul(np.swapaxes(db, -1, -2), np.asarray(phi_q, dtype=np.float64)))


# --------------------------------------------------------------------- SVD ---
def truncated_svd(bias: np.ndarray, R: int, method: str = "full"):
    """Top-R SVD factors of one ``[N,N]`` bias: ``phi_q = U_R sqrt(S_R)``, ``phi_k = V_R sqrt(S_R)``.

    ``method="full"`` uses ``numpy.linalg.svd`` (every singular value);
    ``method="arpack"`` uses ``scipy.sparse.linalg.svds`` for the top R only (large N).
    Returns a dict with ``phi_q``, ``phi_k`` (``[N,R]``), ``sigma`` (all singular values
    for "full", the top R otherwise, descending) and ``energy`` = sum_{r<R} s_r^2 / ||b||_F^2.
    """
    bias = np.asarray(bias, dtype=np.float64)
    if method == "full":
        U, S, Vt = np.linalg.svd(bias)
        Ur, Sr, Vr = U[:, :R], S[:R], Vt[:R].T
        sigma = S
    elif method == "arpack":
        from scipy.sparse.linalg import svds
        U, S, Vt = svds(bias, k=R, which="LM", random_state=0)
        order = np.argsort(S)[::-1]
        Ur, Sr, Vr = U[:, order], S[order], Vt[order].T
        sigma = Sr
    else:
        raise ValueError(method)
    root = np.sqrt(Sr)
    total = float(np.sum(bias * bias))
    energy = float(np.sum(Sr ** 2) / total) if total > 0 else 1.0
    return {"phi_q": Ur * root[None, :], "phi_k": Vr * root[None, :], "sigma": sigma, "energy": energy}


def bias_energy(bias: np.ndarray, phi_q: np.ndarray, phi_k: np.ndarray) -> dict:
    """Approximation error of ``phi_q phi_k^T`` against a dense bias: relative Frobenius error
    and max-abs error."""
    diff = np.asarray(bias, dtype=np.float64) - lowrank_bias(phi_q, phi_k)
    return {"rel_fro": float(np.linalg.norm(diff) / np.linalg.norm(bias)),
            "max_abs": float(np.abs(diff).max())}


def rank_for_energy(bias: np.ndarray, target: float = 0.95, R_max: Optional[int] = None) -> dict:
    """Smallest rank R whose truncated SVD keeps ``target`` of the energy of one ``[N,N]``
    bias: sum_{r<R} s_r^2 >= target * ||b||_F^2 (the 95%-energy criterion of the rebuttal,
    answer to Reviewer Bp2x, Q2).  Every singular value from ``numpy.linalg.svd``; the search
    stops at ``R_max`` (default N), returning R_max with ``reached`` False if the target is
    not met.  An all-zero bias needs rank 1."""
    bias = np.asarray(bias, dtype=np.float64)
    N = bias.shape[0]
    R_max = N if R_max is None else int(R_max)
    sigma = np.linalg.svd(bias, compute_uv=False)
    total = float(np.sum(bias * bias))
    if total == 0.0:
        return {"R": 1, "energy": 1.0, "reached": True}
    kept = np.cumsum(sigma[:R_max] ** 2)
    hit = np.nonzero(kept >= target * total)[0]
    if len(hit):
        R = int(hit[0]) + 1
        return {"R": R, "energy": float(kept[R - 1] / total), "reached": True}
    return {"R": R_max, "energy": float(kept[-1] / total), "reached": False}
