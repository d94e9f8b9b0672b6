"""Pins of the fp64 CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not contain: closed-form
values derived by hand (tests/golden/closed_forms.json), a library routine
(torch's scaled_dot_product_attention on the CPU in fp64, numpy eigvalsh,
scipy logsumexp), invariants of softmax attention, and brute force with scalar
loops on tiny inputs.  A dropped term, a wrong sign or index, or a transposed
operand in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _eval(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"cos": math.cos, "sin": math.sin}))


# ------------------------------------------------------------------ ALiBi ----
def test_alibi_slopes_closed_form():
    g = _golden()["alibi_slopes_H8"]
    np.testing.assert_array_equal(oracle.alibi_slopes(8), [_eval(e) for e in g["values_expr"]])
    m12 = oracle.alibi_slopes(12)
    assert m12[0] == pytest.approx(2.0 ** (-2.0 / 3.0), rel=1e-15)
    assert m12[-1] == 2.0 ** -8          # the last head always gets 2^-8
    assert np.all(np.diff(m12) < 0)


def test_alibi_bias_closed_form_values():
    g = _golden()["alibi_bias_examples"]
    b = oracle.alibi_bias(oracle.alibi_slopes(g["H"]), 16)
    for c in g["cases"]:
        assert b[c["h"], c["i"], c["j"]] == _eval(c["value_expr"])


def test_alibi_bias_structure():
    m = oracle.alibi_slopes(12)
    b = oracle.alibi_bias(m, 64)
    assert np.all(np.diagonal(b, axis1=1, axis2=2) == 0)
    np.testing.assert_array_equal(b, -np.swapaxes(b, 1, 2))      # antisymmetric
    np.testing.assert_allclose(np.diff(b, axis=2), np.broadcast_to(m[:, None, None], (12, 64, 63)), rtol=0, atol=1e-13)
    assert np.all(b[:, 0, 1] > 0)                                   # positive for j > i


def test_alibi_factor_identity_1e12():
    """phi_q phi_k^T reproduces m_h (j - i) to 1e-12 at the GPT-2 size (N = 2048)."""
    m = oracle.alibi_slopes(12)
    pq, pk = oracle.alibi_factors(m, 2048)
    assert pq.shape == pk.shape == (12, 2048, 2)
    err = np.abs(oracle.lowrank_bias(pq, pk) - oracle.alibi_bias(m, 2048)).max()
    assert err <= 1e-12


# --------------------------------------------------------------- Sandwich ----
@pytest.mark.parametrize("key", ["sandwich_C4", "sandwich_C2"])
def test_sandwich_closed_forms(key):
    g = _golden()[key]
    N = max(max(c["i"], c["j"]) for c in g["cases"]) + 1
    b = oracle.sandwich_bias(N, g["C"])
    for c in g["cases"]:
        assert b[c["i"], c["j"]] == pytest.approx(_eval(c["value_expr"]), abs=1e-14)


def test_sandwich_frequencies_closed_form():
    w = oracle.sandwich_frequencies(4).astype(np.float64)
    np.testing.assert_allclose(w, [1e-2, 1e-4], rtol=1e-15)
    w64 = oracle.sandwich_frequencies(64).astype(np.float64)
    assert w64[0] == pytest.approx(10000.0 ** (-1.0 / 32.0), rel=1e-15)   # highest frequency < 1
    assert w64[-1] == pytest.approx(1e-4, rel=1e-15)


def test_sandwich_structure():
    C, N = 64, 300
    b = oracle.sandwich_bias(N, C)
    np.testing.assert_allclose(np.diagonal(b), C / 2, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(b, b.T)                                   # symmetric
    np.testing.assert_array_equal(b[1:, 1:], b[:-1, :-1])                   # Toeplitz
    ev = np.linalg.eigvalsh(b)
    assert ev.min() > -1e-9                                                 # Gram matrix: PSD


def test_sandwich_factor_identity_1e12():
    """phi phi^T reproduces the cosine sum to 1e-12 at the Sandwich size (N = 4096, C = 64)."""
    N, C = 4096, 64
    phi = oracle.sandwich_factors(N, C)
    assert phi.shape == (N, C)
    np.testing.assert_allclose(phi[:, 0::2] ** 2 + phi[:, 1::2] ** 2, 1.0, rtol=0, atol=1e-15)
    err = np.abs(oracle.lowrank_bias(phi, phi) - oracle.sandwich_bias(N, C)).max()
    assert err <= 1e-12


# --------------------------------------------------------------- attention ---
def _sdpa(q, k, v, mask=None, scale=None, causal=False):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    m = None if mask is None else t(np.broadcast_to(mask, q.shape[:2] + (q.shape[2], k.shape[2])))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale,
                                                         is_causal=causal)
    return o.numpy()


def _qkv(B, H, N, D, seed, std=1.0):
    r = np.random.default_rng(seed)
    return tuple(r.standard_normal((B, H, N, D)) * std for _ in range(3))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_no_bias_matches_library(causal):
    q, k, v = _qkv(2, 3, 77, 32, 1)
    o, _ = oracle.attention(q, k, v, causal=causal)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=causal), rtol=0, atol=1e-12)


def test_attention_bias_matches_library():
    """An asymmetric per-head bias passed as a float attn_mask: pins the bias sign,
    its orientation (row = query) and the scale."""
    q, k, v = _qkv(2, 3, 65, 16, 2)
    r = np.random.default_rng(3)
    bias = r.standard_normal((3, 65, 65)) * 2.0
    for scale in (None, 0.3):
        o, _ = oracle.attention(q, k, v, bias=bias, scale=scale)
        np.testing.assert_allclose(o, _sdpa(q, k, v, mask=bias[None], scale=scale), rtol=0, atol=1e-12)


def test_attention_causal_bias_matches_library():
    q, k, v = _qkv(1, 2, 50, 8, 4)
    m = oracle.alibi_slopes(2)
    bias = oracle.alibi_bias(m, 50)
    o, _ = oracle.attention(q, k, v, bias=bias, causal=True)
    mask = np.where(np.arange(50)[None, :] > np.arange(50)[:, None], -np.inf, 0.0) + bias
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask=mask[None]), rtol=0, atol=1e-12)


def _brute(q, k, v, bias, scale, causal):
    """Scalar loops with math.fsum: O and LSE by the definition."""
    B, H, N, D = q.shape
    O = np.zeros((B, H, N, D))
    LSE = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                js = [j for j in range(N) if not (causal and j > i)]
                L = [scale * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) + bias[h, i, j] for j in js]
                mx = max(L)
                p = [math.exp(x - mx) for x in L]
                l = math.fsum(p)
                LSE[b, h, i] = mx + math.log(l)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(pj * v[b, h, j, d] for pj, j in zip(p, js)) / l
    return O, LSE


@pytest.mark.parametrize("N,causal", [(1, False), (5, True), (8, False), (8, True)])
def test_attention_brute_force_tiny(N, causal):
    q, k, v = _qkv(1, 2, N, 4, 10 + N)
    bias = np.random.default_rng(N).standard_normal((2, N, N))
    o, lse = oracle.attention(q, k, v, bias=bias, scale=0.7, causal=causal)
    ob, lb = _brute(q, k, v, bias, 0.7, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-14)


def test_lse_matches_logsumexp():
    from scipy.special import logsumexp
    q, k, v = _qkv(1, 1, 40, 8, 5)
    bias = np.random.default_rng(6).standard_normal((40, 40))
    _, lse = oracle.attention(q, k, v, bias=bias)
    _, lse2 = oracle.attention(q, k, v, bias=bias - lse[0, 0][:, None])
    np.testing.assert_allclose(lse2, 0.0, atol=1e-13)
    # library check of the same quantity on the scores the SDPA pin fixed
    s = 1 / math.sqrt(8)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s * q[0, 0] @ k[0, 0].T + bias, axis=1), rtol=0, atol=1e-12)


def test_row_constant_invariance():
    """Adding a per-row constant to b leaves O unchanged (ALiBi's -m_h*i is such a term)."""
    q, k, v = _qkv(2, 2, 33, 16, 7)
    bias = np.random.default_rng(8).standard_normal((2, 33, 33))
    row_c = np.random.default_rng(9).standard_normal((2, 33, 1)) * 100
    o1, l1 = oracle.attention(q, k, v, bias=bias, causal=True)
    o2, l2 = oracle.attention(q, k, v, bias=bias + row_c, causal=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, np.broadcast_to(row_c[None, :, :, 0], l1.shape), rtol=0, atol=1e-10)


def test_softmax_value_path_invariants():
    q, k, v = _qkv(1, 1, 20, 8, 11)
    # constant V rows -> O equals that constant
    vc = np.broadcast_to(np.arange(8.0), v.shape).copy()
    o, _ = oracle.attention(q, k, vc, bias=np.random.default_rng(1).standard_normal((20, 20)))
    np.testing.assert_allclose(o, vc, rtol=0, atol=1e-13)
    # one key with a +50 bias captures every row
    bias = np.zeros((20, 20))
    bias[:, 13] = 50.0
    o, _ = oracle.attention(q, k, v, bias=bias)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 13], (20, 8)), rtol=0, atol=1e-12)
    # permuting keys (K, V and bias columns together) leaves O unchanged
    bias = np.random.default_rng(2).standard_normal((20, 20))
    perm = np.random.default_rng(3).permutation(20)
    o1, _ = oracle.attention(q, k, v, bias=bias)
    o2, _ = oracle.attention(q, k[:, :, perm], v[:, :, perm], bias=bias[:, perm])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)


def test_rows_subset_equals_full():
    q, k, v = _qkv(2, 2, 30, 8, 12)
    bias = np.random.default_rng(13).standard_normal((2, 30, 30))
    rows = np.array([0, 7, 29, 3])
    of, lf = oracle.attention(q, k, v, bias=bias, causal=True)
    os_, ls = oracle.attention(q, k, v, bias=bias, causal=True, rows=rows)
    np.testing.assert_array_equal(os_, of[:, :, rows])
    np.testing.assert_array_equal(ls, lf[:, :, rows])


def test_lowrank_bias_folds_into_contraction():
    """softmax(s QK^T + phi_q phi_k^T) V equals plain attention on Q' = [Q s, phi_q], K' = [K, phi_k]
    with unit scale -- the augmented contraction of the FlashBias recipe."""
    q, k, v = _qkv(1, 2, 24, 8, 14)
    r = np.random.default_rng(15)
    pq, pk = r.standard_normal((2, 24, 3)), r.standard_normal((2, 24, 3))
    s = 1 / math.sqrt(8)
    o1, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    qa = np.concatenate([q * s, pq[None]], axis=-1)
    ka = np.concatenate([k, pk[None]], axis=-1)
    np.testing.assert_allclose(o1, _sdpa(qa, ka, v, scale=1.0), rtol=0, atol=1e-12)


# --------------------------------------------------------------------- SVD ---
def test_svd_singular_values_match_eigvalsh():
    b = np.random.default_rng(16).standard_normal((60, 60))
    f = oracle.truncated_svd(b, 5)
    ref = np.sqrt(np.clip(np.linalg.eigvalsh(b.T @ b), 0, None))[::-1]
    np.testing.assert_allclose(f["sigma"], ref, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("method", ["full", "arpack"])
def test_svd_eckart_young(method):
    r = np.random.default_rng(17)
    b = r.standard_normal((80, 80)) @ np.diag(0.8 ** np.arange(80)) @ r.standard_normal((80, 80))
    R = 6
    f = oracle.truncated_svd(b, R, method=method)
    s_all = np.linalg.svd(b, compute_uv=False)
    err2 = np.linalg.norm(b - oracle.lowrank_bias(f["phi_q"], f["phi_k"])) ** 2
    assert err2 == pytest.approx(np.sum(s_all[R:] ** 2), rel=1e-8)
    assert f["energy"] == pytest.approx(np.sum(s_all[:R] ** 2) / np.sum(s_all ** 2), rel=1e-10)
    np.testing.assert_allclose(f["sigma"][:R], s_all[:R], rtol=1e-9)


def test_svd_exact_on_rank_r():
    r = np.random.default_rng(18)
    a, c = r.standard_normal((50, 4)), r.standard_normal((50, 4))
    b = a @ c.T
    f = oracle.truncated_svd(b, 4)
    np.testing.assert_allclose(oracle.lowrank_bias(f["phi_q"], f["phi_k"]), b, rtol=0, atol=1e-12)
    assert f["energy"] == pytest.approx(1.0, abs=1e-14)


def test_svd_recovers_alibi_and_sandwich_rank():
    """The exact biases have the rank their factors claim: 2 for ALiBi, C for Sandwich."""
    b = oracle.alibi_bias(oracle.alibi_slopes(4), 64)[1]
    f = oracle.truncated_svd(b, 2)
    assert f["sigma"][2] < 1e-12 * f["sigma"][0]
    sw = oracle.sandwich_bias(256, 4)
    f = oracle.truncated_svd(sw, 4)
    assert f["sigma"][4] < 1e-10 * f["sigma"][0]


# ----------------------------------------------------------- synth inputs ----
def test_synth_vision_bias_structure():
    w = synth.workload("vision_svd", grid=8, B=1, H=2)
    inp = synth.make_inputs(w)
    b = inp["bias_src"]
    assert b.shape == (2, 64, 64)
    # b_ij depends only on (y_i - y_j, x_i - x_j): translating both tokens leaves it unchanged
    G = 8
    tok = lambda y, x: G * y + x
    assert b[0, tok(1, 1), tok(2, 3)] == b[0, tok(4, 2), tok(5, 4)]
    # the diagonal is t_h[0,0] = 4 + 0.05 * noise
    assert np.allclose(np.diagonal(b[1]), np.diagonal(b[1])[0])
    assert abs(np.diagonal(b[1])[0] - 4.0) < 0.5


def test_synth_rounding_is_representable():
    w = synth.workload("sandwich", B=1, H=1, N=64)
    q, k, v = synth.draw_qkv(w, synth.rng_for(w))
    np.testing.assert_array_equal(synth.round_to(q, "bf16"), q)
    # bf16 keeps 8 significant bits: every value times 2^k is an integer below 2^8
    m, _ = np.frexp(q[q != 0])
    assert np.all(np.abs(m * 256) == np.round(np.abs(m * 256)))


# --------------------------------------------------- rank for a target energy ---
def _with_singular_values(sig, N, seed):
    r = np.random.default_rng(seed)
    U, _ = np.linalg.qr(r.standard_normal((N, N)))
    V, _ = np.linalg.qr(r.standard_normal((N, N)))
    s = np.zeros(N)
    s[:len(sig)] = sig
    return (U * s) @ V.T


def test_rank_for_energy_closed_form():
    # singular values 4, 2, 1, 1/2: energies 16, 4, 1, 1/4 of 21.25 -> cumulative shares
    # 0.753, 0.941, 0.988, 1: 95% needs rank 3, 99% rank 4, 75% rank 1
    b = _with_singular_values([4.0, 2.0, 1.0, 0.5], 12, 1)
    assert oracle.rank_for_energy(b, 0.95)["R"] == 3
    assert oracle.rank_for_energy(b, 0.99)["R"] == 4
    assert oracle.rank_for_energy(b, 0.75)["R"] == 1
    e = oracle.rank_for_energy(b, 0.95)["energy"]
    assert abs(e - 21.0 / 21.25) < 1e-12
    miss = oracle.rank_for_energy(b, 0.99, R_max=2)
    assert miss == {"R": 2, "energy": miss["energy"], "reached": False} and abs(miss["energy"] - 20 / 21.25) < 1e-12


def test_rank_for_energy_exact_biases():
    # ALiBi has rank 2, Sandwich rank C: full energy at exactly that rank
    N = 96
    alibi = oracle.alibi_bias(oracle.alibi_slopes(4), N)[1]
    assert oracle.rank_for_energy(alibi, 1 - 1e-9)["R"] == 2
    # Sandwich has rank C, but its low-frequency terms are nearly collinear at small N, so
    # high energy shares come earlier; rank C keeps all of it
    sw = oracle.sandwich_bias(N, 16)
    full = oracle.rank_for_energy(sw, 1 - 1e-12, R_max=16)
    assert full["reached"] and full["R"] <= 16
    assert oracle.rank_for_energy(np.zeros((5, 5)), 0.95)["R"] == 1


# ------------------------------------------------------- multiplicative bias ---
def test_mulbias_all_ones_is_plain_attention():
    r = np.random.default_rng(41)
    q, k, v = (r.standard_normal((2, 2, 20, 8)) for _ in range(3))
    o1, l1 = oracle.attention_mulbias(q, k, v, np.ones((20, 20)))
    o2, l2 = oracle.attention(q, k, v)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_mulbias_brute_force_cos_example(causal):
    """The pages' example b_ij = cos(i - j) with factors [cos i, sin i] (rank 2), against
    element-by-element loops that evaluate cos(i - j) directly."""
    r = np.random.default_rng(42)
    B, H, N, D = 1, 2, 6, 4
    q, k, v = (r.standard_normal((B, H, N, D)) for _ in range(3))
    idx = np.arange(N, dtype=np.float64)
    phi = np.stack([np.cos(idx), np.sin(idx)], axis=1)
    got, lse = oracle.attention_mulbias(q, k, v, oracle.lowrank_bias(phi, phi), scale=0.7, causal=causal)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                L = []
                for j in range(N):
                    if causal and j > i:
                        continue
                    dot = sum(q[b, h, i, c] * k[b, h, j, c] for c in range(D))
                    L.append((j, 0.7 * dot * math.cos(i - j)))
                m = max(x for _, x in L)
                w = [(j, math.exp(x - m)) for j, x in L]
                tot = sum(x for _, x in w)
                for c in range(D):
                    ref = sum(x * v[b, h, j, c] for j, x in w) / tot
                    assert abs(got[b, h, i, c] - ref) < 1e-12
                assert abs(lse[b, h, i] - (m + math.log(tot))) < 1e-12


def test_mulbias_expansion_identity():
    """Eq. (3) of the same answer: with q' = s [q phi_q,1 .. q phi_q,R] and
    k' = [k phi_k,1 .. k phi_k,R], q' k'^T equals (s q k^T) * (phi_q phi_k^T)."""
    r = np.random.default_rng(43)
    N, D, R, s = 9, 5, 3, 0.3
    q, k = r.standard_normal((N, D)), r.standard_normal((N, D))
    pq, pk = r.standard_normal((N, R)), r.standard_normal((N, R))
    qe = s * np.concatenate([q * pq[:, [c]] for c in range(R)], axis=1)
    ke = np.concatenate([k * pk[:, [c]] for c in range(R)], axis=1)
    np.testing.assert_allclose(qe @ ke.T, (s * q @ k.T) * oracle.lowrank_bias(pq, pk), rtol=1e-12, atol=1e-12)


def test_mulbias_scale_moves_between_scores_and_bias():
    r = np.random.default_rng(44)
    q, k, v = (r.standard_normal((1, 1, 15, 8)) for _ in range(3))
    b = r.standard_normal((15, 15))
    o1, _ = oracle.attention_mulbias(q, k, v, b, scale=0.5)
    o2, _ = oracle.attention_mulbias(q, k, v, 2.5 * b, scale=0.2)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)


def test_cos_mulbias_factors_closed_form():
    phi = oracle.cos_mulbias_factors(50)
    i = np.arange(50)
    np.testing.assert_allclose(oracle.lowrank_bias(phi, phi), np.cos(i[:, None] - i[None, :]), rtol=0, atol=1e-13)
    assert phi[0].tolist() == [1.0, 0.0]


# ------------------------------------------------------------------ backward ---
def _loss(q, k, v, do, bias, causal, scale):
    o, _ = oracle.attention(q, k, v, bias=bias, causal=causal, scale=scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    """Central differences of <dO, O> in fp64 against the analytic gradients, for every
    entry of Q, K, V and the bias on a tiny problem."""
    r = np.random.default_rng(61)
    B, H, N, D, s = 1, 2, 5, 3, 0.6
    q, k, v, do = (r.standard_normal((B, H, N, D)) for _ in range(4))
    bias = r.standard_normal((B, H, N, N))
    dq, dk, dv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=causal, scale=s)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv), (bias, db)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, bias, causal, s)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, bias, causal, s)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_lowrank_factor_grads_match_finite_differences():
    r = np.random.default_rng(62)
    B, H, N, D, R = 1, 1, 6, 4, 3
    q, k, v, do = (r.standard_normal((B, H, N, D)) for _ in range(4))
    pq, pk = r.standard_normal((H, N, R)), r.standard_normal((H, N, R))
    _, _, _, db = oracle.attention_backward(q, k, v, do, bias=oracle.lowrank_bias(pq, pk))
    gq, gk = oracle.lowrank_factor_grads(db[0], pq, pk)
    eps = 1e-6
    for x, g in ((pq, gq), (pk, gk)):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, oracle.lowrank_bias(pq, pk), False, None)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, oracle.lowrank_bias(pq, pk), False, None)
            x[idx] = old
            assert abs(g[idx] - (lp - lm) / (2 * eps)) < 1e-7


def test_backward_invariants():
    """dO = 0 gives zero gradients; the bias gradient rows sum to 0 (softmax is shift
    invariant along a row); with dO = V-independent constant rows, dV columns sum to
    N times that constant."""
    r = np.random.default_rng(63)
    q, k, v = (r.standard_normal((1, 2, 7, 4)) for _ in range(3))
    z = oracle.attention_backward(q, k, v, np.zeros_like(q))
    assert all(np.all(x == 0) for x in z)
    do = r.standard_normal(q.shape)
    _, _, dv, db = oracle.attention_backward(q, k, v, do, bias=r.standard_normal((7, 7)), causal=True)
    np.testing.assert_allclose(db.sum(axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_backward_stored_output_form():
    """The row term as rowsum(dO * O) with the exact O (computed here by the forward
    oracle) gives the same gradients as sum_k P_ik dP_ik (the identity
    sum_k P_ik (dO V^T)_ik = sum_d dO_id (P V)_id); with a perturbed O the gradients move
    by exactly P (dO . dO_err) terms, so the option is really used."""
    r = np.random.default_rng(64)
    q, k, v, do = (r.standard_normal((2, 2, 9, 4)) for _ in range(4))
    bias = r.standard_normal((9, 9))
    o, _ = oracle.attention(q, k, v, bias=bias, causal=True)
    a = oracle.attention_backward(q, k, v, do, bias=bias, causal=True)
    b = oracle.attention_backward(q, k, v, do, bias=bias, causal=True, o_stored=o)
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)
    e = 1e-3 * r.standard_normal(o.shape)
    _, _, dv2, db2 = oracle.attention_backward(q, k, v, do, bias=bias, causal=True, o_stored=o + e)
    np.testing.assert_allclose(dv2, a[2], atol=1e-15)              # dV does not involve the row term
    P = db2 - a[3]                                                 # = -P * rowsum(dO * e)
    shift = np.sum(do * e, axis=-1, keepdims=True)
    P0 = np.where(np.abs(shift) > 0, -P / shift, 0.0)              # recovers P, rows sum to 1
    np.testing.assert_allclose(P0.sum(axis=-1), 1.0, atol=1e-9)


# ------------------------------------------------ approximation error report ---
def test_bias_energy_eckart_young_closed_form():
    """A bias with chosen singular values 4, 2, 1, 1/2 (random orthogonal U, V, built here,
    not by the oracle's SVD) truncated to rank R with the known singular vectors: the
    relative Frobenius error is sqrt(sum_{r>=R} s_r^2 / sum_r s_r^2) exactly, e.g.
    sqrt(5.25 / 21.25) at R = 1 and sqrt(0.25 / 21.25) at R = 3, and rank 4 leaves nothing."""
    N = 12
    r = np.random.default_rng(5)
    U, _ = np.linalg.qr(r.standard_normal((N, N)))
    V, _ = np.linalg.qr(r.standard_normal((N, N)))
    sig = np.array([4.0, 2.0, 1.0, 0.5])
    b = (U[:, :4] * sig) @ V[:, :4].T
    for R, expect in ((1, math.sqrt(5.25 / 21.25)), (2, math.sqrt(1.25 / 21.25)), (3, math.sqrt(0.25 / 21.25)),
                      (4, 0.0)):
        pq = U[:, :R] * np.sqrt(sig[:R])
        pk = V[:, :R] * np.sqrt(sig[:R])
        e = oracle.bias_energy(b, pq, pk)
        assert e["rel_fro"] == pytest.approx(expect, abs=1e-13), R
    # the residual after rank 3 is the rank-1 term 0.5 u_4 v_4^T: its largest entry
    pq, pk = U[:, :3] * np.sqrt(sig[:3]), V[:, :3] * np.sqrt(sig[:3])
    res = 0.5 * np.abs(np.outer(U[:, 3], V[:, 3])).max()
    assert oracle.bias_energy(b, pq, pk)["max_abs"] == pytest.approx(res, rel=1e-12)


def test_bias_energy_single_entry_residual_and_orientation():
    """b = phi_q phi_k^T plus one entry c at (i, j), with asymmetric factors: the residual is
    that one entry, so max-abs is |c| and the relative Frobenius error |c| / ||b||_F.  Using
    phi_k phi_q^T (a transposed product) instead would leave a far larger residual."""
    r = np.random.default_rng(6)
    N, R = 9, 2
    pq, pk = r.standard_normal((N, R)), 3.0 * r.standard_normal((N, R))
    b = pq @ pk.T
    c = -0.625
    b[2, 7] += c
    e = oracle.bias_energy(b, pq, pk)
    assert e["max_abs"] == pytest.approx(abs(c), abs=1e-14)
    assert e["rel_fro"] == pytest.approx(abs(c) / math.sqrt(float(np.sum(b * b))), rel=1e-12)
    wrong = oracle.bias_energy(b, pk, pq)
    assert wrong["max_abs"] > 10 * abs(c)
