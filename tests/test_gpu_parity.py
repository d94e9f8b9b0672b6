"""GPU parity of the HIP path (libflashbias, through the C ABI) against the fp64 oracle.

Bars: fp32 workloads max-abs <= 1e-4 and relative L2 <= 1e-4; bf16 workloads
max-abs <= 2e-2 and relative L2 <= 5e-3, over every compared output element.
Exact biases (ALiBi, Sandwich) are compared with the oracle's bias from its
defining formula; SVD workloads with the oracle fed the same rounded factors.
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import Case, TOL, assert_close, assert_grad_close, errors, round_exact, sample_rows, say, tdtype, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fb(cuda):
    import attention_additive_rank_amd as m
    m.load()
    return m


# ---------------------------------------------------------------- factors ----
def _ulp(x: np.ndarray, dt: str) -> np.ndarray:
    prec, emin = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14)}[dt]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** emin)))
    return 2.0 ** (e - prec + 1)


def _pieces(x: np.ndarray, dt: str, n: int):
    out, rest = [], x.copy()
    for _ in range(n):
        p = round_exact(rest, dt)
        out.append(p)
        rest = rest - p
    return out


@pytest.mark.parametrize("dt,split", [("f32", 1), ("bf16", 1), ("f16", 1), ("f16", 2), ("bf16", 3)])
def test_alibi_factor_kernel(fb, dt, split):
    H, N = 12, 2048
    say(f"alibi factors dt={dt} split={split}")
    pq, pk, r = fb.fb_make_factors("alibi", H, N, dtype=tdtype(dt), split=split, R_pad=16)
    assert r == 2 * split * (split + 1) // 2
    gq, gk = to_np(pq), to_np(pk)
    assert np.all(gq[:, :, r:] == 0) and np.all(gk[:, :, r:] == 0)
    oq, ok = oracle.alibi_factors(oracle.alibi_slopes(H), N)
    pairs = [(a, s - a) for s in range(split) for a in range(s + 1)]   # (0,0), (0,1), (1,0), (0,2), ...
    for c in range(2):
        qp, kp = _pieces(oq[:, :, c], dt, split), _pieces(ok[:, :, c], dt, split)
        for t, (a, b) in enumerate(pairs):
            col = c * len(pairs) + t
            assert np.all(np.abs(gq[:, :, col] - qp[a]) <= _ulp(qp[a], dt))
            assert np.all(np.abs(gk[:, :, col] - kp[b]) <= _ulp(kp[b], dt))
    # the split factors reproduce m_h (j - i)
    rec = oracle.lowrank_bias(gq[:, :, :r], gk[:, :, :r])
    err = np.abs(rec - oracle.alibi_bias(oracle.alibi_slopes(H), N)).max()
    bound = {("f32", 1): 2e-3, ("bf16", 1): 20.0, ("f16", 1): 1.0, ("f16", 2): 1e-3, ("bf16", 3): 1e-3}[(dt, split)]
    say(f"  max |phi_q phi_k^T - b| = {err:.3e}")
    assert err <= bound


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_sandwich_factor_kernel(fb, dt):
    N, C = 4096, 64
    say(f"sandwich factors dt={dt}")
    pq, pk, r = fb.fb_make_factors("sandwich", 1, N, C=C, dtype=tdtype(dt))
    assert r == C
    g = to_np(pq)[0]
    ref = round_exact(oracle.sandwich_factors(N, C), dt)
    assert np.all(np.abs(g - ref) <= _ulp(ref, dt))
    np.testing.assert_array_equal(to_np(pk), to_np(pq))


@pytest.mark.parametrize("kind,dt", [("alibi", "bf16"), ("alibi", "f32"), ("sandwich", "bf16"), ("sandwich", "f16")])
def test_dense_bias_kernel(fb, kind, dt):
    H, N, C = (4, 640, 0) if kind == "alibi" else (1, 1000, 64)
    say(f"dense bias {kind} {dt}")
    b = fb.fb_make_dense_bias(kind, H, N, C=C, dtype=tdtype(dt))
    ref = oracle.alibi_bias(oracle.alibi_slopes(H), N) if kind == "alibi" else oracle.sandwich_bias(N, C)[None]
    ref = round_exact(ref, dt)
    got = to_np(b)
    assert np.all(np.abs(got - ref) <= _ulp(ref, dt))


# --------------------------------------------------------------- attention ---
REDUCED = [
    ("tiny_alibi_f32", {}),
    ("gpt2_alibi_causal", dict(B=2, H=3, N=300)),
    ("gpt2_alibi_causal", dict(B=1, H=12, N=2048 - 37, causal=False)),
    ("sandwich", dict(B=1, H=2, N=520)),
    ("vision_svd", dict(B=1, H=2, grid=20)),
    ("pairformer_svd", dict(B=4, H=2, N=200)),
]


@pytest.mark.parametrize("name,over", REDUCED, ids=[f"{n}-{i}" for i, (n, _) in enumerate(REDUCED)])
def test_attention_parity_reduced(fb, name, over):
    """Every output element at sizes spanning several tiles with a ragged tail."""
    w = synth.workload(name, **over)
    say(f"parity {w}")
    c = Case(w)
    import torch
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o = c.run_lowrank(lse=lse)
    torch.cuda.synchronize()
    ro, rl = c.reference()
    assert_close(to_np(o), ro, w.dtype, f"{name} O")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2 if w.dtype != "f32" else 1e-4)


LOG2 = [x for x in REDUCED if synth.workload(x[0], **x[1]).dtype != "f32"]


@pytest.mark.parametrize("name,over", LOG2, ids=[f"{n}-{i}" for i, (n, _) in enumerate(LOG2)])
def test_log2_factors_parity_reduced(fb, name, over):
    """fb_attn_fwd_lowrank_log2 with phi_q in exp2 units (fb_make_factors_log2 for the exact
    biases): every output element and LSE against the oracle, to the same bars."""
    w = synth.workload(name, **over)
    say(f"log2 parity {w}")
    c = Case(w, log2=True)
    import torch
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o = c.run_lowrank(lse=lse)
    torch.cuda.synchronize()
    ro, rl = c.reference()
    assert_close(to_np(o), ro, w.dtype, f"{name} log2 O")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2)


@pytest.mark.parametrize("kind,dt,split", [("sandwich", "f16", 1), ("alibi", "f16", 2), ("alibi", "bf16", 3)])
def test_log2_factor_kernel(fb, kind, dt, split):
    """fb_make_factors_log2: phi_q is the exact factor times log2(e), split and rounded like
    fb_make_factors; phi_k is fb_make_factors' phi_k."""
    H, N = (3, 700) if kind == "alibi" else (1, 1000)
    say(f"log2 factors {kind} {dt} split={split}")
    args = dict(C=64) if kind == "sandwich" else {}
    q2, k2, r = fb.fb_make_factors_log2(kind, H, N, dtype=tdtype(dt), split=split, **args)
    q1, k1, _ = fb.fb_make_factors(kind, H, N, dtype=tdtype(dt), split=split, **args)
    np.testing.assert_array_equal(to_np(k2), to_np(k1))
    if kind == "sandwich":
        ref = oracle.sandwich_factors(N, 64)[None] / np.log(2.0)
        assert np.all(np.abs(to_np(q2) - round_exact(ref, dt)) <= _ulp(ref, dt))
    # the pieces' products reproduce log2(e) b
    b = oracle.alibi_bias(oracle.alibi_slopes(H), N) if kind == "alibi" else oracle.sandwich_bias(N, 64)[None]
    rec = oracle.lowrank_bias(to_np(q2)[:, :, :r], to_np(k2)[:, :, :r]) * np.log(2.0)
    rec1 = oracle.lowrank_bias(to_np(q1)[:, :, :r], to_np(k1)[:, :, :r])
    e2, e1 = np.abs(rec - b).max(), np.abs(rec1 - b).max()
    say(f"  max |ln2 phi_q phi_k^T - b| = {e2:.3e} (fb_make_factors: {e1:.3e})")
    assert e2 <= 2 * e1 + 1e-6


def test_svd_approximation_error_reported(fb):
    """For SVD workloads the rank-R factors are an approximation: report it (not a bar)."""
    w = synth.workload("pairformer_svd", B=2, H=2, N=256)
    c = Case(w)
    import torch
    o = c.run_lowrank()
    torch.cuda.synchronize()
    full, _ = oracle.attention(c.q, c.k, c.v, bias=c.bias_full, causal=False)
    ma, rl = errors(to_np(o), full)
    fro = [oracle.bias_energy(c.bias_full[h], c.pq_np[h], c.pk_np[h])["rel_fro"] for h in range(w.H)]
    say(f"  vs full bias: max-abs {ma:.3e} rel-L2 {rl:.3e}; bias rel-Frobenius {np.round(fro, 5).tolist()}")
    assert np.isfinite(ma)


# ----------------------------------------------------------- cross kernel ----
@pytest.mark.parametrize("name,over", [("sandwich", dict(B=1, H=2, N=333)),
                                       ("gpt2_alibi_causal", dict(B=1, H=4, N=257)),
                                       ("tiny_alibi_f32", dict(N=200))])
def test_densebias_kernel_parity(fb, name, over):
    """The dense-bias baseline against the oracle fed the same rounded dense bias (the
    oracle's closed form, rounded once to the input dtype on the host, is both sides' input)."""
    import torch
    w = synth.workload(name, **over)
    say(f"densebias parity {w}")
    c = Case(w)
    if w.bias == "alibi":
        bnp = round_exact(oracle.alibi_bias(oracle.alibi_slopes(w.H), w.N), w.dtype)
    else:
        bnp = round_exact(oracle.sandwich_bias(w.N, w.C), w.dtype)
    o = fb.fb_attn_fwd_densebias(c.qd, c.kd, c.vd, to_dev(bnp, w.dtype), causal=w.causal)
    torch.cuda.synchronize()
    ro, _ = oracle.attention(c.q, c.k, c.v, bias=bnp, causal=w.causal)
    assert_close(to_np(o), ro, w.dtype, f"densebias {name}")


def test_lowrank_and_densebias_on_same_factors(fb):
    """Both kernels on one SVD bias: the low-rank kernel against the oracle with
    b = phi_q phi_k^T, the dense kernel against the oracle with that b rounded to bf16
    (its input), and the two outputs differ only by that rounding of b."""
    import torch
    w = synth.workload("vision_svd", B=1, H=2, grid=16)
    c = Case(w)
    o1 = c.run_lowrank()
    dense_np = round_exact(oracle.lowrank_bias(c.pq_np, c.pk_np), "bf16")   # [H, N, N], rounded once
    o2 = fb.fb_attn_fwd_densebias(c.qd, c.kd, c.vd, to_dev(dense_np, "bf16"))
    torch.cuda.synchronize()
    ro1, _ = c.reference()
    ro2, _ = oracle.attention(c.q, c.k, c.v, bias=dense_np)
    assert_close(to_np(o1), ro1, "bf16", "lowrank vs oracle(phi_q phi_k^T)")
    assert_close(to_np(o2), ro2, "bf16", "densebias vs oracle(bf16(phi_q phi_k^T))")
    ma, rl = errors(to_np(o1), to_np(o2))
    mo, ro = errors(ro1, ro2)
    say(f"  kernel difference {ma:.3e}/{rl:.3e}; oracle difference from rounding b: {mo:.3e}/{ro:.3e}")
    assert ma <= mo + 2e-2


def test_rank0_equals_densebias_zero(fb):
    import torch
    w = synth.workload("sandwich", B=2, H=2, N=300)
    c = Case(w)
    o1 = fb.fb_attn_fwd_lowrank(c.qd, c.kd, c.vd)
    zero = torch.zeros((w.N, w.N), dtype=torch.bfloat16, device="cuda:0")
    o2 = fb.fb_attn_fwd_densebias(c.qd, c.kd, c.vd, zero)
    torch.cuda.synchronize()
    # Same scores and the same rounded P; the two modes form the softmax denominator
    # differently (low rank: sum of the rounded P on the matrix core; dense bias: fp32 sum
    # before rounding), a relative difference far below bf16 resolution, so the outputs
    # agree to one bf16 ulp.
    a, b = to_np(o1).astype(np.float64), to_np(o2).astype(np.float64)
    assert np.all(np.abs(a - b) <= _ulp(np.maximum(np.abs(a), np.abs(b)), "bf16"))
    ro, _ = oracle.attention(c.q, c.k, c.v)
    assert_close(to_np(o1), ro, "bf16", "R=0")
    # plain attention in the exp2 form (the log2 entry point without factors)
    o3 = fb.fb_attn_fwd_lowrank_log2(c.qd, c.kd, c.vd)
    torch.cuda.synchronize()
    assert_close(to_np(o3), ro, "bf16", "R=0, exp2 form")


# -------------------------------------------------------------- edge cases ---
@pytest.mark.parametrize("N", [1, 17, 129])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes(fb, N, D, causal):
    import torch
    r = np.random.default_rng(N * 1000 + D + causal)
    B, H, R = 2, 3, 5
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(3))
    pq = synth.round_to(r.standard_normal((H, N, R)), "f16")
    pk = synth.round_to(r.standard_normal((H, N, R)), "f16")
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               to_dev(pq, "f16"), to_dev(pk, "f16"), causal=causal)
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk), causal=causal)
    assert_close(to_np(o), ro, "bf16", f"N={N} D={D} causal={causal}")
    # the exp2-unit kernel on the same shapes, phi_q times log2(e) rounded once to f16
    pq2 = round_exact(pq / np.log(2.0), "f16")
    o2 = fb.fb_attn_fwd_lowrank_log2(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                     to_dev(pq2, "f16"), to_dev(pk, "f16"), causal=causal)
    torch.cuda.synchronize()
    ro2, _ = oracle.attention(q, k, v, bias=np.log(2.0) * oracle.lowrank_bias(pq2, pk), causal=causal)
    assert_close(to_np(o2), ro2, "bf16", f"exp2 units N={N} D={D} causal={causal}")


@pytest.mark.parametrize("R,phi", [(0, "f16"), (3, "bf16"), (16, "f16"), (20, "f16"), (48, "bf16"), (64, "f16"),
                                   (100, "f16"), (128, "bf16")])
def test_ranks(fb, R, phi):
    import torch
    r = np.random.default_rng(R)
    B, H, N, D = 1, 2, 160, 64
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(3))
    pq = synth.round_to(r.standard_normal((B, H, N, R)) * 0.3, phi)
    pk = synth.round_to(r.standard_normal((B, H, N, R)) * 0.3, phi)
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               to_dev(pq, phi), to_dev(pk, phi))
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(o), ro, "bf16", f"R={R} {phi}")
    pq2 = round_exact(pq / np.log(2.0), phi)
    o2 = fb.fb_attn_fwd_lowrank_log2(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                     to_dev(pq2, phi), to_dev(pk, phi))
    torch.cuda.synchronize()
    ro2, _ = oracle.attention(q, k, v, bias=np.log(2.0) * oracle.lowrank_bias(pq2, pk))
    assert_close(to_np(o2), ro2, "bf16", f"exp2 units R={R} {phi}")


@pytest.mark.parametrize("R", [1, 2, 4, 7, 32])
def test_ranks_fp32(fb, R):
    import torch
    r = np.random.default_rng(100 + R)
    B, H, N, D = 1, 2, 150, 32
    q, k, v = (r.standard_normal((B, H, N, D)).astype(np.float32).astype(np.float64) for _ in range(3))
    pq = r.standard_normal((H, N, R)).astype(np.float32).astype(np.float64)
    pk = r.standard_normal((H, N, R)).astype(np.float32).astype(np.float64)
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"),
                               to_dev(pq, "f32"), to_dev(pk, "f32"))
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(o), ro, "f32", f"fp32 R={R}")


def test_per_batch_dynamic_factors(fb):
    """Factors that change with the batch element but are shared by the heads ([B,1,N,R],
    head stride 0): the shape a per-sample factor network would feed."""
    import torch
    r = np.random.default_rng(31)
    B, H, N, D, R = 3, 4, 200, 64, 24
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(3))
    pq = synth.round_to(r.standard_normal((B, 1, N, R)) * 0.4, "f16")
    pk = synth.round_to(r.standard_normal((B, 1, N, R)) * 0.4, "f16")
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               to_dev(pq, "f16"), to_dev(pk, "f16"))
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(o), ro, "bf16", "per-batch factors")


def test_energy_selected_ranks_per_head(fb):
    """Per-head rank chosen for 95% energy on the host, factors from the host SVD at that
    rank, zero-padded to the largest rank of the call; the kernel matches the oracle run on
    the same factors, and the approximation error against the full bias is reported."""
    import torch
    w = synth.workload("vision_svd", grid=16, B=1, H=3)
    inp = synth.make_inputs(w)
    bias = inp["bias_src"]                                     # [H, N, N] fp64
    H, N = bias.shape[0], bias.shape[1]
    sel = [fb.fb_svd_rank_for_energy(bias[h], 0.95, R_max=48, seed=h) for h in range(H)]
    Rp = max(x["R"] for x in sel)
    pq = np.zeros((H, N, Rp))
    pk = np.zeros((H, N, Rp))
    for h in range(H):
        f = fb.fb_svd_factors(bias[h], sel[h]["R"], seed=h)
        pq[h, :, :sel[h]["R"]] = f["phi_q"]
        pk[h, :, :sel[h]["R"]] = f["phi_k"]
    pq, pk = synth.round_to(pq, "f16"), synth.round_to(pk, "f16")
    r = np.random.default_rng(32)
    q, k, v = (synth.round_to(r.standard_normal((1, H, N, w.D)) * 0.5, "bf16") for _ in range(3))
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               to_dev(pq, "f16"), to_dev(pk, "f16"))
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(o), ro, "bf16", f"energy-selected ranks {[x['R'] for x in sel]}")
    rf, _ = oracle.attention(q, k, v, bias=bias)
    say(f"ranks {[x['R'] for x in sel]} energy {[round(x['energy'], 4) for x in sel]}: "
        f"output vs full bias max-abs {np.abs(to_np(o) - rf).max():.3e}")
    assert all(x["reached"] and x["energy"] >= 0.95 for x in sel)


def test_strided_inputs_and_broadcast_factors(fb):
    """Q/K/V as views into wider / permuted buffers; factors broadcast over batch and heads."""
    import torch
    r = np.random.default_rng(7)
    B, H, N, D, R = 2, 3, 190, 64, 16
    big = to_dev(synth.round_to(r.standard_normal((B, N, H, 3 * D + 8)) * 0.5, "bf16"), "bf16")
    qd = big[..., 0:D].permute(0, 2, 1, 3)               # [B,H,N,D] with row stride 3D+8... -> multiple of 8
    kd = big[..., D:2 * D].permute(0, 2, 1, 3)
    vd = big[..., 2 * D:3 * D].permute(0, 2, 1, 3)
    pq = synth.round_to(r.standard_normal((N, R)) * 0.4, "f16")
    pk = synth.round_to(r.standard_normal((N, R)) * 0.4, "f16")
    out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda:0").permute(0, 2, 1, 3)
    fb.fb_attn_fwd_lowrank(qd, kd, vd, to_dev(pq, "f16"), to_dev(pk, "f16"), out=out)
    torch.cuda.synchronize()
    qn, kn, vn = (to_np(x) for x in (qd, kd, vd))
    ro, _ = oracle.attention(qn, kn, vn, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(out), ro, "bf16", "strided + broadcast")


def test_resident_strided_inputs_and_broadcast_factors(fb, monkeypatch):
    """The resident kernel's copies and stores on strided views: Q/K/V as permuted views into one
    packed buffer, a permuted output view, factors broadcast over batch and heads, LSE too;
    compared with the oracle through both kernels."""
    import torch
    r = np.random.default_rng(8)
    B, H, N, D, R = 3, 2, 300, 32, 16
    big = to_dev(synth.round_to(r.standard_normal((B, N, H, 3 * D + 8)) * 0.5, "bf16"), "bf16")
    qd, kd, vd = (big[..., i * D:(i + 1) * D].permute(0, 2, 1, 3) for i in range(3))
    pq = synth.round_to(r.standard_normal((N, R)) * 0.6, "f16")
    pk = synth.round_to(r.standard_normal((N, R)) * 0.6, "f16")
    qn, kn, vn = (to_np(x) for x in (qd, kd, vd))
    ro, rl = oracle.attention(qn, kn, vn, bias=oracle.lowrank_bias(pq, pk) * np.log(2.0))
    for streaming in (False, True):
        if streaming:
            monkeypatch.setenv("FB_ATTN_STREAMING", "1")
        out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device="cuda:0").permute(0, 2, 1, 3)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        fb.fb_attn_fwd_lowrank_log2(qd, kd, vd, to_dev(pq, "f16"), to_dev(pk, "f16"), out=out, lse=lse)
        torch.cuda.synchronize()
        what = "streaming" if streaming else "resident"
        assert_close(to_np(out), ro, "bf16", f"{what} strided + broadcast")
        np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2, err_msg=f"{what} LSE")
    monkeypatch.delenv("FB_ATTN_STREAMING")


def test_unaligned_factor_rows(fb):
    """Factor rows that are not 16-byte aligned take the element-wise load path."""
    import torch
    r = np.random.default_rng(8)
    B, H, N, D, R = 1, 2, 100, 32, 9
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(3))
    pq = synth.round_to(r.standard_normal((H, N, R)), "f16")
    pk = synth.round_to(r.standard_normal((H, N, R)), "f16")
    pqd = to_dev(pq, "f16")                                # row stride 9 elements: unaligned rows
    pkd = to_dev(pk, "f16")
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), pqd, pkd)
    torch.cuda.synchronize()
    ro, _ = oracle.attention(q, k, v, bias=oracle.lowrank_bias(pq, pk))
    assert_close(to_np(o), ro, "bf16", "unaligned factors")


def test_degenerate_bias_cases(fb):
    """A bias that dominates one key (+40 on key 5) routes every row to v_5; a constant
    V gives a constant output."""
    import torch
    r = np.random.default_rng(9)
    B, H, N, D = 1, 1, 96, 32
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(3))
    pq = np.ones((N, 1))
    pk = np.zeros((N, 1))
    pk[5, 0] = 40.0
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(pq, "f16"),
                               to_dev(pk, "f16"))
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(o)[0, 0], np.broadcast_to(v[0, 0, 5], (N, D)), rtol=0, atol=1e-2)
    vc = np.broadcast_to(synth.round_to(r.standard_normal(D), "bf16"), (B, H, N, D)).copy()
    o = fb.fb_attn_fwd_lowrank(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(vc, "bf16"))
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(o), vc, rtol=0, atol=1e-2)


def test_empty_batch_is_noop(fb):
    import torch
    q = torch.empty((0, 2, 64, 64), dtype=torch.bfloat16, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == q.shape


def test_deterministic(fb):
    import torch
    w = synth.workload("sandwich", B=1, H=2, N=700)
    c = Case(w)
    o1 = c.run_lowrank()
    o2 = c.run_lowrank()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---------------------------------------------------- multiplicative bias ---
MUL = [
    # (shape, R, dtype, factor dtype, causal, factors)
    (dict(B=2, H=3, N=300, D=64), 2, "bf16", "f32", False, "cos"),
    (dict(B=1, H=2, N=200, D=32), 3, "bf16", "bf16", True, "rand"),
    (dict(B=1, H=2, N=129, D=32), 5, "f16", "f16", False, "rand"),
    (dict(B=1, H=2, N=257, D=16), 9, "bf16", "f16", True, "rand"),
    (dict(B=2, H=2, N=100, D=128), 2, "bf16", "bf16", False, "rand"),
    (dict(B=1, H=2, N=150, D=64), 1, "bf16", "f32", False, "rand"),
]


@pytest.mark.parametrize("shape,R,dt,pdt,causal,kind", MUL, ids=[f"mul-{i}" for i in range(len(MUL))])
def test_mulbias_parity(fb, shape, R, dt, pdt, causal, kind):
    """Multiplicative low-rank bias through operand expansion: every output element and the
    LSE against the oracle's element-wise definition with the same (rounded) factors."""
    import torch
    B, H, N, D = shape["B"], shape["H"], shape["N"], shape["D"]
    r = np.random.default_rng(500 + N + R)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    if kind == "cos":
        pq = pk = synth.round_to(oracle.cos_mulbias_factors(N), pdt)
    else:
        pq = synth.round_to(r.standard_normal((H, N, R)) * 0.7, pdt)
        pk = synth.round_to(r.standard_normal((H, N, R)) * 0.7, pdt)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_mulbias(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(pq, pdt), to_dev(pk, pdt),
                               causal=causal, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_mulbias(q, k, v, oracle.lowrank_bias(pq, pk), causal=causal)
    assert_close(to_np(o), ro, dt, f"mulbias R={R} D={D} {kind}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2)


def test_mulbias_strided_inputs_and_reused_workspace(fb):
    """Q/K as permuted views, per-(b, h) factors, and one workspace reused by two calls."""
    import torch
    r = np.random.default_rng(510)
    B, H, N, D, R = 2, 2, 170, 32, 3
    big = to_dev(synth.round_to(r.standard_normal((B, N, H, 2 * D)) * 0.5, "bf16"), "bf16")
    qd = big[..., :D].permute(0, 2, 1, 3)
    kd = big[..., D:].permute(0, 2, 1, 3)
    v = synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16")
    ws = torch.empty(fb.fb_mulbias_workspace_bytes(qd, R) + 256, dtype=torch.uint8, device="cuda:0")
    outs = []
    for t in range(2):
        pq = synth.round_to(r.standard_normal((B, H, N, R)) * 0.6, "f16")
        pk = synth.round_to(r.standard_normal((B, H, N, R)) * 0.6, "f16")
        o = fb.fb_attn_fwd_mulbias(qd, kd, to_dev(v, "bf16"), to_dev(pq, "f16"), to_dev(pk, "f16"), workspace=ws)
        torch.cuda.synchronize()
        ro, _ = oracle.attention_mulbias(to_np(qd), to_np(kd), v, oracle.lowrank_bias(pq, pk))
        assert_close(to_np(o), ro, "bf16", f"mulbias strided call {t}")


def test_mulbias_two_stage_equals_one_call(fb):
    """Expansion stage + the low-rank kernel on its outputs gives bit-identical results to
    the one-call entry point (the benchmark times the two stages separately)."""
    import torch
    r = np.random.default_rng(520)
    B, H, N, D, R = 2, 2, 300, 64, 3
    q, k, v = (to_dev(synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16"), "bf16") for _ in range(3))
    pq = to_dev(synth.round_to(r.standard_normal((N, R)), "f32"), "f32")
    pk = to_dev(synth.round_to(r.standard_normal((N, R)), "f32"), "f32")
    o1 = fb.fb_attn_fwd_mulbias(q, k, v, pq, pk)
    e = fb.fb_mulbias_expand(q, k, pq, pk)
    o2 = fb.fb_attn_fwd_lowrank(e["q1"], e["k1"], v, e["phi_q"], e["phi_k"], scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    s = 1.0 / np.sqrt(D)
    q1 = (q.double() * pq.double()[:, 0][None, None, :, None] * s)
    np.testing.assert_allclose(to_np(e["q1"]), to_np(q1), rtol=2 ** -8, atol=0)


# ------------------------------------------------------------------- backward ---
def _sum_to(x: np.ndarray, shape) -> np.ndarray:
    """Sum a [B, H, N, R] gradient over the axes a factor of ``shape`` is broadcast on."""
    shape = tuple(shape)
    full = (1,) * (4 - len(shape)) + shape
    for ax in range(4):
        if full[ax] == 1 and x.shape[ax] != 1:
            x = x.sum(axis=ax, keepdims=True)
    return x.reshape(shape)


BWD = [
    # (B, H, N, D, R, factor shape, dtype, factor dtype, causal)
    (2, 2, 300, 64, 0, None, "bf16", "bf16", False),
    (1, 2, 257, 64, 0, None, "bf16", "bf16", True),
    (2, 2, 200, 64, 64, "shared", "bf16", "f16", False),
    (1, 3, 190, 32, 16, "head", "bf16", "bf16", True),
    (2, 2, 160, 32, 24, "full", "f16", "f16", False),
    (1, 2, 130, 64, 8, "head", "bf16", "f16", True),
    # one tile; fewer rows than one MFMA block; many tiles through the three-buffer rotation
    (1, 1, 64, 64, 16, "shared", "bf16", "f16", True),
    (1, 2, 17, 32, 8, "shared", "f16", "f16", False),
    (1, 1, 1000, 64, 64, "shared", "bf16", "f16", True),
    # a per-head factor shared over three batches: gradient summed over the batch axis only
    (3, 2, 150, 64, 16, "head", "bf16", "f16", False),
    # R not a multiple of 8: the library pads the factors in its workspace (exact ALiBi rank 2,
    # its split f16 pieces R' = 6, and wider ranks), every factor shape
    (2, 3, 210, 64, 2, "head", "bf16", "f16", True),
    (2, 2, 180, 64, 6, "shared", "bf16", "f16", True),
    (1, 2, 140, 32, 20, "full", "f16", "f16", False),
    (2, 2, 260, 64, 60, "shared", "bf16", "bf16", False),
    (3, 1, 100, 32, 3, "head", "bf16", "f16", False),
    # head dim 16 (run in the head-dim-32 layout with zero operands past 16)
    (2, 2, 230, 16, 8, "head", "bf16", "f16", False),
    (1, 3, 140, 16, 0, None, "f16", "f16", True),
    (2, 1, 100, 16, 6, "shared", "bf16", "f16", True),
    # head dim 128 (one workgroup per compute unit)
    (2, 2, 200, 128, 0, None, "bf16", "bf16", False),
    (1, 2, 260, 128, 64, "shared", "bf16", "f16", True),
    (2, 1, 150, 128, 16, "head", "f16", "f16", False),
    (1, 2, 130, 128, 6, "full", "bf16", "f16", True),
]


@pytest.mark.parametrize("B,H,N,D,R,fs,dt,pdt,causal", BWD, ids=[f"bwd-{i}" for i in range(len(BWD))])
def test_backward_parity(fb, B, H, N, D, R, fs, dt, pdt, causal):
    """dQ, dK, dV and the factor gradients against the oracle's chain rule (fp64) on the
    same rounded inputs; the forward output and LSE come from the fused forward."""
    import torch
    r = np.random.default_rng(700 + N + R)
    q, k, v, do = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(4))
    shape = {"shared": (N, R), "head": (H, N, R), "full": (B, H, N, R)}.get(fs)
    pq = pk = None
    if R:
        pq = synth.round_to(r.standard_normal(shape) * 0.4, pdt)
        pk = synth.round_to(r.standard_normal(shape) * 0.4, pdt)
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    pqd = to_dev(pq, pdt) if R else None
    pkd = to_dev(pk, pdt) if R else None
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal)
    torch.cuda.synchronize()
    bias = oracle.lowrank_bias(pq, pk) if R else None
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=causal)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_grad_close(to_np(got), ref, f"{name} R={R} D={D} {dt}")
    if R:
        full_q = np.broadcast_to(pq, (B, H, N, R)) if pq.ndim < 4 else pq
        full_k = np.broadcast_to(pk, (B, H, N, R)) if pk.ndim < 4 else pk
        rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
        assert_grad_close(gpq.cpu().double().numpy(), _sum_to(rgq, shape), f"dphi_q R={R}")
        assert_grad_close(gpk.cpu().double().numpy(), _sum_to(rgk, shape), f"dphi_k R={R}")


# fp32 Q/K/V and factors: the fp32 matrix-core kernels (any R up to 64, factors read in place).
# Their arithmetic is fp32 throughout (products, accumulation, exp2 of the recomputed scores
# against the fp32 LSE), so the bar is that of fp32 rounding over contractions of a few
# hundred terms: relative L2 <= 2e-5 and max-abs <= 2e-4 of the largest reference entry.
BWD_F32 = [
    # (B, H, N, D, R, factor shape, causal); the tiny ALiBi configuration first (B1 H2 N128 D32
    # with the exact ALiBi factors, rank 2 padded to 4 columns)
    (1, 2, 128, 32, "alibi", "head", False),
    (2, 3, 150, 64, 5, "full", True),
    (1, 2, 200, 16, 0, None, False),
    (2, 2, 100, 32, 16, "shared", True),
    (1, 1, 70, 64, 32, "head", False),
    (3, 2, 90, 16, 7, "head", True),
]
F32_GRAD_TOL = (2e-5, 2e-4)


def _assert_f32_grad(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    ma, rl = errors(got, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    say(f"  {what}: rel-L2 {rl:.3e}, max-abs/max|ref| {ma / scale:.3e}")
    assert rl <= F32_GRAD_TOL[0] and ma / scale <= F32_GRAD_TOL[1], f"{what}: rel-L2 {rl:.3e}, max-abs {ma:.3e}"


@pytest.mark.parametrize("B,H,N,D,R,fs,causal", BWD_F32, ids=[f"bwdf32-{i}" for i in range(len(BWD_F32))])
def test_backward_fp32(fb, B, H, N, D, R, fs, causal):
    """fp32 backward on the fp32 forward's own output and LSE: dQ, dK, dV and the factor
    gradients against the oracle's chain rule (fp64)."""
    import torch
    r = np.random.default_rng(900 + N + D)
    q, k, v, do = (r.standard_normal((B, H, N, D)).astype(np.float32).astype(np.float64) * 0.5 for _ in range(4))
    if R == "alibi":
        pqd, pkd, _ = fb.fb_make_factors("alibi", H, N, dtype=torch.float32)
        pq, pk = to_np(pqd), to_np(pkd)
        R, shape = pq.shape[-1], pq.shape
    else:
        shape = {"shared": (N, R), "head": (H, N, R), "full": (B, H, N, R)}.get(fs)
        pq = r.standard_normal(shape).astype(np.float32).astype(np.float64) * 0.4 if R else None
        pk = r.standard_normal(shape).astype(np.float32).astype(np.float64) * 0.4 if R else None
        pqd = to_dev(pq, "f32") if R else None
        pkd = to_dev(pk, "f32") if R else None
    say(f"fp32 backward B={B} H={H} N={N} D={D} R={R} {fs} causal={causal}")
    qd, kd, vd, dod = (to_dev(x, "f32") for x in (q, k, v, do))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal)
    torch.cuda.synchronize()
    bias = oracle.lowrank_bias(pq, pk) if R else None
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=causal)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        _assert_f32_grad(to_np(got), ref, f"{name} fp32 R={R} D={D}")
    if R:
        full_q = np.broadcast_to(pq, (B, H, N, R)) if pq.ndim < 4 else pq
        full_k = np.broadcast_to(pk, (B, H, N, R)) if pk.ndim < 4 else pk
        rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
        _assert_f32_grad(gpq.cpu().double().numpy(), _sum_to(rgq, shape), f"dphi_q fp32 R={R}")
        _assert_f32_grad(gpk.cpu().double().numpy(), _sum_to(rgk, shape), f"dphi_k fp32 R={R}")


def test_backward_fp32_rank64(fb):
    """Rank 64 with fp32 factors (the fp32 forward stops at rank 32): the backward given the
    oracle's forward output and LSE, rounded to fp32, against the oracle's gradients."""
    import torch
    B, H, N, D, R = 1, 2, 150, 64, 64
    r = np.random.default_rng(990)
    q, k, v, do = (r.standard_normal((B, H, N, D)).astype(np.float32).astype(np.float64) * 0.5 for _ in range(4))
    pq, pk = (r.standard_normal((N, R)).astype(np.float32).astype(np.float64) * 0.3 for _ in range(2))
    bias = oracle.lowrank_bias(pq, pk)
    ro, rl = oracle.attention(q, k, v, bias=bias, causal=True)
    o32 = ro.astype(np.float32).astype(np.float64)
    qd, kd, vd, dod, od = (to_dev(x, "f32") for x in (q, k, v, do, o32))
    lse = torch.from_numpy(rl.astype(np.float32)).to("cuda:0")
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, od, lse, dod, to_dev(pq, "f32"), to_dev(pk, "f32"),
                                                  causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=True)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        _assert_f32_grad(to_np(got), ref, f"{name} fp32 R=64")
    rgq, rgk = oracle.lowrank_factor_grads(db, np.broadcast_to(pq, (B, H, N, R)), np.broadcast_to(pk, (B, H, N, R)))
    _assert_f32_grad(gpq.cpu().double().numpy(), _sum_to(rgq, (N, R)), "dphi_q fp32 R=64")
    _assert_f32_grad(gpk.cpu().double().numpy(), _sum_to(rgk, (N, R)), "dphi_k fp32 R=64")


def test_backward_full_size_sampled(fb):
    """The Sandwich workload at full size (B4 H8 N4096 D64, R = 64 f16 factors shared by all
    (b, h)) in the benchmark's launch, the backward alone: every gradient element of two
    (b, h) pairs, given the oracle's forward output, and the factor gradients through a
    per-(b, h) view of the same factors.  (The backward on its own forward's output is
    covered over every (b, h) in the full-size tests.)"""
    import torch
    w = synth.workload("sandwich")
    inp = synth.make_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    r = np.random.default_rng(20260013)
    do = synth.round_to(r.standard_normal(q.shape) * 0.5, "bf16")
    # the oracle's Sandwich factors rounded once to f16: both sides' input
    pq = pk = round_exact(oracle.sandwich_factors(w.N, w.C), "f16")
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    phd = to_dev(pq, "f16")
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, phd, phd, lse=lse)
    torch.cuda.synchronize()
    # The row term Delta = rowsum(dO * O) reads the stored forward output.  For the sampled
    # pairs both sides take the oracle's O rounded to bf16 and its LSE, so the check measures
    # the backward alone: dphi = dS phi cancels for the smooth low-frequency Sandwich columns
    # (sum_j dS_ij = 0), and an error e in Delta_i moves dphi_i by about e |phi| while the
    # result itself is of size |phi| |dP - Delta| sqrt(sum_j P_ij^2), some sqrt(N) smaller, so
    # the forward's own rounding of O would swamp the comparison.
    bias = oracle.lowrank_bias(pq, pk)
    pairs = [(0, 0), (3, 7)]
    refs = {}
    for (b, h) in pairs:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle.attention(q[sl], k[sl], v[sl], bias=bias)
        o_16 = round_exact(o_ref, "bf16")
        o[b, h] = torch.from_numpy(o_16[0, 0]).to(o.dtype).to(o.device)
        lse[b, h] = torch.from_numpy(l_ref[0, 0]).float().to(lse.device)
        refs[(b, h)] = o_16
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, to_dev(do, "bf16"), phd, phd)
    # the same factors as a [B, H, N, R] view (0 strides): the factor gradients then come per
    # (b, h), written directly, so single pairs can be compared with the oracle
    shape4 = (w.B, w.H, w.N, phd.shape[-1])
    _, _, _, gpq4, gpk4 = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, to_dev(do, "bf16"),
                                                 phd.expand(shape4), phd.expand(shape4))
    torch.cuda.synchronize()
    for (b, h) in pairs:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv, db = oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], bias=bias,
                                                   o_stored=refs[(b, h)])
        for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            assert_grad_close(to_np(got[b:b + 1, h:h + 1]), ref, f"full-size {name} b={b} h={h}")
        rgq, rgk = oracle.lowrank_factor_grads(db[0, 0], pq, pk)
        # Beyond the common gradient bar: the same cancellation leaves the 16-bit rounding of dS
        # visible against dphi_q, so its error is also held against the uncancelled size
        # M_ic = sqrt(sum_j (dS_ij phi_jc)^2).  f16 rounding of dS (relative half-ulp 2^-11)
        # gives |err|_F of about 2^-11 / sqrt(3) |M|_F; allowed 2^-9
        for name, got, ref, A, F in (("dphi_q", gpq4, rgq, db[0, 0], pk), ("dphi_k", gpk4, rgk, db[0, 0].T, pq)):
            g = got[b, h].double().cpu().numpy()
            assert_grad_close(g, ref, f"full-size {name} b={b} h={h}")
            M = np.sqrt((A ** 2) @ (F ** 2))
            ratio = np.linalg.norm(g - ref) / np.linalg.norm(M)
            say(f"  full-size {name} b={b} h={h}: |err|_F / |M|_F {ratio:.3e} (<= {2.0 ** -9:.3e})")
            assert ratio <= 2.0 ** -9, name
    # the factor gradients summed over all (b, h) equal the per-(b, h) ones added up (the same
    # fp32 partials in another order)
    for name, g, g4 in (("dphi_q", gpq, gpq4), ("dphi_k", gpk, gpk4)):
        g = g.double().cpu().numpy()
        assert np.all(np.isfinite(g)), name
        host = g4.double().cpu().numpy().sum(axis=(0, 1))
        rl = float(np.linalg.norm(g - host) / np.linalg.norm(host))
        say(f"  summed {name} vs host sum of per-(b, h) gradients: rel-L2 {rl:.3e}")
        assert rl <= 1e-5, name


# ------------------------------------------------------- in-kernel ALiBi factors ---
JIT = [
    (dict(B=2, H=4, N=300, D=64), "bf16", False, None),
    (dict(B=1, H=3, N=257, D=32), "bf16", True, None),
    (dict(B=1, H=2, N=4500, D=64), "bf16", True, None),       # indices past 2048: split hi / lo
    (dict(B=1, H=2, N=200, D=16), "f16", False, None),
    (dict(B=1, H=2, N=190, D=128), "bf16", True, None),
    (dict(B=1, H=3, N=150, D=64), "bf16", False, [0.5, 0.1234567, 1.7]),   # slopes that f16 cannot hold
]


@pytest.mark.parametrize("shape,dt,causal,slopes", JIT, ids=[f"jit-{i}" for i in range(len(JIT))])
def test_alibi_in_kernel_factors(fb, shape, dt, causal, slopes):
    """ALiBi with the factors formed in the kernel against the oracle's closed-form bias."""
    import torch
    B, H, N, D = shape["B"], shape["H"], shape["N"], shape["D"]
    r = np.random.default_rng(800 + N + D)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    m = oracle.alibi_slopes(H) if slopes is None else np.asarray(slopes, dtype=np.float64)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_alibi(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), slopes=slopes, causal=causal, lse=lse)
    torch.cuda.synchronize()
    rows = None if N <= 600 else sample_rows(N, 64, seed=4)
    ro, rl = oracle.attention(q, k, v, bias=oracle.alibi_bias(m, N), causal=causal, rows=rows)
    got = to_np(o) if rows is None else to_np(o)[:, :, rows]
    assert_close(got, ro, dt, f"in-kernel ALiBi N={N} D={D}")
    gl = lse.cpu().double().numpy()
    np.testing.assert_allclose(gl if rows is None else gl[:, :, rows], rl, rtol=0, atol=2e-2)


# ---------------------------------------------------- in-kernel Sandwich factors ---
SWJIT = [
    # (B, H, N, D, C, dtype, causal, rows sampled)
    (1, 2, 520, 64, 64, "bf16", False, False),
    (2, 1, 300, 32, 32, "bf16", True, False),
    (1, 3, 200, 16, 16, "f16", False, False),
    (1, 1, 129, 64, 2, "bf16", True, False),
    (1, 2, 64, 64, 48, "f16", False, False),
    (1, 1, 12000, 64, 64, "bf16", True, True),     # key indices far past one tile table
]


@pytest.mark.parametrize("B,H,N,D,C,dt,causal,sampled", SWJIT, ids=[f"swjit-{i}" for i in range(len(SWJIT))])
def test_sandwich_in_kernel_factors(fb, B, H, N, D, C, dt, causal, sampled):
    """Sandwich with the cos / sin factors formed in the kernel (fb_attn_fwd_sandwich) against
    the oracle's bias from its defining sum of cosines: O and LSE."""
    import torch
    r = np.random.default_rng(1100 + N + C)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    say(f"in-kernel Sandwich B={B} H={H} N={N} D={D} C={C} {dt} causal={causal}")
    o = fb.fb_attn_fwd_sandwich(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), C=C, causal=causal, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, seed=6) if sampled else None
    ro, rl = oracle.attention(q, k, v, bias=oracle.sandwich_bias(N, C), causal=causal, rows=rows)
    got, gl = to_np(o), lse.cpu().double().numpy()
    if sampled:
        got, gl = got[:, :, rows], gl[:, :, rows]
    assert_close(got, ro, dt, f"in-kernel Sandwich N={N} C={C}")
    np.testing.assert_allclose(gl, rl, rtol=0, atol=2e-2)


# ------------------------------------------------------- seeded random sweep ----
def _sweep_configs(n=16, seed=20260200):
    """Small random configurations across the supported space (shapes, ranks, factor
    shapes, dtypes, causal), drawn once from a fixed seed."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(r.choice([32, 64]))
        R = int(r.choice([0, 8, 16, 24, 40, 64]))
        N = int(r.integers(1, 330))
        B, H = int(r.integers(1, 4)), int(r.integers(1, 4))
        fs = str(r.choice(["shared", "head", "full"]))
        dt = str(r.choice(["bf16", "f16"]))
        pdt = "f16" if dt == "f16" else str(r.choice(["bf16", "f16"]))
        out.append((B, H, N, D, R, fs, dt, pdt, bool(r.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,H,N,D,R,fs,dt,pdt,causal", _sweep_configs(), ids=[f"sweep-{i}" for i in range(16)])
def test_random_sweep_forward_and_backward(fb, B, H, N, D, R, fs, dt, pdt, causal):
    """Forward output and LSE, then all gradients, against the oracle on the same rounded
    inputs, for a seeded random configuration."""
    import torch
    r = np.random.default_rng(900 + B * 1000 + H * 100 + N + R)
    q, k, v, do = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(4))
    shape = {"shared": (N, R), "head": (H, N, R), "full": (B, H, N, R)}[fs]
    pq = pk = None
    if R:
        pq = synth.round_to(r.standard_normal(shape) * 0.4, pdt)
        pk = synth.round_to(r.standard_normal(shape) * 0.4, pdt)
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    pqd = to_dev(pq, pdt) if R else None
    pkd = to_dev(pk, pdt) if R else None
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal)
    torch.cuda.synchronize()
    bias = oracle.lowrank_bias(pq, pk) if R else None
    ro, rl = oracle.attention(q, k, v, bias=bias, causal=causal)
    assert_close(to_np(o), ro, dt, f"O {B}x{H}x{N} D={D} R={R} {fs} {dt}/{pdt} causal={causal}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2)
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=causal)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_grad_close(to_np(got), ref, name)
    if R:
        full_q = np.broadcast_to(pq, (B, H, N, R)) if pq.ndim < 4 else pq
        full_k = np.broadcast_to(pk, (B, H, N, R)) if pk.ndim < 4 else pk
        rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
        assert_grad_close(gpq.cpu().double().numpy(), _sum_to(rgq, shape), "dphi_q")
        assert_grad_close(gpk.cpu().double().numpy(), _sum_to(rgk, shape), "dphi_k")


def _sweep_configs_f32(n=8, seed=20260300):
    """The same for fp32 Q/K/V and factors (head dims 16-64; the fp32 forward takes ranks up
    to 32)."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(r.choice([16, 32, 64]))
        R = int(r.choice([0, 3, 8, 16, 32]))
        N = int(r.integers(1, 330))
        B, H = int(r.integers(1, 4)), int(r.integers(1, 4))
        fs = str(r.choice(["shared", "head", "full"]))
        out.append((B, H, N, D, R, fs, bool(r.integers(0, 2))))
    return out


@pytest.mark.parametrize("B,H,N,D,R,fs,causal", _sweep_configs_f32(), ids=[f"sweepf32-{i}" for i in range(8)])
def test_random_sweep_fp32(fb, B, H, N, D, R, fs, causal):
    """fp32 forward output and LSE, then all gradients, against the oracle (fp32 bars)."""
    import torch
    r = np.random.default_rng(950 + B * 1000 + H * 100 + N + R)
    q, k, v, do = (r.standard_normal((B, H, N, D)).astype(np.float32).astype(np.float64) * 0.5 for _ in range(4))
    shape = {"shared": (N, R), "head": (H, N, R), "full": (B, H, N, R)}[fs]
    pq = r.standard_normal(shape).astype(np.float32).astype(np.float64) * 0.4 if R else None
    pk = r.standard_normal(shape).astype(np.float32).astype(np.float64) * 0.4 if R else None
    qd, kd, vd, dod = (to_dev(x, "f32") for x in (q, k, v, do))
    pqd = to_dev(pq, "f32") if R else None
    pkd = to_dev(pk, "f32") if R else None
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal)
    torch.cuda.synchronize()
    bias = oracle.lowrank_bias(pq, pk) if R else None
    ro, rl = oracle.attention(q, k, v, bias=bias, causal=causal)
    assert_close(to_np(o), ro, "f32", f"O fp32 {B}x{H}x{N} D={D} R={R} {fs} causal={causal}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=1e-4)
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=bias, causal=causal)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        _assert_f32_grad(to_np(got), ref, name)
    if R:
        full_q = np.broadcast_to(pq, (B, H, N, R)) if pq.ndim < 4 else pq
        full_k = np.broadcast_to(pk, (B, H, N, R)) if pk.ndim < 4 else pk
        rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
        _assert_f32_grad(gpq.cpu().double().numpy(), _sum_to(rgq, shape), "dphi_q")
        _assert_f32_grad(gpk.cpu().double().numpy(), _sum_to(rgk, shape), "dphi_k")


# ------------------------------------------- several work items per workgroup ----
# Non-causal 16-bit kernels with D + R_pad <= 80 take several (b, h, query block) items per
# workgroup when there are more items than compute units: one key-tile stream runs across
# the items and the next item's query rows load while the current one runs.  These shapes
# have more items than the 256 compute units of an MI355X, ragged sequence lengths (partial
# key tiles and query blocks) and a last workgroup with fewer items than the others.
MULTI = [
    # (entry, B, H, N, D, R, dtype)
    ("lowrank_log2", 40, 8, 300, 32, 16, "bf16"),
    ("lowrank", 40, 8, 300, 32, 16, "bf16"),
    ("lowrank_log2", 70, 4, 200, 16, 8, "f16"),
    ("lowrank_log2", 30, 10, 130, 32, 20, "bf16"),
    ("lowrank", 30, 10, 130, 32, 0, "bf16"),
    ("sandwich", 20, 8, 512, 32, 32, "bf16"),
    ("alibi", 33, 8, 260, 32, 0, "bf16"),
    # one key tile per item (every step switches items), per-batch factors
    ("lowrank_log2", 300, 2, 40, 32, 8, "bf16"),
    ("lowrank_batch", 130, 4, 70, 16, 16, "f16"),
    # D = 64 with 16 factor columns (D + R_pad = 80)
    ("lowrank_log2", 36, 8, 300, 64, 16, "bf16"),
    ("lowrank", 300, 2, 60, 64, 8, "f16"),
    ("alibi", 33, 8, 260, 64, 0, "bf16"),
    ("sandwich", 20, 8, 520, 64, 16, "bf16"),
    ("lowrank_batch", 70, 4, 130, 64, 12, "bf16"),
]


@pytest.mark.parametrize("entry,B,H,N,D,R,dt", MULTI, ids=[f"{m[0]}-{i}" for i, m in enumerate(MULTI)])
def test_multi_item_workgroups(fb, entry, B, H, N, D, R, dt):
    """Every output row and LSE of shapes with more work items than compute units, against
    the oracle (the factors the kernel reads, or the exact bias for in-kernel factors)."""
    import torch
    nqb = (N + 255) // 256
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"multi-item {entry} B={B} H={H} N={N} D={D} R={R} {dt}: {B * H * nqb} items, {ncu} CUs")
    r = np.random.default_rng(1500 + N + D + R)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    qd, kd, vd = (to_dev(x, dt) for x in (q, k, v))
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    if entry in ("lowrank", "lowrank_log2", "lowrank_batch"):
        fshape = (B, H, N, R) if entry == "lowrank_batch" else (H, N, R)
        pq = synth.round_to(r.standard_normal(fshape) * 0.5, "f16") if R else None
        pk = synth.round_to(r.standard_normal(fshape) * 0.5, "f16") if R else None
        run = fb.fb_attn_fwd_lowrank_log2 if entry == "lowrank_log2" else fb.fb_attn_fwd_lowrank
        o = run(qd, kd, vd, to_dev(pq, "f16") if R else None, to_dev(pk, "f16") if R else None, lse=lse)
        bias = None
        if R:
            bias = oracle.lowrank_bias(pq, pk) * (np.log(2.0) if entry == "lowrank_log2" else 1.0)
    elif entry == "sandwich":
        o = fb.fb_attn_fwd_sandwich(qd, kd, vd, C=R, lse=lse)
        bias = oracle.sandwich_bias(N, R)
    else:
        o = fb.fb_attn_fwd_alibi(qd, kd, vd, lse=lse)
        bias = oracle.alibi_bias(oracle.alibi_slopes(H), N)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, bias=bias)
    assert_close(to_np(o), ro, dt, f"multi-item {entry}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2)


# ------------------------------------------- whole K' and V resident in LDS ----
# Non-causal 16-bit launches in exp2 units with D + R_pad <= 48 whose K' and V tiles all fit
# in 80 KB of LDS run the resident kernel (one workgroup per (b, h), no barrier in the key
# loop); FB_ATTN_STREAMING=1 sends the same launch to the streaming kernel.  Shapes: the
# largest N of each (D, R_pad) (512 keys at D 32 / R_pad 16, 640 at D 32 / 0 and D 16 / 16,
# 512 at D 16 / 32, 832 at D 16 / 0), one key, ragged tails, R not a multiple of 16 (zero
# padding inside the kernel), per-batch factors, bf16 factors, f16 operands, more (b, h) than
# compute units, and two shapes just outside (D 64; D 32 with R_pad 32) that stream.
RESIDENT = [
    # (B, H, N, D, R, factor shape, Q/K/V dtype, factor dtype)
    (3, 4, 512, 32, 16, "head", "bf16", "f16"),
    (2, 3, 301, 32, 16, "head", "bf16", "f16"),
    (1, 2, 1, 32, 16, "head", "bf16", "f16"),
    (2, 2, 64, 16, 8, "batch", "f16", "f16"),
    (2, 2, 640, 16, 16, "head", "bf16", "f16"),
    (2, 2, 512, 16, 24, "batch", "bf16", "f16"),
    (2, 3, 640, 32, 0, None, "bf16", "f16"),
    (1, 2, 832, 16, 0, None, "f16", "f16"),
    (4, 2, 97, 16, 32, "head", "f16", "f16"),
    (2, 2, 130, 32, 16, "head", "bf16", "bf16"),
    (160, 4, 200, 32, 16, "head", "bf16", "f16"),
    (1, 3, 256, 64, 16, "head", "bf16", "f16"),
    (2, 2, 384, 32, 24, "batch", "bf16", "f16"),
    # wide, fast-moving scores (factor entries of scale 2.5: bias spread of about 25 in
    # exp2 units, running maxima that jump by more than the lazy-rescale headroom)
    (4, 2, 512, 32, 16, "wide", "bf16", "f16"),
    (2, 2, 512, 16, 32, "wide", "f16", "f16"),
]


@pytest.mark.parametrize("B,H,N,D,R,fsh,dt,pdt", RESIDENT, ids=[f"res-{i}" for i in range(len(RESIDENT))])
def test_resident_kernel(fb, B, H, N, D, R, fsh, dt, pdt, monkeypatch):
    """Every output row and LSE of fb_attn_fwd_lowrank_log2 against the oracle (factors in exp2
    units, i.e. the oracle's bias is ln 2 phi_q phi_k^T), once through the resident kernel and
    once through the streaming kernel."""
    import torch
    say(f"resident B={B} H={H} N={N} D={D} R={R} {fsh} {dt}/{pdt}")
    r = np.random.default_rng(2700 + N + D + R)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    qd, kd, vd = (to_dev(x, dt) for x in (q, k, v))
    pq = pk = None
    bias = None
    if R:
        fshape = (B, H, N, R) if fsh == "batch" else (H, N, R)
        fs = 2.5 if fsh == "wide" else 0.5
        pq, pk = (synth.round_to(r.standard_normal(fshape) * fs, pdt) for _ in range(2))
        bias = oracle.lowrank_bias(pq, pk) * np.log(2.0)
    ro, rl = oracle.attention(q, k, v, bias=bias)
    for streaming in (False, True):
        if streaming:
            monkeypatch.setenv("FB_ATTN_STREAMING", "1")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        o = fb.fb_attn_fwd_lowrank_log2(qd, kd, vd, to_dev(pq, pdt) if R else None,
                                        to_dev(pk, pdt) if R else None, lse=lse)
        torch.cuda.synchronize()
        what = "streaming" if streaming else "resident"
        assert_close(to_np(o), ro, dt, f"{what} O")
        np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2, err_msg=f"{what} LSE")
    monkeypatch.delenv("FB_ATTN_STREAMING")


def _resident_sweep(n=12, seed=20261204):
    """Random shapes the resident kernel takes (non-causal, D + R_pad <= 48, N up to the keys
    that fit), drawn once from a fixed seed: ragged N, every factor layout, both Q/K/V dtypes,
    factor scales from narrow to wide score ranges."""
    r = np.random.default_rng(seed)
    maxkeys = {(16, 0): 832, (16, 16): 640, (16, 32): 512, (32, 0): 640, (32, 16): 512}
    out = []
    for i in range(n):
        D = int(r.choice([16, 32]))
        R = int(r.choice([0, 8, 16] + ([24, 32] if D == 16 else [])))
        rp = 0 if R == 0 else 16 * ((R + 15) // 16)
        N = int(r.integers(1, maxkeys[(D, rp)] + 1))
        B, H = int(r.integers(1, 5)), int(r.integers(1, 4))
        fsh = str(r.choice(["head", "batch"]))
        dt = str(r.choice(["bf16", "f16"]))
        pdt = "f16" if dt == "f16" else str(r.choice(["bf16", "f16"]))
        out.append((B, H, N, D, R, fsh, dt, pdt, float(r.choice([0.25, 0.5, 1.5, 2.5]))))
    return out


@pytest.mark.parametrize("B,H,N,D,R,fsh,dt,pdt,fs", _resident_sweep(), ids=[f"res-sweep-{i}" for i in range(12)])
def test_resident_random_sweep(fb, B, H, N, D, R, fsh, dt, pdt, fs, monkeypatch):
    """Every output row and LSE of fb_attn_fwd_lowrank_log2 on seeded random resident-kernel
    shapes, through the resident and the streaming kernel, against the oracle."""
    import torch
    say(f"resident sweep B={B} H={H} N={N} D={D} R={R} {fsh} {dt}/{pdt} scale {fs}")
    r = np.random.default_rng(3100 + N + 7 * D + R)
    q, k, v = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3))
    qd, kd, vd = (to_dev(x, dt) for x in (q, k, v))
    pq = pk = bias = None
    if R:
        fshape = (B, H, N, R) if fsh == "batch" else (H, N, R)
        pq, pk = (synth.round_to(r.standard_normal(fshape) * fs, pdt) for _ in range(2))
        bias = oracle.lowrank_bias(pq, pk) * np.log(2.0)
    ro, rl = oracle.attention(q, k, v, bias=bias)
    for streaming in (False, True):
        if streaming:
            monkeypatch.setenv("FB_ATTN_STREAMING", "1")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        o = fb.fb_attn_fwd_lowrank_log2(qd, kd, vd, to_dev(pq, pdt) if R else None,
                                        to_dev(pk, pdt) if R else None, lse=lse)
        torch.cuda.synchronize()
        what = "streaming" if streaming else "resident"
        assert_close(to_np(o), ro, dt, f"{what} O")
        np.testing.assert_allclose(lse.cpu().double().numpy(), rl, rtol=0, atol=2e-2, err_msg=f"{what} LSE")
    monkeypatch.delenv("FB_ATTN_STREAMING")


# ------------------------------------------------ backward in exp2 units ----
BWD_LOG2 = [
    # (B, H, N, D, R, factor shape, dtype, causal)
    (2, 2, 230, 64, 64, "shared", "bf16", False),
    (1, 3, 190, 32, 16, "head", "bf16", True),
    (2, 2, 150, 64, 6, "full", "f16", True),
    (2, 1, 130, 16, 8, "head", "bf16", False),
]


@pytest.mark.parametrize("B,H,N,D,R,fs,dt,causal", BWD_LOG2, ids=[f"bwdlog2-{i}" for i in range(len(BWD_LOG2))])
def test_backward_log2_units(fb, B, H, N, D, R, fs, dt, causal):
    """fb_attn_bwd_lowrank_log2 on fb_attn_fwd_lowrank_log2's output: dQ, dK, dV and the
    gradients with respect to the exp2-unit phi_q and phi_k, against the oracle's chain rule for
    the bias ln(2) phi_q phi_k^T (d/d phi_q = ln(2) db phi_k, d/d phi_k = db^T ln(2) phi_q)."""
    import torch
    r = np.random.default_rng(1600 + N + R + D)
    q, k, v, do = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(4))
    shape = {"shared": (N, R), "head": (H, N, R), "full": (B, H, N, R)}[fs]
    pq2 = synth.round_to(r.standard_normal(shape) * 0.6, "f16")   # exp2 units
    pk = synth.round_to(r.standard_normal(shape) * 0.4, "f16")
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    pqd, pkd = to_dev(pq2, "f16"), to_dev(pk, "f16")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank_log2(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    dq, dk, dv, gpq, gpk = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal, log2=True)
    torch.cuda.synchronize()
    ln2 = np.log(2.0)
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=ln2 * oracle.lowrank_bias(pq2, pk), causal=causal)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_grad_close(to_np(got), ref, f"{name} exp2 units R={R} D={D}")
    full_q = np.broadcast_to(pq2, (B, H, N, R))
    full_k = np.broadcast_to(pk, (B, H, N, R))
    rgq_nat, rgk = oracle.lowrank_factor_grads(db, ln2 * full_q, full_k)
    assert_grad_close(gpq.cpu().double().numpy(), _sum_to(ln2 * rgq_nat, shape), f"dphi_q (exp2 units) R={R}")
    assert_grad_close(gpk.cpu().double().numpy(), _sum_to(rgk, shape), f"dphi_k R={R}")
