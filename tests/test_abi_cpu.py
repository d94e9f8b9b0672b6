"""CPU checks of the C-ABI library: it loads, exports every entry point that
include/fb.h declares, rejects bad arguments before any launch, and its host
SVD agrees with the oracle's.  No GPU kernel is launched here: every call below
either fails validation (which runs before any HIP call) or is host-only."""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_additive_rank_amd as fb
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "fb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fb_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ["fb_make_factors", "fb_attn_fwd_lowrank", "fb_attn_fwd_densebias", "fb_svd_factors",
              "fb_status_str", "fb_make_dense_bias", "fb_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = fb.load()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {fb.library_path}").read()
    for n in _declared_functions():
        assert re.search(rf"\bT {n}\b", out), n


def test_status_strings():
    assert fb.fb_status_str(0) == "FB_OK"
    for s in range(1, 5):
        assert fb.fb_status_str(s).startswith("FB_E")


# ------------------------------------------------------- validation paths ----
FAKE = 0x10000          # 16-byte-aligned address never dereferenced: validation fails first


def _args(**kw):
    a = fb._AttnArgs()
    a.B, a.H, a.N, a.D = kw.get("B", 1), kw.get("H", 1), kw.get("N", 64), kw.get("D", 64)
    a.dt = kw.get("dt", fb.FB_BF16)
    a.causal = 0
    a.scale = kw.get("scale", 0.125)
    a.q = kw.get("q", FAKE)
    a.k = kw.get("k", FAKE)
    a.v = kw.get("v", FAKE)
    a.o = kw.get("o", FAKE)
    D = a.D
    st = kw.get("strides", (a.H * a.N * D, a.N * D, D))
    a.sq = fb._I64x3(*st)
    a.sk = fb._I64x3(*st)
    a.sv = fb._I64x3(*st)
    a.so = fb._I64x3(*kw.get("so", st))
    a.lse = kw.get("lse", None)
    return a


def _lowrank(a, R=0, phi_dt=fb.FB_BF16, pq=FAKE, pk=FAKE, s=(0, 0, 64), entry="fb_attn_fwd_lowrank"):
    sp = fb._I64x3(*s)
    return getattr(fb.load(), entry)(ctypes.byref(a), pq, pk, phi_dt, R, ctypes.byref(sp), ctypes.byref(sp), None)


def _dense(a, bias=FAKE, bdt=fb.FB_BF16, s=(0, 0, 64)):
    sb = fb._I64x3(*s)
    return fb.load().fb_attn_fwd_densebias(ctypes.byref(a), bias, bdt, ctypes.byref(sb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=48), fb.FB_EUNSUPPORTED),
    (dict(D=256), fb.FB_EUNSUPPORTED),
    (dict(dt=7), fb.FB_EUNSUPPORTED),
    (dict(q=None), fb.FB_EINVAL),
    (dict(o=None), fb.FB_EINVAL),
    (dict(q=FAKE + 8), fb.FB_EINVAL),                       # misaligned
    (dict(strides=(4096, 64, 68)), fb.FB_EINVAL),           # row stride not a multiple of 8 elements
    (dict(strides=(4096, 64, 32)), fb.FB_EINVAL),           # row stride < D
    (dict(strides=(4096, -64, 64)), fb.FB_EINVAL),
    (dict(B=-1), fb.FB_EINVAL),
    (dict(lse=FAKE + 2), fb.FB_EINVAL),
    (dict(scale=float("nan")), fb.FB_EINVAL),
])
def test_attention_validation(kw, code):
    assert _lowrank(_args(**kw)) == code
    assert _lowrank(_args(**kw), entry="fb_attn_fwd_lowrank_log2") == code
    assert fb.fb_last_error() != ""
    if kw.get("dt") is None:
        assert _dense(_args(**kw)) == code


def test_empty_inputs_are_noops():
    # B*H*N == 0 returns before any pointer is looked at, so no launch happens
    assert _lowrank(_args(N=0, q=None, k=None, v=None, o=None)) == fb.FB_OK
    assert _dense(_args(B=0, q=None, k=None, v=None, o=None), bias=None) == fb.FB_OK


@pytest.mark.parametrize("R,phi_dt,kw,code", [
    (-1, fb.FB_BF16, {}, fb.FB_EINVAL),
    (129, fb.FB_BF16, {}, fb.FB_EUNSUPPORTED),
    (8, fb.FB_F32, {}, fb.FB_EUNSUPPORTED),                  # fp32 factors with bf16 q/k/v
    (8, fb.FB_BF16, dict(pq=None), fb.FB_EINVAL),
    (8, fb.FB_BF16, dict(s=(0, 0, 4)), fb.FB_EINVAL),       # factor row stride < R
    (8, fb.FB_BF16, dict(pq=FAKE + 1), fb.FB_EINVAL),       # not element aligned
])
def test_lowrank_factor_validation(R, phi_dt, kw, code):
    assert _lowrank(_args(), R=R, phi_dt=phi_dt, **kw) == code
    assert _lowrank(_args(), R=R, phi_dt=phi_dt, entry="fb_attn_fwd_lowrank_log2", **kw) == code


def test_lowrank_log2_needs_16bit():
    a = _args(dt=fb.FB_F32, D=32, strides=(2048, 1024, 32))
    assert _lowrank(a, R=8, phi_dt=fb.FB_F32, entry="fb_attn_fwd_lowrank_log2") == fb.FB_EUNSUPPORTED
    assert "bf16 or f16" in fb.fb_last_error()


def test_lowrank_fp32_limits():
    a = _args(dt=fb.FB_F32, D=32, strides=(2048, 1024, 32))
    assert _lowrank(a, R=33, phi_dt=fb.FB_F32) == fb.FB_EUNSUPPORTED
    assert _lowrank(a, R=4, phi_dt=fb.FB_BF16) == fb.FB_EUNSUPPORTED


@pytest.mark.parametrize("bdt,kw,code", [
    (fb.FB_F16, {}, fb.FB_EUNSUPPORTED),                    # bias dtype must match q/k/v
    (fb.FB_BF16, dict(bias=None), fb.FB_EINVAL),
    (fb.FB_BF16, dict(s=(0, 0, 32)), fb.FB_EINVAL),         # row stride < N
    (fb.FB_BF16, dict(bias=FAKE + 1), fb.FB_EINVAL),
])
def test_densebias_validation(bdt, kw, code):
    assert _dense(_args(), bdt=bdt, **kw) == code


def _mul(a, R=2, phi_dt=fb.FB_BF16, pq=FAKE, pk=FAKE, s=(0, 0, 64), ws=0x100000, wsb=None):
    sp = fb._I64x3(*s)
    if wsb is None:
        wsb = fb.load().fb_mulbias_workspace_bytes(ctypes.byref(a), R)
    return fb.load().fb_attn_fwd_mulbias(ctypes.byref(a), pq, pk, phi_dt, R, ctypes.byref(sp), ctypes.byref(sp),
                                         ws, wsb, None)


@pytest.mark.parametrize("kw,mkw,code", [
    ({}, dict(R=0), fb.FB_EINVAL),
    ({}, dict(R=4), fb.FB_EUNSUPPORTED),                    # (R - 1) D = 192 > 128
    (dict(D=32, strides=(2048, 1024, 32)), dict(R=6), fb.FB_EUNSUPPORTED),
    (dict(dt=fb.FB_F32), {}, fb.FB_EUNSUPPORTED),
    ({}, dict(pq=None), fb.FB_EINVAL),
    ({}, dict(phi_dt=9), fb.FB_EUNSUPPORTED),
    ({}, dict(s=(0, 0, 1)), fb.FB_EINVAL),                  # factor row stride < R
    ({}, dict(ws=None), fb.FB_EINVAL),
    ({}, dict(ws=0x100000 + 16), fb.FB_EINVAL),             # workspace not 256-byte aligned
    ({}, dict(wsb=1024), fb.FB_EINVAL),                     # workspace too small
    (dict(q=None), {}, fb.FB_EINVAL),
])
def test_mulbias_validation(kw, mkw, code):
    assert _mul(_args(**kw), **mkw) == code
    assert fb.fb_last_error() != ""


def test_mulbias_workspace_size():
    a = _args(B=2, H=3, N=100, D=32, strides=(9600, 3200, 32))
    rows, es = 2 * 3 * 100, 2
    up = lambda x: (x + 255) // 256 * 256
    for R in (1, 2, 5):
        want = 2 * up(rows * 32 * es) + 2 * up(rows * (R - 1) * 32 * es)
        assert fb.load().fb_mulbias_workspace_bytes(ctypes.byref(a), R) == want
    assert fb.load().fb_mulbias_workspace_bytes(ctypes.byref(a), 0) == 0
    assert fb.load().fb_mulbias_workspace_bytes(ctypes.byref(_args(N=0)), 2) == 0
    assert _mul(_args(N=0, q=None, k=None, v=None, o=None), ws=None) == fb.FB_OK


def _bwd(a, R=0, phi_dt=fb.FB_BF16, pq=FAKE, pk=FAKE, s=(0, 0, 64), **gk):
    g = fb._BwdArgs()
    st = (a.H * a.N * a.D, a.N * a.D, a.D)
    g.dout, g.dq, g.dk, g.dv = gk.get("dout", FAKE), gk.get("dq", FAKE), gk.get("dk", FAKE), gk.get("dv", FAKE)
    for n in ("sdo", "sdq", "sdk", "sdv"):
        setattr(g, n, fb._I64x3(*gk.get(n, st)))
    g.dphi_q, g.dphi_k = gk.get("dphi_q", FAKE), gk.get("dphi_k", FAKE)
    g.sdphi_q = g.sdphi_k = fb._I64x3(*gk.get("sdphi", (0, 0, 64)))
    g.work = gk.get("work", FAKE)
    g.work_bytes = gk.get("work_bytes", 1 << 40)
    sp = fb._I64x3(*s)
    return fb.load().fb_attn_bwd_lowrank(ctypes.byref(a), pq, pk, phi_dt, R, ctypes.byref(sp), ctypes.byref(sp),
                                         ctypes.byref(g), None)


@pytest.mark.parametrize("kw,bkw,code", [
    (dict(D=8, strides=(1024, 1024, 8), lse=FAKE), {}, fb.FB_EUNSUPPORTED),   # head dim 8: no kernel
    (dict(dt=fb.FB_F32, D=128, strides=(8192, 8192, 128), lse=FAKE), {}, fb.FB_EUNSUPPORTED),   # fp32: D <= 64
    (dict(dt=fb.FB_F32, D=32, strides=(2048, 2048, 32), lse=FAKE), dict(R=8, phi_dt=fb.FB_BF16),
     fb.FB_EUNSUPPORTED),                                                         # fp32 q/k/v, bf16 factors
    (dict(dt=fb.FB_F32, D=32, strides=(2048, 2048, 32), lse=FAKE), dict(R=8, phi_dt=fb.FB_F32, pq=FAKE + 2),
     fb.FB_EINVAL),                                                               # fp32 factors: element misaligned
    (dict(lse=FAKE), dict(R=12, pq=FAKE + 1), fb.FB_EINVAL),     # padded factors: element misaligned
    (dict(lse=FAKE), dict(R=12, dphi_q=FAKE + 2), fb.FB_EINVAL),  # padded gradients: not 4-byte aligned
    (dict(lse=FAKE), dict(R=72), fb.FB_EUNSUPPORTED),
    (dict(lse=FAKE), dict(R=8, phi_dt=fb.FB_F32), fb.FB_EUNSUPPORTED),
    (dict(lse=FAKE), dict(R=8, pq=FAKE + 8), fb.FB_EUNSUPPORTED),   # factor rows not 16-byte aligned
    (dict(lse=FAKE), dict(R=8, dphi_q=None), fb.FB_EINVAL),
    (dict(lse=FAKE), dict(R=-1), fb.FB_EINVAL),
    ({}, {}, fb.FB_EINVAL),                                     # no forward LSE
    (dict(lse=FAKE), dict(dq=None), fb.FB_EINVAL),
    (dict(lse=FAKE), dict(work=None), fb.FB_EINVAL),
    (dict(lse=FAKE), dict(work=FAKE + 16), fb.FB_EINVAL),              # workspace not 256-byte aligned
    (dict(lse=FAKE), dict(work_bytes=128), fb.FB_EINVAL),              # workspace too small (256 needed)
    (dict(lse=FAKE), dict(R=8, dphi_k=FAKE + 8), fb.FB_EINVAL),        # dphi not 16-byte aligned
    (dict(lse=FAKE), dict(R=8, sdphi=(0, 0, 10)), fb.FB_EINVAL),       # dphi row stride not 4 floats
    (dict(lse=FAKE), dict(dv=FAKE + 8), fb.FB_EINVAL),
    (dict(lse=FAKE), dict(sdk=(4096, 64, 60)), fb.FB_EINVAL),
    (dict(lse=FAKE), dict(sdo=(1 << 30, 1 << 30, 1 << 24)), fb.FB_EUNSUPPORTED),   # a dO tile spans 2^31 bytes
])
def test_backward_validation(kw, bkw, code):
    assert _bwd(_args(**kw), **bkw) == code
    assert fb.fb_last_error() != ""


def test_backward_log2_needs_16bit():
    """exp2-unit factors are a 16-bit path (as in the forward): fp32 q/k/v is refused."""
    a = _args(dt=fb.FB_F32, D=32, strides=(2048, 2048, 32), lse=FAKE)
    g = fb._BwdArgs()
    st = (a.H * a.N * a.D, a.N * a.D, a.D)
    g.dout = g.dq = g.dk = g.dv = g.dphi_q = g.dphi_k = FAKE
    for n in ("sdo", "sdq", "sdk", "sdv"):
        setattr(g, n, fb._I64x3(*st))
    g.sdphi_q = g.sdphi_k = fb._I64x3(0, 0, 8)
    g.work, g.work_bytes = FAKE, 1 << 40
    sp = fb._I64x3(0, 0, 8)
    assert fb.load().fb_attn_bwd_lowrank_log2(ctypes.byref(a), FAKE, FAKE, fb.FB_F32, 8, ctypes.byref(sp),
                                              ctypes.byref(sp), ctypes.byref(g), None) == fb.FB_EUNSUPPORTED
    assert "bf16 or f16" in fb.fb_last_error()


def _bwd_noalloc(a, R=0, **gk):
    g = fb._BwdArgs()
    st = (a.H * a.N * a.D, a.N * a.D, a.D)
    g.dout = g.dq = g.dk = g.dv = g.dphi_q = g.dphi_k = FAKE
    for n in ("sdo", "sdq", "sdk", "sdv"):
        setattr(g, n, fb._I64x3(*st))
    g.sdphi_q = g.sdphi_k = fb._I64x3(*gk.get("sdphi", (0, 0, 64)))
    g.work = gk.get("work", None)
    g.work_bytes = gk.get("work_bytes", 0)
    sp = fb._I64x3(0, 0, 64)
    return fb.load().fb_attn_bwd_lowrank_noalloc(ctypes.byref(a), FAKE, FAKE, fb.FB_F16, R, ctypes.byref(sp),
                                                 ctypes.byref(sp), ctypes.byref(g), None)


def test_backward_noalloc_validation():
    """The no-alloc backward rejects a caller workspace, and sizes whose workspace exceeds its
    scratch, before any HIP call; empty inputs are a no-op."""
    assert _bwd_noalloc(_args(lse=FAKE), work=FAKE, work_bytes=1 << 20) == fb.FB_EINVAL
    assert _bwd_noalloc(_args(lse=FAKE), work_bytes=256) == fb.FB_EINVAL
    # shared R = 64 factors over B8 H8 N8192: Delta plus two [B][H][N][64] fp32 partials, 268 MB
    big = _args(B=8, H=8, N=8192, lse=FAKE, strides=(8 * 8192 * 64, 8192 * 64, 64))
    assert _bwd_noalloc(big, R=64) == fb.FB_EUNSUPPORTED
    assert "scratch" in fb.fb_last_error()
    assert _bwd_noalloc(_args(N=0, q=None, k=None, v=None, o=None)) == fb.FB_OK


def test_backward_empty_is_noop():
    assert _bwd(_args(N=0, q=None, k=None, v=None, o=None), dq=None, work=None) == fb.FB_OK


def test_backward_workspace_bytes():
    """Delta ([B][H][N] fp32), then one [B][H][N][R] fp32 partial per factor gradient that is
    summed over an axis of size > 1 (0 stride); every part rounded up to 256 bytes."""
    ws = fb.fb_attn_bwd_workspace_bytes
    up = lambda x: -(-x // 256) * 256
    full = (3 * 100 * 8, 100 * 8, 8)
    assert ws(2, 3, 100, 0) == up(2 * 3 * 100 * 4)
    assert ws(2, 3, 100, 8, (0, 0, 8), full) == up(2400) + up(2 * 3 * 100 * 8 * 4)
    assert ws(2, 3, 100, 8, (0, 800, 8), (2400, 0, 8)) == up(2400) + 2 * up(19200)
    assert ws(2, 3, 100, 8, full, full) == up(2400)                   # per-(b, h) factors: written directly
    assert ws(1, 1, 100, 8, (0, 0, 8), (0, 0, 8)) == up(400)          # one (b, h): nothing to sum
    assert ws(0, 3, 100, 8) == 0 and ws(-1, 3, 100, 8) == 0


def test_alibi_in_kernel_validation():
    lib = fb.load()
    sl = (ctypes.c_double * 200)(*([0.5] * 200))
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args(dt=fb.FB_F32)), sl, None) == fb.FB_EUNSUPPORTED
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args(H=129, strides=(129 * 64 * 64, 4096, 64))), sl,
                                 None) == fb.FB_EUNSUPPORTED
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args(N=70000, strides=(70000 * 64, 70000 * 64, 64))), sl,
                                 None) == fb.FB_EUNSUPPORTED
    bad = (ctypes.c_double * 1)(float("nan"))
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args()), bad, None) == fb.FB_EINVAL
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args(D=48)), None, None) == fb.FB_EUNSUPPORTED
    assert lib.fb_attn_fwd_alibi(ctypes.byref(_args(N=0, q=None, k=None, v=None, o=None)), None, None) == fb.FB_OK


def test_make_factors_validation():
    lib = fb.load()
    r = ctypes.c_int(0)
    call = lambda kind=0, H=2, N=16, C=0, dt=fb.FB_F16, split=1, pq=FAKE, pk=FAKE, R_pad=16, fn=lib.fb_make_factors: \
        fn(kind, H, N, C, None, dt, split, pq, pk, R_pad, ctypes.byref(r), None)
    assert call(fn=lib.fb_make_factors_log2, kind=5) == fb.FB_EINVAL
    assert call(fn=lib.fb_make_factors_log2, split=2, R_pad=4) == fb.FB_EINVAL and r.value == 6
    assert call(kind=5) == fb.FB_EINVAL
    assert call(H=0) == fb.FB_EINVAL
    assert call(kind=1, C=3) == fb.FB_EINVAL
    assert call(split=4) == fb.FB_EINVAL
    assert call(R_pad=1) == fb.FB_EINVAL and r.value == 2
    assert call(split=2, R_pad=4) == fb.FB_EINVAL and r.value == 6
    assert call(kind=1, C=64, R_pad=32) == fb.FB_EINVAL and r.value == 64
    assert call(pq=None) == fb.FB_EINVAL
    assert call(pq=FAKE + 2) == fb.FB_EINVAL


def test_make_dense_bias_validation():
    lib = fb.load()
    call = lambda kind=0, H=2, N=16, C=0, bias=FAKE, hs=256, rs=16: \
        lib.fb_make_dense_bias(kind, H, N, C, None, fb.FB_BF16, bias, hs, rs, None)
    assert call(bias=None) == fb.FB_EINVAL
    assert call(rs=8) == fb.FB_EINVAL
    assert call(hs=100) == fb.FB_EINVAL
    assert call(kind=1, C=0) == fb.FB_EINVAL


def test_svd_validation():
    lib = fb.load()
    a = np.zeros((4, 4))
    p = a.ctypes.data_as(fb._DP)
    assert lib.fb_svd_factors(None, 4, 2, 0, p, p, None, None) == fb.FB_EINVAL
    assert lib.fb_svd_factors(p, 4, 5, 0, p, p, None, None) == fb.FB_EINVAL
    assert lib.fb_svd_factors(p, 4, 0, 0, p, p, None, None) == fb.FB_EINVAL


# ------------------------------------------------------------- host SVD ----
def test_host_svd_matches_oracle_on_random_decay():
    r = np.random.default_rng(3)
    N, R = 200, 8
    b = r.standard_normal((N, N)) @ np.diag(0.85 ** np.arange(N)) @ r.standard_normal((N, N))
    got = fb.fb_svd_factors(b, R, seed=1)
    ref = oracle.truncated_svd(b, R)
    np.testing.assert_allclose(got["sigma"], ref["sigma"][:R], rtol=1e-9)
    assert got["energy"] == pytest.approx(ref["energy"], rel=1e-10)
    err2 = np.linalg.norm(b - oracle.lowrank_bias(got["phi_q"], got["phi_k"])) ** 2
    assert err2 == pytest.approx(np.sum(ref["sigma"][R:] ** 2), rel=1e-7)


def test_host_svd_exact_rank():
    r = np.random.default_rng(4)
    a, c = r.standard_normal((96, 5)), r.standard_normal((96, 5))
    b = a @ c.T
    got = fb.fb_svd_factors(b, 5, seed=2)
    np.testing.assert_allclose(oracle.lowrank_bias(got["phi_q"], got["phi_k"]), b, rtol=0, atol=1e-10)
    assert got["energy"] == pytest.approx(1.0, abs=1e-12)


def test_host_svd_log2_units():
    """fb_svd_factors_log2: phi_q in exp2 units, so ln(2) phi_q phi_k^T is the same best rank-R
    approximation (Eckart-Young against the oracle's singular values); phi_k and sigma are
    fb_svd_factors' own."""
    r = np.random.default_rng(5)
    N, R = 120, 6
    b = r.standard_normal((N, N)) @ np.diag(0.8 ** np.arange(N)) @ r.standard_normal((N, N))
    got = fb.fb_svd_factors(b, R, seed=3, log2=True)
    nat = fb.fb_svd_factors(b, R, seed=3)
    ref = oracle.truncated_svd(b, R)
    np.testing.assert_array_equal(got["phi_k"], nat["phi_k"])
    np.testing.assert_array_equal(got["sigma"], nat["sigma"])
    np.testing.assert_allclose(got["phi_q"] * np.log(2.0), nat["phi_q"], rtol=1e-15, atol=0)
    err2 = np.linalg.norm(b - np.log(2.0) * oracle.lowrank_bias(got["phi_q"], got["phi_k"])) ** 2
    assert err2 == pytest.approx(np.sum(ref["sigma"][R:] ** 2), rel=1e-7)
    lib = fb.load()
    a = np.zeros((4, 4))
    p = a.ctypes.data_as(fb._DP)
    assert lib.fb_svd_factors_log2(None, 4, 2, 0, p, p, None, None) == fb.FB_EINVAL


@pytest.mark.parametrize("kind", ["vision", "pairformer"])
def test_host_svd_on_workload_biases(kind):
    """Small versions of the vision (spatial) and pair-rep biases: the host SVD
    reaches the optimal rank-R error and the oracle's singular values."""
    if kind == "vision":
        w = synth.workload("vision_svd", grid=12, B=1, H=2)
    else:
        w = synth.workload("pairformer_svd", N=96, B=1, H=2)
    b = synth.make_inputs(w)["bias_src"]
    for h in range(b.shape[0]):
        got = fb.fb_svd_factors(b[h], w.R, seed=h)
        ref = oracle.truncated_svd(b[h], w.R)
        np.testing.assert_allclose(got["sigma"], ref["sigma"][:w.R], rtol=1e-9)
        opt = np.sum(ref["sigma"][w.R:] ** 2)
        err2 = np.linalg.norm(b[h] - oracle.lowrank_bias(got["phi_q"], got["phi_k"])) ** 2
        assert err2 == pytest.approx(opt, rel=1e-6)


@pytest.mark.parametrize("kind", ["vision", "pairformer"])
@pytest.mark.parametrize("target", [0.9, 0.95, 0.99])
def test_rank_for_energy_matches_oracle(kind, target):
    """Rank selection by retained energy (the pages keep heads at 95%): the library's
    randomized singular values pick the same rank as the oracle's full SVD."""
    if kind == "vision":
        w = synth.workload("vision_svd", grid=12, B=1, H=2)
    else:
        w = synth.workload("pairformer_svd", N=96, B=1, H=2)
    b = synth.make_inputs(w)["bias_src"]
    for h in range(b.shape[0]):
        got = fb.fb_svd_rank_for_energy(b[h], target, R_max=40, seed=h)
        ref = oracle.rank_for_energy(b[h], target, R_max=40)
        assert got["R"] == ref["R"] and got["reached"] == ref["reached"]
        assert got["energy"] == pytest.approx(ref["energy"], rel=1e-9)


def test_rank_for_energy_validation():
    lib = fb.load()
    a = np.ones((4, 4))
    p = a.ctypes.data_as(fb._DP)
    r = ctypes.c_int(0)
    assert lib.fb_svd_rank_for_energy(None, 4, 2, 0.95, 0, ctypes.byref(r), None, None) == fb.FB_EINVAL
    assert lib.fb_svd_rank_for_energy(p, 4, 5, 0.95, 0, ctypes.byref(r), None, None) == fb.FB_EINVAL
    assert lib.fb_svd_rank_for_energy(p, 4, 2, 0.0, 0, ctypes.byref(r), None, None) == fb.FB_EINVAL
    assert lib.fb_svd_rank_for_energy(p, 4, 2, 1.5, 0, ctypes.byref(r), None, None) == fb.FB_EINVAL
    assert lib.fb_svd_rank_for_energy(p, 4, 2, 0.95, 0, None, None, None) == fb.FB_EINVAL
    assert lib.fb_svd_rank_for_energy(p, 4, 2, 0.95, 0, ctypes.byref(r), None, None) == fb.FB_OK and r.value == 1
    z = fb.fb_svd_rank_for_energy(np.zeros((6, 6)), 0.95, R_max=3)
    assert z == {"R": 1, "energy": 1.0, "reached": True}


def test_round_exact_helper_matches_numpy_half():
    """The test-side single-rounding helper agrees with numpy's direct fp64 -> fp16 cast."""
    from _parity import round_exact
    x = np.random.default_rng(5).standard_normal(100000) * np.exp(np.random.default_rng(6).uniform(-12, 12, 100000))
    x = x[np.abs(x) < 60000]
    np.testing.assert_array_equal(round_exact(x, "f16"), x.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(round_exact(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_fp32_head_dim_limit_and_stride_limit():
    a = _args(dt=fb.FB_F32, D=128, strides=(128 * 64, 128 * 64, 128))
    assert _lowrank(a) == fb.FB_EUNSUPPORTED
    big = _args(N=64, strides=(1 << 33, 4096, 64))           # batch stride beyond 32 bits
    assert _lowrank(big) == fb.FB_EUNSUPPORTED


def test_backward_workspace_with_padded_factors():
    """R not a multiple of 8: Delta, then two [B][H][N][R8] 16-bit factor copies and two fp32
    per-(b, h) gradient buffers, each part rounded up to 256 bytes; R a multiple of 8 with
    per-(b, h) gradient outputs needs Delta only."""
    up = lambda x: (x + 255) // 256 * 256
    B, H, N = 2, 3, 100
    rows = B * H * N
    full = fb._I64x3(H * N * 12, N * 12, 12)
    got = fb.load().fb_attn_bwd_workspace_bytes(B, H, N, 12, ctypes.byref(full), ctypes.byref(full))
    assert got == up(rows * 4) + 2 * up(rows * 16 * 2) + 2 * up(rows * 16 * 4)
    got6 = fb.load().fb_attn_bwd_workspace_bytes(B, H, N, 6, ctypes.byref(full), ctypes.byref(full))
    assert got6 == up(rows * 4) + 2 * up(rows * 8 * 2) + 2 * up(rows * 8 * 4)
    full16 = fb._I64x3(H * N * 16, N * 16, 16)
    assert fb.load().fb_attn_bwd_workspace_bytes(B, H, N, 16, ctypes.byref(full16), ctypes.byref(full16)) == up(rows * 4)
