"""Helpers shared by the GPU parity tests and smoke(): run one workload through the
HIP path (libflashbias) and through the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys
from typing import Optional

import numpy as np

import oracle
import synth

# (max-abs, relative L2) bars of the parity contract
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 5e-3), "f16": (2e-2, 5e-3)}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def round_exact(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> dtype with a single round-to-nearest-even (torch's fp64 casts go through fp32
    and can round twice).  Values are returned as fp64."""
    prec, emin = {"f32": (24, -126), "bf16": (8, -126), "f16": (11, -14)}[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ex = np.maximum(e - 1, emin)
    q = np.ldexp(1.0, ex - prec + 1)
    return np.where(x == 0, x, np.rint(x / q) * q)


def to_dev(x: np.ndarray, dtype: str, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdtype(dtype)).to(device)


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def errors(got: np.ndarray, ref: np.ndarray):
    d = got - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


# Gradient tolerance (16-bit operands): relative L2 error and max-abs error relative to the
# largest reference magnitude (gradients have no fixed scale).  Budget: the gradients are
# stored in bf16 (rms relative rounding ~2^-9/sqrt(3) ~ 1.1e-3), P and dS are rounded to
# bf16 before their products (~1.1e-3 each after averaging over the contraction) and
# Delta uses the bf16 forward output: about 2e-3 rms, bounded here with a 2.5x margin;
# the largest element may carry a few half-ulp errors (1e-2 of the largest magnitude).
GRAD_TOL = (5e-3, 1e-2)


def assert_grad_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    ma, rl = errors(got, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    say(f"  {what}: rel-L2 {rl:.3e} (<= {GRAD_TOL[0]}), max-abs/max|ref| {ma / scale:.3e} (<= {GRAD_TOL[1]})")
    assert rl <= GRAD_TOL[0] and ma / scale <= GRAD_TOL[1], f"{what}: rel-L2 {rl:.3e}, max-abs {ma:.3e}"
    return ma, rl


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma, rl = errors(got, ref)
    amax, rmax = TOL[dtype]
    say(f"  {what}: max-abs {ma:.3e} (<= {amax}), rel-L2 {rl:.3e} (<= {rmax})")
    assert ma <= amax and rl <= rmax, f"{what}: max-abs {ma:.3e}, rel-L2 {rl:.3e}"
    return ma, rl


# ------------------------------------------------------------------ factors --
def factor_plan(w: synth.Workload):
    """Factor dtype and split used for each exact-bias workload on the GPU path.

    ALiBi in 16-bit: the factor m_h*j reaches ~1300 at N=2048, so one f16 value
    loses ~0.5 absolute; two f16 pieces per value (split=2) keep 22 bits.
    Sandwich: f16 factors (|phi| <= 1, 11 bits).  fp32 workloads: fp32 factors."""
    if w.dtype == "f32":
        return "f32", 1
    if w.bias == "alibi":
        return "f16", 2
    return "f16", 1


def exact_bias_oracle(w: synth.Workload):
    """Callable (b, h) -> [N, N] fp64 closed-form bias, from the oracle."""
    if w.bias == "alibi":
        m = oracle.alibi_slopes(w.H)
        cache = {}

        def f(b, h):
            if h not in cache:
                cache.clear()
                cache[h] = oracle.alibi_bias(m[h:h + 1], w.N)[0]
            return cache[h]
        return f
    if w.bias == "sandwich":
        bb = oracle.sandwich_bias(w.N, w.C)
        return lambda b, h: bb
    raise ValueError(w.bias)


def device_exact_factors(w: synth.Workload, device="cuda:0", log2: bool = False):
    """fb_make_factors (log2: fb_make_factors_log2) on the GPU for an exact-bias workload;
    returns (phi_q, phi_k) views broadcastable to [B, H, N, R]."""
    import attention_additive_rank_amd as fb
    dt, split = factor_plan(w)
    make = fb.fb_make_factors_log2 if log2 else fb.fb_make_factors
    if w.bias == "alibi":
        pq, pk, r = make("alibi", w.H, w.N, dtype=tdtype(dt), split=split, device=device)
        return pq, pk
    pq, pk, r = make("sandwich", 1, w.N, C=w.C, dtype=tdtype(dt), split=split, device=device)
    return pq, pk


def oracle_svd_factors(w: synth.Workload, bias_src: np.ndarray, phi_dtype: str = "f16"):
    """Per-head truncated-SVD factors from the oracle, rounded to the factor dtype
    (the kernel and the oracle then use the very same factor values)."""
    method = "full" if w.N <= 1024 else "arpack"
    pq = np.empty((w.H, w.N, w.R))
    pk = np.empty((w.H, w.N, w.R))
    energy = []
    for h in range(w.H):
        f = oracle.truncated_svd(bias_src[h], w.R, method=method)
        pq[h], pk[h] = f["phi_q"], f["phi_k"]
        energy.append(f["energy"])
    return synth.round_to(pq, phi_dtype), synth.round_to(pk, phi_dtype), energy


# ---------------------------------------------------------------- workloads --
class Case:
    """One workload prepared for both sides."""

    def __init__(self, w: synth.Workload, device="cuda:0", rows: Optional[np.ndarray] = None, log2: bool = False):
        """log2: the kernel gets phi_q in exp2 units (fb_attn_fwd_lowrank_log2); the oracle's
        bias is unchanged for exact biases, and ln(2) phi_q phi_k^T of the very same rounded
        factors for SVD workloads."""
        self.w = w
        self.device = device
        self.rows = rows
        self.log2 = log2
        inp = synth.make_inputs(w)
        self.q, self.k, self.v = inp["q"], inp["k"], inp["v"]
        self.qd, self.kd, self.vd = (to_dev(x, w.dtype, device) for x in (self.q, self.k, self.v))
        if w.bias in ("alibi", "sandwich"):
            self.bias_ref = exact_bias_oracle(w)
            self.phq, self.phk = device_exact_factors(w, device, log2)
            self.energy = None
        else:
            pq, pk, self.energy = oracle_svd_factors(w, inp["bias_src"], "f16")
            self.bias_full = inp["bias_src"]
            self.pq_np, self.pk_np = pq, pk
            if log2:
                pq2 = round_exact(pq * (1.0 / math.log(2.0)), "f16")
                self.bias_ref = lambda b, h: math.log(2.0) * oracle.lowrank_bias(pq2[h], pk[h])
                self.phq, self.phk = to_dev(pq2, "f16", device), to_dev(pk, "f16", device)
            else:
                self.bias_ref = lambda b, h: oracle.lowrank_bias(pq[h], pk[h])
                self.phq, self.phk = to_dev(pq, "f16", device), to_dev(pk, "f16", device)

    def run_lowrank(self, **kw):
        import attention_additive_rank_amd as fb
        run = fb.fb_attn_fwd_lowrank_log2 if self.log2 else fb.fb_attn_fwd_lowrank
        return run(self.qd, self.kd, self.vd, self.phq, self.phk, causal=self.w.causal, **kw)

    def reference(self, rows=None, bh=None):
        """Oracle output for all (b, h) or the listed pairs, restricted to `rows`."""
        w = self.w
        rows = self.rows if rows is None else rows
        if bh is None:
            o, lse = oracle.attention(self.q, self.k, self.v, bias=self.bias_ref, causal=w.causal, rows=rows)
            return o, lse
        outs, lses = [], []
        for (b, h) in bh:
            o, l = oracle.attention(self.q[b:b + 1, h:h + 1], self.k[b:b + 1, h:h + 1], self.v[b:b + 1, h:h + 1],
                                    bias=lambda _b, _h: self.bias_ref(b, h), causal=w.causal, rows=rows)
            outs.append(o[0, 0])
            lses.append(l[0, 0])
        return np.stack(outs), np.stack(lses)


def sample_rows(N: int, n: int, seed: int = 0) -> np.ndarray:
    """A fixed sample of query rows: the first and last rows, tile edges and random rows."""
    r = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, N // 2, N - 2, N - 1]
    extra = r.choice(N, size=min(N, n), replace=False)
    return np.unique(np.clip(np.concatenate([fixed, extra]), 0, N - 1))


def compare_whole(o_dev, ref_fn, B: int, H: int, dtype: str, what: str, lse_dev=None):
    """Every (b, h) and every row of a full-size output against the oracle, streamed one
    (b, h) at a time: ``ref_fn(b, h) -> (O [N, D], LSE [N])`` in fp64.  The relative L2 error
    is taken over the whole tensor (the contract's bar), max-abs over every element; the
    LSE (when given) to 2e-2 (16-bit) / 1e-4 (fp32) absolute."""
    got = to_np(o_dev)
    gl = lse_dev.detach().cpu().double().numpy() if lse_dev is not None else None
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    num = den = 0.0
    mx = lmx = 0.0
    for b in range(B):
        for h in range(H):
            ro, rl = ref_fn(b, h)
            d = got[b, h] - ro
            num += float(np.sum(d * d))
            den += float(np.sum(ro * ro))
            mx = max(mx, float(np.abs(d).max()))
            if gl is not None:
                lmx = max(lmx, float(np.abs(gl[b, h] - rl).max()))
    rl2 = math.sqrt(num / max(den, 1e-300))
    amax, rmax = TOL[dtype]
    ltol = 1e-4 if dtype == "f32" else 2e-2
    say(f"  {what}: {B * H} (b, h) x all rows: max-abs {mx:.3e} (<= {amax}), rel-L2 {rl2:.3e} (<= {rmax})"
        + (f", LSE max-abs {lmx:.3e} (<= {ltol})" if gl is not None else ""))
    assert mx <= amax and rl2 <= rmax, f"{what}: max-abs {mx:.3e}, rel-L2 {rl2:.3e}"
    if gl is not None:
        assert lmx <= ltol, f"{what}: LSE max-abs {lmx:.3e}"
    return mx, rl2


def pair_reference(c, b: int, h: int):
    """Oracle O and LSE of one (b, h) of a Case, all rows."""
    sl = (slice(b, b + 1), slice(h, h + 1))
    o, l = oracle.attention(c.q[sl], c.k[sl], c.v[sl], bias=lambda _b, _h: c.bias_ref(b, h), causal=c.w.causal)
    return o[0, 0], l[0, 0]
