"""Benchmark of the biased-attention forward hot path on one MI355X.

One step = the whole hot path over one batch of synthetic input, inputs already
resident in HBM:
  1. exact factor generation on the GPU (fb_make_factors_log2: phi_q in exp2 units), and
  2. the fused low-rank-biased attention forward (fb_attn_fwd_lowrank_log2)
(fp32 workloads: fb_make_factors and fb_attn_fwd_lowrank, natural units).
(--workload mulbias_cos, the multiplicative bias b_ij = cos(i - j) of rank 2: 1. the
operand expansion fb_mulbias_expand, 2. the same fused kernel on the expanded operands.)
Default workload: Sandwich-bias attention, B=4, H=8, N=4096, D=64, C=R=64, bf16
(Q'/K' width 128), the configuration the N=4096, D=64 MFMA target is quoted on.

Prints ONE JSON line (rank 0): metric/value (whole-step TFLOP/s with
F = 4*B*H*N^2*(D + R/2)), the dominant kernel's roofline (HIP-event timed, against
the bf16 dense MFMA peak), the in-house dense-bias kernel on the same inputs
(speedup), and the fp64 CPU oracle timed on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["attention_additive_rank_amd/csrc/fb_attn_kernel.h",
                  "attention_additive_rank_amd/csrc/fb_attn_inst.hip"]


LOG2E = 1.4426950408889634   # log2(e)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def flops(w) -> float:
    """4 B H pairs (D + R/2); for the multiplicative bias the score contraction is D R wide
    (2 B H pairs (D R + D) in all)."""
    pairs = w.N * (w.N + 1) / 2 if w.causal else float(w.N) ** 2
    if w.bias == "mulbias_cos":
        return 2.0 * w.B * w.H * pairs * (w.D * w.R + w.D)
    return 4.0 * w.B * w.H * pairs * (w.D + w.R / 2.0)


def algorithmic_bytes(w, es: int, phi_es: int, phi_shared_over_heads: bool) -> float:
    """Q, K, V read and O written once, plus the factors (read once)."""
    qkvo = 4.0 * w.B * w.H * w.N * w.D * es
    phi_rows = w.N if phi_shared_over_heads else w.H * w.N
    return qkvo + 2.0 * phi_rows * w.R * phi_es


def cpu_oracle_baseline(w, budget_s: float, factors=None):
    """Time the fp64 oracle (numpy) on (b, h) pairs of the same workload until the budget is used.
    ``factors``: per-head (phi_q, phi_k) [H, N, R] of a low-rank (SVD) workload."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    inp = synth.make_inputs(w, with_bias_source=False)
    t0 = time.time()
    attn = oracle.attention
    if w.bias == "mulbias_cos":
        phi = oracle.cos_mulbias_factors(w.N)
        bias = oracle.lowrank_bias(phi, phi)
        bias_fn = lambda b, h: bias
        attn = oracle.attention_mulbias
    elif w.bias == "sandwich":
        bias = oracle.sandwich_bias(w.N, w.C)
        bias_fn = lambda b, h: bias
    elif factors is not None:
        bias_fn = lambda b, h: oracle.lowrank_bias(factors[0][h], factors[1][h])
    else:
        slopes = oracle.alibi_slopes(w.H)
        bias_fn = lambda b, h: oracle.alibi_bias(slopes[h:h + 1], w.N)[0]
    t_bias = time.time() - t0
    done, t_attn = 0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            s = time.time()
            attn(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1], inp["v"][b:b + 1, h:h + 1],
                 bias=lambda _b, _h: bias_fn(b, h), causal=w.causal)
            t_attn += time.time() - s
            done += 1
            if t_attn >= budget_s:
                break
        if t_attn >= budget_s:
            break
    f = flops(w) * done / (w.B * w.H)
    return {"value": round(f / t_attn / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.B * w.H} (batch, head) pairs, all {w.N} rows, fp64 numpy; "
                      f"bias materialisation {t_bias:.2f}s not included", "seconds": round(t_attn, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="sandwich",
                    choices=["sandwich", "gpt2_alibi_causal", "mulbias_cos", "vision_svd", "pairformer_svd"])
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-bias baseline")
    ap.add_argument("--cold-launches", type=int, default=21,
                    help="launches timed one by one after a cache flush (median reported; 0 = skip)")
    ap.add_argument("--alibi-jit", action="store_true",
                    help="ALiBi workloads: factors formed inside the kernel (fb_attn_fwd_alibi), no factor step")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fb_attn_bwd_lowrank) of the workload instead")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; multi-GPU runs are not provided "
                                   "(every (batch, head) pair is independent: see DESIGN.md for how it would shard)"}))
        sys.exit(2)

    import torch
    import attention_additive_rank_amd as fb
    import synth

    fb.load()
    dev = torch.device("cuda:0")
    w = synth.workload(args.workload)
    svd = w.bias in ("vision", "pairformer")
    inp = synth.make_inputs(w, with_bias_source=svd)
    dt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.dtype]
    q, k, v = (torch.from_numpy(inp[n]).to(dt).to(dev) for n in "qkv")
    svd_info = None
    if svd:
        # static per-head biases: rank-R factors from the library's host SVD (offline, not
        # timed); the dense-bias baseline streams the full [H, N, N] bias
        import numpy as np
        t0 = time.time()
        fs = [fb.fb_svd_factors(inp["bias_src"][h], w.R, seed=h) for h in range(w.H)]
        svd_info = {"seconds": round(time.time() - t0, 2), "energy_min": round(min(f["energy"] for f in fs), 6)}
        svd_phi = [np.stack([f[n] for f in fs]) for n in ("phi_q", "phi_k")]
        svd_bias = torch.from_numpy(inp["bias_src"]).to(dt).to(dev)
    del inp
    out = torch.empty_like(q)
    phi_dt = torch.float16 if w.dtype != "f32" else torch.float32
    split = 2 if (w.bias == "alibi" and w.dtype != "f32") else 1
    mul = w.bias == "mulbias_cos"
    if mul:
        # b_ij = cos(i - j) = cos i cos j + sin i sin j: fp32 factors [cos i, sin i], an input
        import numpy as np
        ii = np.arange(w.N, dtype=np.float64)
        phi_dt = torch.float32
        phi = torch.from_numpy(np.stack([np.cos(ii), np.sin(ii)], axis=1)).to(phi_dt).to(dev)
        ws = torch.empty(fb.fb_mulbias_workspace_bytes(q, w.R) + 256, dtype=torch.uint8, device=dev)
        fH, fC, R_used = 1, 0, w.R
    elif w.bias == "sandwich":
        fH, fC, R_used = 1, w.C, w.C * split * (split + 1) // 2
    elif svd:
        fH, fC, R_used = w.H, 0, w.R
    else:
        fH, fC, R_used = w.H, 0, 2 * split * (split + 1) // 2
    # factor rows padded with zero columns to a whole 16-byte chunk: the kernel then copies
    # phi_k rows with 16-byte loads (the zero columns add nothing to phi_q phi_k^T)
    ce = 16 // (2 if phi_dt == torch.float16 else 4)
    R_cols = (R_used + ce - 1) // ce * ce
    if not mul:
        pq = torch.zeros((fH, w.N, R_cols), dtype=phi_dt, device=dev)
        pk = torch.zeros_like(pq)
    jit = args.alibi_jit
    if jit and w.bias != "alibi":
        raise SystemExit("--alibi-jit needs an ALiBi workload")
    # 16-bit workloads take phi_q in exp2 units (phi_q log2(e), rounded once): the kernel then
    # skips one operation per score.  SVD factors are scaled on the host, in fp64.
    use_log2 = not (jit or mul or args.backward) and w.dtype != "f32"
    if svd:
        pq[..., :w.R] = torch.from_numpy(svd_phi[0] * (LOG2E if use_log2 else 1.0)).to(phi_dt).to(dev)
        pk[..., :w.R] = torch.from_numpy(svd_phi[1]).to(phi_dt).to(dev)
    stream = torch.cuda.current_stream(dev)


    def stage1(log2=use_log2):
        """factor generation (additive) or operand expansion (multiplicative)"""
        if jit or svd:
            return None
        if mul:
            return fb.fb_mulbias_expand(q, k, phi, phi, workspace=ws)
        make = fb.fb_make_factors_log2 if log2 else fb.fb_make_factors
        make(w.bias, fH, w.N, C=fC, dtype=phi_dt, split=split, phi_q=pq, phi_k=pk)
        return None

    def stage2(e):
        """the fused attention kernel"""
        if jit:
            fb.fb_attn_fwd_alibi(q, k, v, causal=w.causal, out=out)
        elif mul:
            fb.fb_attn_fwd_lowrank(e["q1"], e["k1"], v, e["phi_q"], e["phi_k"], causal=w.causal, scale=1.0, out=out)
        elif use_log2:
            fb.fb_attn_fwd_lowrank_log2(q, k, v, pq, pk, causal=w.causal, out=out)
        else:
            fb.fb_attn_fwd_lowrank(q, k, v, pq, pk, causal=w.causal, out=out)

    def step():
        stage2(stage1())

    if args.backward:
        if mul:
            raise SystemExit("--backward covers the additive workloads")
        return bench_backward(args, w, fb, torch, q, k, v, pq, pk, stage1, out, dev, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        e = stage1()
        ev[i][0].record(stream)
        stage2(e)
        ev[i][1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_stop) / K
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / K

    # cold caches: a 512 MiB scratch write before each launch evicts L2 and the Infinity
    # Cache, so the kernel reads its inputs from HBM; median over the launches
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def cold_median(fn, n=args.cold_launches):
        ts = []
        for _ in range(n):
            scratch.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2] if ts else None

    cold_step_ms = cold_median(step)
    e0 = stage1()
    cold_kern_ms = cold_median(lambda: stage2(e0))

    F = flops(w)
    value = F / (step_ms * 1e-3) / 1e12
    kern_tflops = F / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]

    # dense-bias baseline on the same inputs (shared [N,N] bias for Sandwich, per-head for ALiBi)
    dense = None
    if not args.no_dense and not mul:
        if w.bias == "sandwich":
            bias = fb.fb_make_dense_bias("sandwich", 1, w.N, C=w.C, dtype=dt)
        elif svd:
            bias = svd_bias
        else:
            bias = fb.fb_make_dense_bias("alibi", w.H, w.N, dtype=dt)
        for _ in range(args.warmup):
            fb.fb_attn_fwd_densebias(q, k, v, bias, causal=w.causal, out=out)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            fb.fb_attn_fwd_densebias(q, k, v, bias, causal=w.causal, out=out)
        b.record(stream)
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b) / K
        dense_cold = cold_median(lambda: fb.fb_attn_fwd_densebias(q, k, v, bias, causal=w.causal, out=out))
        dense = {"ms": round(dense_ms, 4), "tflops": round(F / (dense_ms * 1e-3) / 1e12, 2),
                 "cold_ms_median": round(dense_cold, 4) if dense_cold else None,
                 "bias_shape": list(bias.shape), "bias_bytes_unique": bias.numel() * bias.element_size()}
        del bias
    if svd:
        del svd_bias
    del scratch

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        x = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        del x, y

    # HBM traffic from rocprofv3 counters, only while they describe this kernel source
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_oracle_baseline(w, args.cpu_budget, factors=svd_phi if svd else None)

    es = 2 if w.dtype != "f32" else 4
    rec = {
        "metric": "biased-attention fwd TFLOP/s + % MFMA peak; speedup vs dense-bias kernel",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D, "R": w.R, "causal": w.causal,
                   "factor_dtype": "f16" if phi_dt == torch.float16 else "f32", "factor_split": split,
                   "factor_columns": R_used, "factor_columns_padded": R_cols,
                   "factor_units": "exp2 (phi_q log2(e))" if use_log2 else "natural",
                   "flops_per_step": F,
                   **({"bias_op": "multiplicative", "expanded_width": w.D * w.R} if mul else {}),
                   **({"factors": "in-kernel (fb_attn_fwd_alibi)"} if jit else {}),
                   **({"factors": "host SVD per head (fb_svd_factors, not timed)", "svd": svd_info} if svd else {})},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "kernel_ms": round(kern_ms, 4),
        "kernel_tflops": round(kern_tflops, 2),
        "cold": {"step_ms_median": round(cold_step_ms, 4) if cold_step_ms else None,
                 "kernel_ms_median": round(cold_kern_ms, 4) if cold_kern_ms else None,
                 "launches": args.cold_launches,
                 "flush": "512 MiB scratch written before each launch (L2 and Infinity Cache evicted)"},
        "densebias": dense,
        "speedup_vs_densebias": round(dense["ms"] / step_ms, 3) if dense else None,
        "roofline": {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / peak, 4), "traffic": traffic,
                     "algorithmic_bytes": (4.0 * w.B * w.H * w.N * w.D * es
                                           + 2.0 * w.B * w.H * w.N * (w.R - 1) * w.D * es) if mul else
                                          algorithmic_bytes(w, es, 2 if phi_dt == torch.float16 else 4,
                                                            w.bias == "sandwich"),
                     "kernel": "attn_fwd_kernel (fb_attn_fwd_lowrank_log2)" if use_log2 else
                               "attn_fwd_kernel (fb_attn_fwd_lowrank)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_backward(args, w, fb, torch, q, k, v, pq_t, pk_t, stage1, out, dev, stream):
    """Backward step: Delta = rowsum(dO * O), zeroed factor gradients, the key-major dK/dV
    kernel and the query-major dQ kernel (fb_attn_bwd_lowrank), after one forward that
    provides O and LSE.  Flops: the five products of the standard backward with the
    augmented width, 2 B H pairs (3 (D + R) + 2 D); the kernels recompute S and dP once
    more (the dQ kernel), which is not counted."""
    import numpy as np
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stage1(False)                   # the factors, as the forward step makes them, in natural units
    fb.fb_attn_fwd_lowrank(q, k, v, pq_t, pk_t, causal=w.causal, out=out, lse=lse)
    g = np.random.default_rng(w.seed + 7).standard_normal(q.shape) * 0.5
    dout = torch.from_numpy(g).to(q.dtype).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for _ in range(args.warmup):
        fb.fb_attn_bwd_lowrank(q, k, v, out, lse, dout, pq_t, pk_t, causal=w.causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        fb.fb_attn_bwd_lowrank(q, k, v, out, lse, dout, pq_t, pk_t, causal=w.causal, dq=dq, dk=dk, dv=dv)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    pairs = w.N * (w.N + 1) / 2 if w.causal else float(w.N) ** 2
    Rp = pq_t.shape[-1]
    F = 2.0 * w.B * w.H * pairs * (3 * (w.D + Rp) + 2 * w.D)
    tf = F / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    print(json.dumps({"metric": "biased-attention bwd TFLOP/s + % MFMA peak", "value": round(tf, 2),
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
                      "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
                      "data": "synthetic",
                      "config": {"workload": w.name + "_backward", "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                                 "R_columns": Rp, "causal": w.causal, "flops_per_step": F},
                      "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                                   "frac": round(tf / peak, 4), "traffic": None,
                                   "kernel": "attn_bwd_dkv_kernel + attn_bwd_dq_kernel (+ delta, factor-gradient sum)"},
                      "cpu_baseline": None}), flush=True)


if __name__ == "__main__":
    main()
