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
the dense matrix-core peak of its dtype), the in-house dense-bias kernel on the same
inputs (speedup), and the fp64 CPU oracle timed on a bounded sample of the same work.

Before the warm-up steps the step runs untimed for --settle-ms of wall time: the GPU
raises its shader clock over tens of milliseconds of sustained load, and a handful of
warm-up steps alone would time part of that ramp.  (The shader clock itself is read in
the --profile harness, from GRBM_COUNT over a dispatch's own timestamps.)

``--profile`` is the rocprofv3 harness: before touching the GPU it runs this script
under rocprofv3 in child processes (a kernel trace, then one counter pass each for
FETCH_SIZE, WRITE_SIZE and the matrix-core busy counters), parses their CSV output and
writes ``profiles/harness_<workload>.json`` and ``profiles/<kernel>_<workload>.md``;
later bench lines read HBM traffic, GB/s and matrix-core busy from that file while the
kernel sources are unchanged (by hash).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import re
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks
PEAK_HBM_GBS = 8000.0
N_XCD = 8
KERNEL_SOURCES = ["attention_additive_rank_amd/csrc/fb_attn_kernel.h",
                  "attention_additive_rank_amd/csrc/fb_attn_resident.h",
                  "attention_additive_rank_amd/csrc/fb_tile_map.h",
                  "attention_additive_rank_amd/csrc/fb_attn_inst.hip"]
WORKLOAD_CHOICES = ["sandwich", "gpt2_alibi_causal", "mulbias_cos", "vision_svd", "pairformer_svd",
                    "tiny_alibi_f32"]

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


def algorithmic_bytes(w, es: int, phi_es: int, phi_rows: int) -> float:
    """Q, K, V read and O written once, plus the factors (read once; phi_rows rows of each)."""
    qkvo = 4.0 * w.B * w.H * w.N * w.D * es
    return qkvo + 2.0 * phi_rows * w.R * phi_es


def harness_file(w, jit: bool = False) -> str:
    return os.path.join(ROOT, "profiles", f"harness_{w.name}{'_jit' if jit else ''}.json")


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
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed steps for this much wall time before the warm-up (shader clock ramp)")
    ap.add_argument("--workload", default="sandwich", choices=WORKLOAD_CHOICES)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-bias baseline")
    ap.add_argument("--cold-launches", type=int, default=21,
                    help="launches timed one by one after a cache flush (median reported; 0 = skip)")
    ap.add_argument("--jit", "--alibi-jit", dest="jit", action="store_true",
                    help="exact biases: factors formed inside the kernel (fb_attn_fwd_alibi / fb_attn_fwd_sandwich), "
                         "no factor step")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (fb_attn_bwd_lowrank) of the workload instead")
    ap.add_argument("--bwd-log2", action="store_true",
                    help="with --backward: factors in exp2 units, fb_attn_fwd_lowrank_log2 / fb_attn_bwd_lowrank_log2")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--profile", action="store_true",
                    help="rocprofv3 harness: trace + counter passes in child processes, then write profiles/")
    ap.add_argument("--profile-reparse", action="store_true",
                    help="with --profile: only re-read the CSV files of an earlier harness run")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "only one GPU is supported; multi-GPU runs are not provided (every (batch, head) "
                                   "pair is independent, so the work would shard over GPUs by (batch, head) with "
                                   "the factors replicated)"}))
        sys.exit(2)
    if args.profile:
        sys.exit(profile_harness(args))

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
    jit = args.jit
    if jit and w.bias not in ("alibi", "sandwich"):
        raise SystemExit("--jit needs an ALiBi or Sandwich workload")
    mul = w.bias == "mulbias_cos"
    # 16-bit workloads take phi_q in exp2 units (phi_q log2(e), rounded once): the kernel then
    # skips one operation per score.
    use_log2 = not (jit or mul or args.backward) and w.dtype != "f32"
    svd_info = None
    if svd:
        # static per-head biases: rank-R factors from the library's host SVD (offline, not
        # timed; phi_q in exp2 units from fb_svd_factors_log2); the dense-bias baseline
        # streams the full [H, N, N] bias
        import numpy as np
        t0 = time.time()
        fs = [fb.fb_svd_factors(inp["bias_src"][h], w.R, seed=h, log2=use_log2) for h in range(w.H)]
        svd_info = {"seconds": round(time.time() - t0, 2), "energy_min": round(min(f["energy"] for f in fs), 6)}
        svd_phi = [np.stack([f[n] for f in fs]) for n in ("phi_q", "phi_k")]
        svd_bias = torch.from_numpy(inp["bias_src"]).to(dt).to(dev)
    del inp
    out = torch.empty_like(q)
    phi_dt = torch.float16 if w.dtype != "f32" else torch.float32
    split = 2 if (w.bias == "alibi" and w.dtype != "f32") else 1
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
    if svd:
        pq[..., :w.R] = torch.from_numpy(svd_phi[0]).to(phi_dt).to(dev)
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
        if jit and w.bias == "alibi":
            fb.fb_attn_fwd_alibi(q, k, v, causal=w.causal, out=out)
        elif jit:
            fb.fb_attn_fwd_sandwich(q, k, v, C=w.C, causal=w.causal, out=out)
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

    settle = settle_phase(torch, step, args.settle_ms)
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
    launch_ms = sorted(a.elapsed_time(b) for a, b in ev)
    kern_ms = sum(launch_ms) / K                     # average launch duration (roofline)
    kern_med = launch_ms[K // 2]

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
        dstep = lambda: fb.fb_attn_fwd_densebias(q, k, v, bias, causal=w.causal, out=out)
        settle_phase(torch, dstep, args.settle_ms / 4)
        for _ in range(args.warmup):
            dstep()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(K):
            dstep()
        b.record(stream)
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b) / K
        dense_cold = cold_median(dstep)
        dense = {"ms": round(dense_ms, 4), "tflops": round(F / (dense_ms * 1e-3) / 1e12, 2),
                 "cold_ms_median": round(dense_cold, 4) if dense_cold else None,
                 "bias_shape": list(bias.shape), "bias_bytes_unique": bias.numel() * bias.element_size()}
        del bias
    if svd:
        del svd_bias
    del scratch

    calib_copy(torch, dev, args.calib_copy_mib)

    # rocprofv3 counters (the --profile harness), only while they describe this kernel source
    es = 2 if w.dtype != "f32" else 4
    phi_es = {torch.float16: 2, torch.bfloat16: 2, torch.float32: 4}[phi_dt]
    if mul:
        alg_bytes = 4.0 * w.B * w.H * w.N * w.D * es + 2.0 * w.B * w.H * w.N * (w.R - 1) * w.D * es
    elif jit:
        alg_bytes = algorithmic_bytes(w, es, phi_es, 0)
    else:
        alg_bytes = algorithmic_bytes(w, es, phi_es, fH * w.N)
    counters = None
    kernel_label = f"fused attention kernel ({entry_name(use_log2, jit, mul, w)})"
    hf = harness_file(w, jit)
    if os.path.exists(hf):
        with open(hf) as f:
            hr = json.load(f)
        if hr.get("kernel_source_hash") == kernel_source_hash() and hr.get("entry") == entry_name(use_log2, jit, mul, w):
            counters = {k2: hr.get(k2) for k2 in ("bytes_per_launch", "fetch_bytes", "write_bytes", "mfma_busy",
                                                  "l2_hit_rate", "sclk_mhz_counters", "trace_avg_us")}
            if hr.get("dense_bias_kernel"):
                counters["dense_bias_kernel"] = {k2: hr["dense_bias_kernel"].get(k2) for k2 in
                                                 ("bytes_per_launch", "mfma_busy", "l2_hit_rate", "hbm_gbs")}
            counters["hbm_gbs"] = round(hr["bytes_per_launch"] / (kern_ms * 1e-3) / 1e9, 1) \
                if hr.get("bytes_per_launch") else None
            counters["source"] = os.path.relpath(hf, ROOT)
            if hr.get("kernel"):
                # the kernel that ran, from the trace: its name up to the template arguments
                m = re.search(r"attn_fwd_(res_)?kernel", hr["kernel"])
                if m:
                    kernel_label = f"{m.group(0)} ({entry_name(use_log2, jit, mul, w)})"

    cpu = None
    if args.cpu_budget > 0:
        # the oracle takes the factors in natural units
        nat = (svd_phi[0] / LOG2E if use_log2 else svd_phi[0], svd_phi[1]) if svd else None
        cpu = cpu_oracle_baseline(w, args.cpu_budget, factors=nat)

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
                   "factor_units": "exp2 (phi_q log2(e))" if (use_log2 or (jit and w.bias == "sandwich")) else "natural",
                   "flops_per_step": F,
                   **({"bias_op": "multiplicative", "expanded_width": w.D * w.R} if mul else {}),
                   **({"factors": f"in-kernel ({entry_name(use_log2, jit, mul, w)})"} if jit else {}),
                   **({"factors": "host SVD per head (fb_svd_factors, not timed)", "svd": svd_info} if svd else {})},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "kernel_ms": round(kern_ms, 4),
        "kernel_ms_median": round(kern_med, 4),
        "kernel_tflops": round(kern_tflops, 2),
        "settle": settle,
        "cold": {"step_ms_median": round(cold_step_ms, 4) if cold_step_ms else None,
                 "kernel_ms_median": round(cold_kern_ms, 4) if cold_kern_ms else None,
                 "launches": args.cold_launches,
                 "flush": "512 MiB scratch written before each launch (L2 and Infinity Cache evicted)"},
        "densebias": dense,
        "speedup_vs_densebias": round(dense["ms"] / step_ms, 3) if dense else None,
        "roofline": {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / peak, 4),
                     "traffic": counters["bytes_per_launch"] if counters else None,
                     "algorithmic_bytes": alg_bytes,
                     "timing": "average of the timed launches (HIP events on the launch stream)",
                     "kernel": kernel_label},
        "counters": counters,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def entry_name(use_log2: bool, jit: bool, mul: bool, w=None) -> str:
    if jit:
        return "fb_attn_fwd_sandwich" if w is not None and w.bias == "sandwich" else "fb_attn_fwd_alibi"
    if use_log2:
        return "fb_attn_fwd_lowrank_log2"
    return "fb_attn_fwd_lowrank"


def settle_phase(torch, fn, ms: float):
    """Untimed steps, enqueued 16 at a time, for ``ms`` of wall time.  Returns {"steps", "ms"}."""
    if ms <= 0:
        return {"steps": 0, "ms": 0.0}
    t0 = time.time()
    n = 0
    while (time.time() - t0) * 1e3 < ms:
        for _ in range(16):
            fn()
        n += 16
        torch.cuda.synchronize()
    return {"steps": n, "ms": round((time.time() - t0) * 1e3, 1)}


def calib_copy(torch, dev, mib: int):
    """One device copy of ``mib`` MiB (the HBM counter calibration of the --profile harness)."""
    if mib <= 0:
        return
    n = mib * (1 << 20) // 4
    x = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y


def bench_backward(args, w, fb, torch, q, k, v, pq_t, pk_t, stage1, out, dev, stream):
    """Backward step: Delta = rowsum(dO * O), zeroed factor gradients, the key-major dK/dV
    kernel and the query-major dQ kernel (fb_attn_bwd_lowrank), after one forward that
    provides O and LSE.  Flops: the five products of the standard backward with the
    augmented width, 2 B H pairs (3 (D + R) + 2 D); the kernels recompute S and dP once
    more (the dQ kernel), which is not counted."""
    import numpy as np
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    lg = args.bwd_log2
    stage1(lg)                      # the factors, as the forward step makes them
    fwd = fb.fb_attn_fwd_lowrank_log2 if lg else fb.fb_attn_fwd_lowrank
    fwd(q, k, v, pq_t, pk_t, causal=w.causal, out=out, lse=lse)
    g = np.random.default_rng(w.seed + 7).standard_normal(q.shape) * 0.5
    dout = torch.from_numpy(g).to(q.dtype).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bstep = lambda: fb.fb_attn_bwd_lowrank(q, k, v, out, lse, dout, pq_t, pk_t, causal=w.causal, dq=dq, dk=dk, dv=dv,
                                           log2=lg)
    settle = settle_phase(torch, bstep, args.settle_ms)
    for _ in range(args.warmup):
        bstep()
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(K):
        bstep()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    calib_copy(torch, dev, args.calib_copy_mib)
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
                                 "R_columns": Rp, "causal": w.causal, "flops_per_step": F,
                                 "factor_units": "exp2 (phi_q log2(e))" if lg else "natural"},
                      "settle": settle,
                      "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                                   "frac": round(tf / peak, 4), "traffic": None,
                                   "kernel": "attn_bwd_dkv_kernel + attn_bwd_dq_kernel (+ delta, factor-gradient sum)"},
                      "cpu_baseline": None}), flush=True)


# --------------------------------------------------------------------------------------
# rocprofv3 harness (--profile).  Runs before anything in this process touches the GPU:
# every GPU run is a child process under rocprofv3.
def _csv_rows(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _run_child(cmd, log, timeout_s):
    """One profiled child run; returns its exit status (0 also when rocprofv3 itself faults
    after the program printed its result line)."""
    print(f"[harness] {' '.join(cmd)}", flush=True)
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout_s)] + cmd, stdout=f, stderr=subprocess.STDOUT,
                           cwd="/tmp", env=env)
    with open(log) as f:
        text = f.read()
    printed = '"metric"' in text
    print(f"[harness]   exit {r.returncode}{' (result line printed)' if printed else ''}", flush=True)
    if r.returncode != 0 and not (printed and r.returncode in (139, -11)):
        print(text[-3000:], flush=True)
        return r.returncode or 1
    return 0


def _harness_backward(args, w, tag, out_root, py, trace_cmd, short) -> int:
    """--profile --backward: the trace and counter passes of the backward step; per kernel
    (key-major dK/dV, query-major dQ) average time, bytes beyond L2, matrix-core busy fraction."""
    passes = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"],
              "busy": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_COUNT"]}

    def shown(cmd):
        return "cd $REPO && TMPDIR=/tmp " + " ".join(("python3" if c == py else c.replace(ROOT + os.sep, ""))
                                                  for c in cmd)
    cmds = {"trace": shown(trace_cmd)}
    hash_file = os.path.join(out_root, "kernel_source_hash")
    if not args.profile_reparse:
        with open(hash_file, "w") as f:
            f.write(kernel_source_hash() + "\n")
        if _run_child(trace_cmd, os.path.join(out_root, "trace.log"), 300):
            return 1
    for name, ctrs in passes.items():
        cmd = ["rocprofv3", "--pmc"] + ctrs + ["-d", os.path.join(out_root, name), "-o", name,
                                               "--output-format", "csv", "--"] + short
        cmds[name] = shown(cmd)
        if not args.profile_reparse and _run_child(cmd, os.path.join(out_root, f"{name}.log"), 120):
            return 1
    stats = _csv_rows(os.path.join(out_root, "trace", "**", "*kernel_stats.csv"))
    trace = {}
    for r in stats:
        nm = r.get("Name") or r.get("KernelName") or ""
        trace[nm] = (int(float(r.get("Calls") or 0)), float(r.get("AverageNs") or 0) / 1e3,
                     float(r.get("Percentage") or 0))

    def counter(name, pred, largest=False):
        vals = {}
        for r in _csv_rows(os.path.join(out_root, name, "**", "*counter_collection.csv")):
            kn = r.get("Kernel_Name") or ""
            if not pred(kn):
                continue
            cid, cn = r.get("Correlation_Id") or r.get("Dispatch_Id"), r.get("Counter_Name")
            vals.setdefault(cn, {}).setdefault(cid, 0.0)
            vals[cn][cid] += float(r.get("Counter_Value") or 0)
        if largest:
            return {c: max(d.values()) for c, d in vals.items() if d}
        return {c: sum(d.values()) / len(d) for c, d in vals.items() if d}
    copy = lambda kn: "copyBuffer" in kn
    fc, wc = counter("fetch", copy, True), counter("write", copy, True)
    if not fc.get("FETCH_SIZE") or not wc.get("WRITE_SIZE"):
        print("[harness] no calibration copy in the counter runs", flush=True)
        return 1
    fs, ws = 512 * 1024.0 / fc["FETCH_SIZE"], 512 * 1024.0 / wc["WRITE_SIZE"]
    src_hash = kernel_source_hash()
    if os.path.exists(hash_file):
        with open(hash_file) as f:
            src_hash = f.read().strip() or src_hash
    res = {"workload": w.name, "entry": "fb_attn_bwd_lowrank", "kernel_source_hash": src_hash, "commands": cmds,
           "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    for key in ("attn_bwd_dkv_kernel", "attn_bwd_dq_kernel", "delta_kernel", "reduce_kernel"):
        pred = lambda kn, key=key: key in kn
        rows = [(n, t) for n, t in trace.items() if key in n]
        if not rows:
            continue
        nm, (calls, avg, pct) = max(rows, key=lambda x: x[1][0])
        f_, w_, b_ = counter("fetch", pred), counter("write", pred), counter("busy", pred)
        k = {"name": nm, "calls": calls, "trace_avg_us": round(avg, 2), "pct_time": round(pct, 1)}
        if f_.get("FETCH_SIZE") is not None:
            k["fetch_bytes"] = int(f_["FETCH_SIZE"] * fs * 1024)
            k["write_bytes"] = int(w_.get("WRITE_SIZE", 0.0) * ws * 1024)
        if b_.get("SQ_BUSY_CU_CYCLES"):
            k["mfma_busy"] = round(b_.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * b_["SQ_BUSY_CU_CYCLES"]), 4)
        res["kernels"][key] = k
    hf = os.path.join(ROOT, "profiles", f"harness_{tag}.json")
    with open(hf, "w") as f:
        json.dump(res, f, indent=1)
    shape = f"b{w.B}h{w.H}n{w.N}d{w.D}r{w.R}"
    md = os.path.join(ROOT, "profiles", f"attn_bwd_lowrank_{w.name}_{shape}.md")
    lines = [f"# `fb_attn_bwd_lowrank` on the {w.name} workload (B={w.B} H={w.H} N={w.N} D={w.D} R={w.R}, "
             f"{w.dtype}; natural-unit factors)", "",
             f"Written by `python bench.py --profile --backward --workload {w.name} --steps {args.steps} "
             f"--warmup {args.warmup}` (the rocprofv3 harness in bench.py); raw CSV under gpurun_out/harness/.", "",
             "Kernel trace (rocprofv3 --kernel-trace --stats) of the timed backward steps:", "", "```",
             cmds["trace"], "```", "", "Counter passes (3 steps after 1 warm-up, a 512 MiB copy for calibration):",
             "", "```"] + [cmds[n] for n in passes] + ["```", "",
             f"Calibration: FETCH_SIZE x{fs:.3f}, WRITE_SIZE x{ws:.3f}.", "",
             "| kernel | calls | avg us | % time | read beyond L2 MB | written MB | matrix cores busy |",
             "|---|---|---|---|---|---|---|"]
    for key, k in res["kernels"].items():
        lines.append(f"| `{key}` | {k['calls']} | {k['trace_avg_us']:.1f} | {k['pct_time']:.1f} | "
                     f"{k.get('fetch_bytes', 0) / 1e6:.1f} | {k.get('write_bytes', 0) / 1e6:.1f} | "
                     f"{100 * k['mfma_busy']:.1f}% |" if "mfma_busy" in k else
                     f"| `{key}` | {k['calls']} | {k['trace_avg_us']:.1f} | {k['pct_time']:.1f} | "
                     f"{k.get('fetch_bytes', 0) / 1e6:.1f} | {k.get('write_bytes', 0) / 1e6:.1f} | — |")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"harness": os.path.relpath(hf, ROOT), "summary": os.path.relpath(md, ROOT),
                      "kernels": {k: v["trace_avg_us"] for k, v in res["kernels"].items()}}), flush=True)
    return 0


def profile_harness(args) -> int:
    import synth
    w = synth.workload(args.workload)
    bwd = args.backward
    tag = w.name + ("_jit" if args.jit else "") + ("_backward" if bwd else "")
    out_root = os.path.join(ROOT, "gpurun_out", "harness", tag)
    os.makedirs(out_root, exist_ok=True)
    py = sys.executable or "python3"
    bench = os.path.join(ROOT, "bench.py")
    base = [py, bench, "--workload", w.name, "--cpu-budget", "0", "--cold-launches", "0"]
    if args.jit:
        base.append("--jit")
    if bwd:
        base.append("--backward")
    # 1. kernel trace of the timed command (steps / warm-up as given)
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", os.path.join(out_root, "trace"), "-o", "trace",
                 "--output-format", "csv", "--"] + base + ["--steps", str(args.steps), "--warmup", str(args.warmup),
                                                          "--settle-ms", str(args.settle_ms)]
    hash_file = os.path.join(out_root, "kernel_source_hash")
    if not args.profile_reparse:
        with open(hash_file, "w") as f:                      # the sources these runs profile
            f.write(kernel_source_hash() + "\n")
        if _run_child(trace_cmd, os.path.join(out_root, "trace.log"), 300):
            return 1
    # 2.-4. counter passes: short runs (every dispatch is serialised under --pmc), with one
    # 512 MiB device copy as the HBM calibration
    # (the dense-bias kernel runs in the same short runs, so its counters come from the same passes)
    short = base + ["--steps", "3", "--warmup", "1", "--settle-ms", "0", "--calib-copy-mib", "512"]
    if bwd:
        return _harness_backward(args, w, tag, out_root, py, trace_cmd, short)
    passes = {"fetch": ["FETCH_SIZE"], "write": ["WRITE_SIZE"],
              "busy": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES",
                       "GRBM_GUI_ACTIVE", "GRBM_COUNT"],
              "l2": ["TCC_HIT_sum", "TCC_MISS_sum"]}
    def shown(cmd):
        """the command as run from the repository root (the child runs with cwd /tmp)"""
        return "cd $REPO && TMPDIR=/tmp " + " ".join(("python3" if c == py else c.replace(ROOT + os.sep, ""))
                                                  for c in cmd)
    cmds = {"trace": shown(trace_cmd)}
    for name, ctrs in passes.items():
        cmd = ["rocprofv3", "--pmc"] + ctrs + ["-d", os.path.join(out_root, name), "-o", name,
                                               "--output-format", "csv", "--"] + short
        cmds[name] = shown(cmd)
        if not args.profile_reparse and _run_child(cmd, os.path.join(out_root, f"{name}.log"), 120):
            if name in ("fetch", "write"):
                return 1
            print(f"[harness] the {name} counter pass failed; continuing without it", flush=True)

    # ---- parse
    stats = _csv_rows(os.path.join(out_root, "trace", "**", "*kernel_stats.csv"))
    entry = entry_name(not (args.jit or w.bias == "mulbias_cos") and w.dtype != "f32", args.jit,
                       w.bias == "mulbias_cos", w)

    def is_attn(name):
        return "attn_fwd_kernel" in name or "attn_fwd_res_kernel" in name

    # the step's attention kernel: the attn_fwd_kernel instance that is not the dense-bias one
    # (template MODE 1 shows as "Li1E" after the head dim and the factor width)
    def mode_of(name):
        """the MODE template argument, from a (partly) mangled ("...Li<D>ELi<RP>ELi<MODE>E...")
        or a demangled ("attn_fwd_kernel<QT, PT, D, RP, MODE, ...>") kernel name"""
        if "attn_fwd_res_kernel" in name:
            return 3          # the resident kernel: low rank in exp2 units only
        try:
            rest = name.split("attn_fwd_kernel")[1]
            li = rest.split("Li")
            if len(li) > 3:
                return int(li[3].split("E")[0])
            return int(rest[1:].split(",")[4].strip())
        except Exception:
            return -1
    trace_rows = []
    for r in stats:
        nm = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name") or ""
        avg = float(r.get("AverageNs") or r.get("Average_Ns") or r.get("AVG_NS") or 0) / 1e3
        calls = int(float(r.get("Calls") or r.get("Count") or 0))
        trace_rows.append((nm, calls, avg, float(r.get("MinNs") or 0) / 1e3, float(r.get("MaxNs") or 0) / 1e3,
                           float(r.get("Percentage") or 0)))
    main_k = [t for t in trace_rows if is_attn(t[0]) and mode_of(t[0]) != 1]
    dense_k = [t for t in trace_rows if is_attn(t[0]) and mode_of(t[0]) == 1]
    if not main_k:
        print("[harness] no attention kernel in the trace", flush=True)
        return 1
    kname, _, kavg, _, _, _ = max(main_k, key=lambda t: t[1])

    durations = {}

    def counter(name, kernel_pred, largest=False):
        """Per-dispatch counter values of the matching kernels, averaged (largest: the
        largest dispatch's, for the calibration copy among the run's other buffer copies)."""
        vals = {}
        for r in _csv_rows(os.path.join(out_root, name, "**", "*counter_collection.csv")):
            kn = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
            if not kernel_pred(kn):
                continue
            cid = r.get("Correlation_Id") or r.get("Dispatch_Id")
            cn = r.get("Counter_Name")
            vals.setdefault(cn, {}).setdefault(cid, 0.0)
            vals[cn][cid] += float(r.get("Counter_Value") or 0)
            try:
                durations.setdefault(name, {})[cid] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            except (KeyError, ValueError, TypeError):
                pass
        if largest:
            return {c: max(d.values()) for c, d in vals.items() if d}
        return {c: sum(d.values()) / len(d) for c, d in vals.items() if d}

    step_pred = lambda kn: is_attn(kn) and mode_of(kn) != 1
    copy_pred = lambda kn: "copyBuffer" in kn
    f_k, f_c = counter("fetch", step_pred), counter("fetch", copy_pred, largest=True)
    w_k, w_c = counter("write", step_pred), counter("write", copy_pred, largest=True)
    busy = counter("busy", step_pred)
    l2 = counter("l2", step_pred)
    dense_pred = lambda kn: is_attn(kn) and mode_of(kn) == 1
    calib = 512 * 1024.0                                     # KiB copied by the calibration run
    src_hash = kernel_source_hash()
    if os.path.exists(hash_file):                            # the sources the runs were taken with
        with open(hash_file) as f:
            src_hash = f.read().strip() or src_hash
    res = {"workload": w.name, "entry": entry, "kernel": kname, "kernel_source_hash": src_hash,
           "trace_avg_us": round(kavg, 2), "commands": cmds}
    if "FETCH_SIZE" in f_k and "FETCH_SIZE" in f_c and "WRITE_SIZE" in w_k and "WRITE_SIZE" in w_c:
        fs, ws = calib / f_c["FETCH_SIZE"], calib / w_c["WRITE_SIZE"]
        res.update({"fetch_kib_raw": f_k["FETCH_SIZE"], "write_kib_raw": w_k["WRITE_SIZE"],
                    "fetch_scale": fs, "write_scale": ws,
                    "fetch_bytes": int(f_k["FETCH_SIZE"] * fs * 1024), "write_bytes": int(w_k["WRITE_SIZE"] * ws * 1024)})
        res["bytes_per_launch"] = res["fetch_bytes"] + res["write_bytes"]
    def hit_rate(c):
        n = c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0)
        return round(c.get("TCC_HIT_sum", 0.0) / n, 4) if n else None
    if busy:
        res["busy_counters"] = busy
        if busy.get("SQ_BUSY_CU_CYCLES"):
            res["mfma_busy"] = round(busy.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * busy["SQ_BUSY_CU_CYCLES"]), 4)
    if l2:
        res["l2_counters"] = l2
        res["l2_hit_rate"] = hit_rate(l2)
    # the dense-bias kernel of the same short runs (absent for workloads without one)
    fd, wd, bd, ld = (counter(n, dense_pred) for n in ("fetch", "write", "busy", "l2"))
    if fd.get("FETCH_SIZE") and "fetch_scale" in res:
        dres = {"fetch_bytes": int(fd["FETCH_SIZE"] * res["fetch_scale"] * 1024),
                "write_bytes": int(wd.get("WRITE_SIZE", 0.0) * res["write_scale"] * 1024)}
        dres["bytes_per_launch"] = dres["fetch_bytes"] + dres["write_bytes"]
        if bd.get("SQ_BUSY_CU_CYCLES"):
            dres["mfma_busy"] = round(bd.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * bd["SQ_BUSY_CU_CYCLES"]), 4)
        if ld:
            dres["l2_counters"] = ld
            dres["l2_hit_rate"] = hit_rate(ld)
        if dense_k:
            dres["trace_avg_us"] = round(dense_k[0][2], 2)
            dres["hbm_gbs"] = round(dres["bytes_per_launch"] / (dense_k[0][2] * 1e-6) / 1e9, 1)
        res["dense_bias_kernel"] = dres
    res["counter_runs"] = "3 steps after 1 warm-up, no settle phase (dispatches serialised by the profiler)"
    # shader clock of the counter runs: GRBM_COUNT counts clocks, summed over the XCDs, over
    # the dispatch's duration (start and end timestamps of the same rows)
    dur = sorted(durations.get("busy", {}).values())
    if busy.get("GRBM_COUNT") and dur:
        res["counter_run_us"] = round(dur[len(dur) // 2], 2)
        res["sclk_mhz_counters"] = round(busy["GRBM_COUNT"] / N_XCD / dur[len(dur) // 2], 0)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(harness_file(w, args.jit), "w") as f:
        json.dump(res, f, indent=1)

    # ---- markdown summary
    shape = f"b{w.B}h{w.H}n{w.N}d{w.D}" + (f"r{w.R}" if not (args.jit and w.bias == "alibi") else "")
    md = os.path.join(ROOT, "profiles", f"{entry.replace('fb_', '')}_{w.name}_{shape}.md")
    lines = [f"# `{entry}` on the {w.name} workload (B={w.B} H={w.H} N={w.N} D={w.D} R={w.R}, {w.dtype})", "",
             "Written by `python bench.py --profile --workload " + w.name +
             (" --jit" if args.jit else "") + f" --steps {args.steps} --warmup {args.warmup}` "
             "(the rocprofv3 harness in bench.py); raw CSV under gpurun_out/harness/.", "",
             "Kernel trace (rocprofv3 --kernel-trace --stats):", "", "```", cmds["trace"], "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for t in sorted(trace_rows, key=lambda t: -t[5])[:6]:
        lines.append(f"| `{t[0][:110]}` | {t[1]} | {t[2]:.1f} | {t[3]:.1f} | {t[4]:.1f} | {t[5]:.1f} |")
    lines += ["", f"Step kernel: `{kname}`, average {kavg:.1f} us per launch in the trace."]
    if dense_k:
        lines.append(f"Dense-bias kernel (same inputs): average {dense_k[0][2]:.1f} us.")
    lines += ["", "Counter passes (one rocprofv3 --pmc run each, 3 steps after 1 warm-up, with a 512 MiB "
              "device copy for calibration):", "", "```"] + [cmds[n] for n in passes] + ["```", ""]
    if "bytes_per_launch" in res:
        lines.append(f"Calibration: the 512 MiB copy reads as FETCH_SIZE {f_c['FETCH_SIZE']:.0f} KiB (scale x"
                     f"{res['fetch_scale']:.3f}) and WRITE_SIZE {w_c['WRITE_SIZE']:.0f} KiB (scale x{res['write_scale']:.3f}).")
        lines.append(f"Step kernel per launch: FETCH_SIZE {res['fetch_kib_raw']:.0f} KiB -> {res['fetch_bytes'] / 1e6:.1f} MB "
                     f"read, WRITE_SIZE {res['write_kib_raw']:.0f} KiB -> {res['write_bytes'] / 1e6:.1f} MB written; "
                     f"{res['bytes_per_launch'] / 1e6:.1f} MB in all, "
                     f"{res['bytes_per_launch'] / (kavg * 1e-6) / 1e9:.0f} GB/s at the traced average.")
    if "mfma_busy" in res:
        b = res["busy_counters"]
        lines.append(f"SQ_VALU_MFMA_BUSY_CYCLES {b.get('SQ_VALU_MFMA_BUSY_CYCLES', 0):.4g}, SQ_BUSY_CU_CYCLES "
                     f"{b.get('SQ_BUSY_CU_CYCLES', 0):.4g}: matrix cores busy {100 * res['mfma_busy']:.1f}% of the "
                     "busy CU cycles (MFMA busy / (4 SIMDs x CU busy cycles)); SQ_WAVE_CYCLES "
                     f"{b.get('SQ_WAVE_CYCLES', 0):.4g}, SQ_BUSY_CYCLES {b.get('SQ_BUSY_CYCLES', 0):.4g}, "
                     f"GRBM_GUI_ACTIVE {b.get('GRBM_GUI_ACTIVE', 0):.4g}, GRBM_COUNT {b.get('GRBM_COUNT', 0):.4g}.")
    if "sclk_mhz_counters" in res:
        lines.append(f"Shader clock in the counter runs: GRBM_COUNT / {N_XCD} XCDs / {res['counter_run_us']} us "
                     f"(the dispatch's own timestamps) = {res['sclk_mhz_counters']:.0f} MHz.")
    if res.get("l2_hit_rate") is not None:
        lines.append(f"L2: TCC_HIT_sum {l2.get('TCC_HIT_sum', 0):.4g}, TCC_MISS_sum {l2.get('TCC_MISS_sum', 0):.4g}: "
                     f"hit rate {100 * res['l2_hit_rate']:.1f}%.")
    if "dense_bias_kernel" in res:
        d = res["dense_bias_kernel"]
        lines += ["", "Dense-bias kernel of the same counter runs (MODE 1, the [.., N, N] bias streamed):"]
        lines.append(f"FETCH_SIZE -> {d['fetch_bytes'] / 1e6:.1f} MB read, WRITE_SIZE -> {d['write_bytes'] / 1e6:.1f} MB "
                     f"written per launch" + (f", {d['hbm_gbs']:.0f} GB/s at its traced average" if "hbm_gbs" in d else "")
                     + (f"; matrix cores busy {100 * d['mfma_busy']:.1f}%" if "mfma_busy" in d else "")
                     + (f"; L2 hit rate {100 * d['l2_hit_rate']:.1f}%" if d.get("l2_hit_rate") is not None else "")
                     + ".")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"harness": os.path.relpath(harness_file(w, args.jit), ROOT), "summary": os.path.relpath(md, ROOT),
                      "trace_avg_us": res["trace_avg_us"], "bytes_per_launch": res.get("bytes_per_launch"),
                      "mfma_busy": res.get("mfma_busy")}), flush=True)
    return 0


if __name__ == "__main__":
    main()
