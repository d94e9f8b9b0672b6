"""fb_attn_bwd_lowrank_noalloc, the backward whose workspace is the library's per-GPU device
scratch (for callers that cannot allocate), against fb_attn_bwd_lowrank with a caller
workspace: two calls in a row, the second with smaller inputs (it reuses the scratch the
first left behind).  Both run the same kernels on the same inputs, so the gradients must be
bit-identical; they are also held against the oracle's chain rule at the gradient bar."""
import numpy as np
import pytest

import oracle
import synth
from _parity import assert_grad_close, say, to_dev, to_np

pytestmark = pytest.mark.gpu

# (B, H, N, D, R, factor shape, causal): the first needs Delta and two summed factor-gradient
# partials in the scratch, the second (smaller) only Delta and one partial
CASES = [(2, 3, 300, 64, 16, "shared", True), (1, 2, 130, 32, 8, "head", False)]


@pytest.fixture(scope="module")
def fb(cuda):
    import attention_additive_rank_amd as m
    m.load()
    return m


def test_noalloc_backward_matches_workspace_backward(fb):
    import torch
    for i, (B, H, N, D, R, fs, causal) in enumerate(CASES):
        say(f"no-alloc backward call {i}: B={B} H={H} N={N} D={D} R={R} {fs} causal={causal}")
        r = np.random.default_rng(1300 + i)
        q, k, v, do = (synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, "bf16") for _ in range(4))
        shape = {"shared": (N, R), "head": (H, N, R)}[fs]
        pq = synth.round_to(r.standard_normal(shape) * 0.4, "f16")
        pk = synth.round_to(r.standard_normal(shape) * 0.4, "f16")
        qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
        pqd, pkd = to_dev(pq, "f16"), to_dev(pk, "f16")
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
        o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
        ref = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal)
        got = fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal, noalloc=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV", "dphi_q", "dphi_k"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from fb_attn_bwd_lowrank"
        rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=oracle.lowrank_bias(pq, pk), causal=causal)
        full_q, full_k = np.broadcast_to(pq, (B, H, N, R)), np.broadcast_to(pk, (B, H, N, R))
        rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
        axes = (0, 1) if fs == "shared" else (0,)
        for name, g, ref_np in (("dQ", got[0], rq), ("dK", got[1], rk), ("dV", got[2], rv),
                                ("dphi_q", got[3], rgq.sum(axis=axes)), ("dphi_k", got[4], rgk.sum(axis=axes))):
            assert_grad_close(to_np(g), ref_np, f"no-alloc call {i} {name}")
