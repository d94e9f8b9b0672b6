"""Every output element is written, and nothing beyond the outputs is.

Each output (O, LSE, the gradients) is a view at the start of a larger device buffer: the
view is filled with NaN before the call and the rest of the buffer with a sentinel value.
After the call the view must be finite and match the oracle (the parity bars), and the
sentinel tail must be unchanged.  Shapes are ragged (N not a multiple of the tiles).
"""
import numpy as np
import pytest

import oracle
import synth
from _parity import assert_close, assert_grad_close, say, tdtype, to_dev, to_np

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements of sentinel after each output
SENTINEL = 777.0


@pytest.fixture(scope="module")
def fb(cuda):
    import attention_additive_rank_amd as m
    m.load()
    return m


class Guarded:
    """A NaN-filled output view followed by GUARD sentinel elements."""

    def __init__(self, shape, dtype):
        import torch
        n = int(np.prod(shape))
        self.buf = torch.full((n + GUARD,), SENTINEL, dtype=dtype, device="cuda:0")
        self.buf[:n] = float("nan")
        self.view = self.buf[:n].view(shape)
        self.tail = self.buf[n:].clone()
        self.what = f"{tuple(shape)} {dtype}"

    def check_tail(self, what):
        import torch
        assert torch.equal(self.buf[-GUARD:], self.tail), f"{what}: write past the end of {self.what}"

    def value(self):
        got = to_np(self.view)
        assert np.all(np.isfinite(got)), f"unwritten (NaN) elements left in {self.what}"
        return got


def _inputs(seed, B, H, N, D, dt):
    r = np.random.default_rng(seed)
    return r, [synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt) for _ in range(3)]


FWD = [
    # (entry, B, H, N, D, dtype, causal)
    ("lowrank", 2, 3, 333, 64, "bf16", False),
    ("lowrank", 1, 2, 257, 16, "bf16", True),
    ("lowrank", 1, 2, 190, 32, "f32", True),
    ("lowrank_log2", 2, 2, 301, 64, "f16", True),
    ("lowrank_log2", 1, 3, 129, 16, "bf16", False),
    # factor rows of whole 16-byte chunks: these take the resident-K'/V kernel
    ("lowrank_log2_res", 2, 3, 301, 32, "bf16", False),
    ("lowrank_log2_res", 3, 1, 129, 16, "f16", False),
    ("densebias", 1, 2, 333, 64, "bf16", False),
    ("densebias", 2, 1, 200, 32, "f16", True),
    ("alibi", 2, 3, 275, 64, "bf16", True),
    ("sandwich", 1, 2, 333, 64, "bf16", False),
    ("sandwich", 1, 1, 150, 32, "f16", True),
    ("mulbias", 1, 2, 230, 32, "bf16", False),
]


@pytest.mark.parametrize("entry,B,H,N,D,dt,causal", FWD, ids=[f"{e[0]}-{i}" for i, e in enumerate(FWD)])
def test_forward_writes_every_output_and_nothing_more(fb, entry, B, H, N, D, dt, causal):
    import torch
    r, (q, k, v) = _inputs(1300 + N + D, B, H, N, D, dt)
    qd, kd, vd = (to_dev(x, dt) for x in (q, k, v))
    o = Guarded((B, H, N, D), tdtype(dt))
    lse = Guarded((B, H, N), torch.float32)
    say(f"poisoned outputs: {entry} B={B} H={H} N={N} D={D} {dt} causal={causal}")
    kw = dict(causal=causal, out=o.view, lse=lse.view)
    # mulbias: (R - 1) D <= 128; the resident kernel needs R a multiple of 8 with D + R <= 48
    R = 3 if entry == "mulbias" else (48 - D if entry == "lowrank_log2_res" else 6)
    pdt = "f32" if dt == "f32" else "f16"
    if entry == "lowrank_log2_res":
        entry = "lowrank_log2"
    if entry in ("lowrank", "lowrank_log2", "mulbias"):
        pq = synth.round_to(r.standard_normal((H, N, R)) * 0.5, pdt)
        pk = synth.round_to(r.standard_normal((H, N, R)) * 0.5, pdt)
        run = {"lowrank": fb.fb_attn_fwd_lowrank, "lowrank_log2": fb.fb_attn_fwd_lowrank_log2,
               "mulbias": fb.fb_attn_fwd_mulbias}[entry]
        run(qd, kd, vd, to_dev(pq, pdt), to_dev(pk, pdt), **kw)
        bias = oracle.lowrank_bias(pq, pk)
        if entry == "lowrank_log2":
            bias = np.log(2.0) * bias
    elif entry == "densebias":
        bias = synth.round_to(r.standard_normal((H, N, N)), dt)
        fb.fb_attn_fwd_densebias(qd, kd, vd, to_dev(bias, dt), **kw)
    elif entry == "alibi":
        fb.fb_attn_fwd_alibi(qd, kd, vd, **kw)
        bias = oracle.alibi_bias(oracle.alibi_slopes(H), N)
    else:
        fb.fb_attn_fwd_sandwich(qd, kd, vd, C=64, **kw)
        bias = oracle.sandwich_bias(N, 64)
    torch.cuda.synchronize()
    o.check_tail("O")
    lse.check_tail("LSE")
    if entry == "mulbias":
        ro, rl = oracle.attention_mulbias(q, k, v, bias, causal=causal)
    else:
        ro, rl = oracle.attention(q, k, v, bias=bias, causal=causal)
    assert_close(o.value(), ro, dt, f"{entry} O")
    np.testing.assert_allclose(lse.value(), rl, rtol=0, atol=1e-4 if dt == "f32" else 2e-2)


BWD = [
    # (B, H, N, D, R, factor shape, dtype, causal)
    (2, 2, 203, 64, 16, "shared", "bf16", True),
    (1, 3, 150, 32, 8, "head", "f16", False),
    (2, 2, 170, 16, 6, "head", "bf16", True),      # head dim 16, padded rank
    (1, 2, 90, 128, 16, "shared", "bf16", False),  # head dim 128
]


@pytest.mark.parametrize("B,H,N,D,R,fs,dt,causal", BWD, ids=[f"bwd-{i}" for i in range(len(BWD))])
def test_backward_writes_every_output_and_nothing_more(fb, B, H, N, D, R, fs, dt, causal):
    import torch
    r, (q, k, v) = _inputs(1400 + N + D, B, H, N, D, dt)
    do = synth.round_to(r.standard_normal((B, H, N, D)) * 0.5, dt)
    shape = {"shared": (N, R), "head": (H, N, R)}[fs]
    pq = synth.round_to(r.standard_normal(shape) * 0.4, "f16")
    pk = synth.round_to(r.standard_normal(shape) * 0.4, "f16")
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    pqd, pkd = to_dev(pq, "f16"), to_dev(pk, "f16")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    o = fb.fb_attn_fwd_lowrank(qd, kd, vd, pqd, pkd, causal=causal, lse=lse)
    grads = {n: Guarded((B, H, N, D), tdtype(dt)) for n in ("dq", "dk", "dv")}
    grads["dphi_q"] = Guarded(shape, torch.float32)
    grads["dphi_k"] = Guarded(shape, torch.float32)
    say(f"poisoned gradients: B={B} H={H} N={N} D={D} R={R} {fs} {dt} causal={causal}")
    fb.fb_attn_bwd_lowrank(qd, kd, vd, o, lse, dod, pqd, pkd, causal=causal,
                           **{n: g.view for n, g in grads.items()})
    torch.cuda.synchronize()
    for n, g in grads.items():
        g.check_tail(n)
    rq, rk, rv, db = oracle.attention_backward(q, k, v, do, bias=oracle.lowrank_bias(pq, pk), causal=causal)
    full_q, full_k = np.broadcast_to(pq, (B, H, N, R)), np.broadcast_to(pk, (B, H, N, R))
    rgq, rgk = oracle.lowrank_factor_grads(db, full_q, full_k)
    axes = (0, 1) if fs == "shared" else (0,)
    refs = {"dq": rq, "dk": rk, "dv": rv, "dphi_q": rgq.sum(axis=axes), "dphi_k": rgk.sum(axis=axes)}
    for n, g in grads.items():
        assert_grad_close(g.value(), refs[n], n)
