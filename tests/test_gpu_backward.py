"""GPU parity of the backward pass (attn_prefill_backward) against the fp64
oracle's gradients, through the C ABI.

The forward kernel's own o and lse feed the backward, as in training. The
tolerance is derived from where the kernels round: P and dS are rounded to
bf16 (relative error at most u = 2^-8) before their matrix products, D is
formed from the bf16-stored O (error at most u times the size of its terms),
the forward's LSE carries an error well below u, the dK/dV kernel forms dS from
the rounded P, and each gradient is rounded once to bf16. Every one of those errors is at most u times a term of the
gradient's sum, so element by element
    |gpu - oracle| <= 4u (M + |oracle|) + 1e-6,
with M the oracle's sum of the absolute values of the terms (its
`magnitudes`); the fp32 accumulation adds far less than u.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, guards_intact, max_err, nan_guarded, need_gpu, scale_of

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _check_grads(got, ref, mags, what):
    for name, g, r, m in zip(("dq", "dk", "dv"), got, ref, mags):
        g = _f64(g)
        sel = ~np.isnan(r)
        assert np.isfinite(g[sel]).all(), f"{what} {name}: non-finite"
        err = np.abs(g[sel] - r[sel])
        bound = 4 * U * (m[sel] + np.abs(r[sel])) + 1e-6
        worst = float((err / bound).max()) if err.size else 0.0
        print(f"    {what} {name}: max|err|={err.max() if err.size else 0:.3e} "
              f"max|ref|={np.abs(r[sel]).max() if err.size else 0:.3e} "
              f"worst err/bound={worst:.3f}", flush=True)
        assert worst <= 1.0, f"{what} {name}: error above the rounding bound"


def _run(dev, seed, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, kv_heads=None):
    announce(f"backward bf16 B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
             f"q_offset={q_offset} seed={seed}")
    q, k, v, do = inputs.backward_inputs(seed, B, Hq, Hkv, Nq, Nk, d)
    qg, kg, vg, dog = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    sc = scale_of(d)
    o, lse = eta.attn_prefill(qg, kg, vg, scale=sc, causal=causal, q_offset=q_offset)
    dq, dk, dv = eta.attn_prefill_backward(qg, kg, vg, o, lse, dog, scale=sc, causal=causal,
                                           q_offset=q_offset)
    torch.cuda.synchronize()
    dQ, dK, dV, M = oracle.prefill_backward(q, k, v, do, sc, causal, q_offset, kv_heads=kv_heads,
                                            magnitudes=True)
    _check_grads((dq, dk, dv), (dQ, dK, dV), M, "backward")
    return dq, dk, dv


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,off", [
    (1, 2, 1, 100, 77, 64, False, 0),
    (1, 4, 2, 150, 150, 128, True, 0),
    (2, 3, 1, 65, 300, 128, True, 235),
    (1, 8, 2, 200, 200, 128, True, 0),
    (1, 4, 4, 129, 129, 64, True, 0),
    (1, 4, 1, 70, 50, 128, True, -20),     # rows 0..19 see no key: their dq is 0
    (2, 2, 2, 33, 257, 128, False, 0),
    (1, 6, 2, 190, 190, 64, True, 0),      # G = 3: two heads per workgroup slot
    (1, 8, 2, 64, 16384, 128, False, 0),   # enough key blocks that each group stays whole
    (1, 32, 4, 96, 96, 128, True, 0),      # G = 8: the group shared by several workgroups
    (1, 4, 2, 520, 520, 64, True, 0),      # d = 64 over many key blocks
    (2, 4, 1, 300, 130, 128, False, 0),    # more query rows than keys
    (1, 2, 1, 1, 1, 128, True, 0),         # one row, one key
])
def test_backward_matches_oracle(B, Hq, Hkv, Nq, Nk, d, causal, off):
    dev = need_gpu()
    _run(dev, 40 + Nq, B, Hq, Hkv, Nq, Nk, d, causal, off)


def test_backward_empty_sides():
    dev = need_gpu()
    announce("backward with Nq=0 (dk = dv = 0) and with Nk=0 (dq = 0)")
    q = torch.randn(1, 4, 0, 128, device=dev).to(torch.bfloat16)
    k = torch.randn(1, 2, 40, 128, device=dev).to(torch.bfloat16)
    lse = torch.empty(1, 4, 0, device=dev)
    dq, dk, dv = eta.attn_prefill_backward(q, k, k, q, lse, q, causal=True)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and bool((dk == 0).all()) and bool((dv == 0).all())
    q = torch.randn(1, 4, 30, 128, device=dev).to(torch.bfloat16)
    k = torch.randn(1, 2, 0, 128, device=dev).to(torch.bfloat16)
    o, lse = eta.attn_prefill(q, k, k, causal=True)
    dq, dk, dv = eta.attn_prefill_backward(q, k, k, o, lse, q, causal=True)
    torch.cuda.synchronize()
    assert bool((dq == 0).all()) and dk.numel() == 0


def test_backward_deterministic_and_in_bounds():
    dev = need_gpu()
    announce("backward determinism + NaN guard bands, B=1 Hq=8 Hkv=2 N=300 d=128 causal")
    q, k, v, do = inputs.backward_inputs(21, 1, 8, 2, 300, 300, 128, device=dev)
    o, lse = eta.attn_prefill(q, k, v, causal=True)
    bq, dq = nan_guarded(q.shape, torch.bfloat16, dev)
    bk, dk = nan_guarded(k.shape, torch.bfloat16, dev)
    bv, dv = nan_guarded(v.shape, torch.bfloat16, dev)
    eta.attn_prefill_backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv)
    first = [t.clone() for t in (dq, dk, dv)]
    for _ in range(4):
        eta.attn_prefill_backward(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv)
        for a, b in zip((dq, dk, dv), first):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    torch.cuda.synchronize()
    assert guards_intact(bq) and guards_intact(bk) and guards_intact(bv)
    assert all(bool(torch.isfinite(t).all()) for t in (dq, dk, dv))


def test_backward_workload_every_element():
    """The 4k causal GQA backward at full size: every element of dQ, dK and dV
    (all 8 K/V heads and their 32 query heads)."""
    dev = need_gpu()
    w = inputs.WORKLOADS["causal_gqa_backward_4k"]
    _run(dev, w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["N"], w["d"], True, 0)
