"""GPU parity of attn_prefill against the fp64 oracle (needs an MI355X).

Small shapes are compared element by element over several tiles with ragged
tails; the 4k causal GQA workload is compared element by element, and the 32k
one on every head and two rows of every 64-row query block, in the same
launch configuration the bench times.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, check, guards_intact, nan_guarded, need_gpu, scale_of

pytestmark = pytest.mark.gpu


def _run_full(dev, seed, B, Hq, Hkv, Nq, Nk, d, dtype, causal, q_offset):
    announce(f"prefill {dtype} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} "
             f"q_offset={q_offset} seed={seed}")
    q, k, v = inputs.prefill_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype)
    o, lse = eta.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=scale_of(d), causal=causal,
                              q_offset=q_offset)
    torch.cuda.synchronize()
    O, L = oracle.prefill_attention(q, k, v, scale_of(d), causal, q_offset)
    return check(o, O, lse, L, dtype, "prefill")


def test_single_head_f32_workload():
    dev = need_gpu()
    w = inputs.WORKLOADS["single_head_f32"]
    _run_full(dev, w["seed"], 1, 1, 1, 256, 256, 64, "f32", False, 0)


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,off", [
    (1, 2, 1, 100, 77, 64, False, 0),
    (1, 4, 2, 150, 150, 128, True, 0),
    (2, 3, 1, 65, 300, 128, True, 235),
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 2, 1, 40, 30, 64, True, -10),     # rows 0..9 see no key
    (1, 1, 1, 300, 1000, 128, False, 0),  # many tiles per wave, ragged tail
    (2, 4, 4, 17, 33, 64, True, 16),      # fewer tiles than waves
])
def test_f32_shapes(B, Hq, Hkv, Nq, Nk, d, causal, off):
    dev = need_gpu()
    _run_full(dev, 11, B, Hq, Hkv, Nq, Nk, d, "f32", causal, off)


BF16_CASES = [
    # several 64-key tiles, ragged tails, every group-size branch (G = 1, 2, 4, 8)
    (1, 8, 2, 300, 300, 128, True, 0),
    (1, 8, 2, 300, 300, 128, False, 0),
    (2, 4, 4, 130, 190, 64, False, 0),
    (1, 16, 2, 257, 257, 128, True, 0),
    (1, 6, 3, 100, 100, 128, True, 0),
    (1, 3, 3, 97, 200, 64, True, 103),
    (1, 8, 1, 64, 1000, 128, True, 936),
    (2, 8, 2, 33, 129, 128, True, 96),
    (1, 4, 1, 1, 513, 128, True, 512),
    (1, 4, 1, 200, 1, 64, False, 0),
    (1, 4, 2, 128, 128, 128, True, -40),   # first 40 rows see no key
    (1, 4, 2, 70, 0, 128, False, 0),       # no keys at all
    # several causal query blocks per head
    (1, 8, 2, 300, 300, 64, True, 0),      # odd number of blocks
    (2, 8, 2, 512, 600, 128, True, 88),    # even number of blocks
    (1, 4, 1, 300, 300, 128, True, -200),  # the earliest block sees no key
    (1, 4, 1, 200, 100, 128, True, -400),  # no row sees a key
]


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d,causal,off", BF16_CASES)
def test_bf16_shapes(B, Hq, Hkv, Nq, Nk, d, causal, off):
    dev = need_gpu()
    _run_full(dev, 12, B, Hq, Hkv, Nq, Nk, d, "bf16", causal, off)


def _workload_on_gpu(dev, name):
    w = inputs.WORKLOADS[name]
    q, k, v = inputs.prefill_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["N"], w["d"],
                                    "bf16", dev)
    o, lse = eta.attn_prefill(q, k, v, scale=scale_of(w["d"]), causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    return w, q, k, v, o, lse


def test_causal_gqa_prefill_4k_every_element():
    """The 4k causal GQA workload in the launch the bench times: every output
    element and every LSE of all 32 heads against the oracle."""
    dev = need_gpu()
    name = "causal_gqa_prefill_4k"
    w, q, k, v, o, lse = _workload_on_gpu(dev, name)
    announce(f"prefill workload {name}: B=1 Hq=32 Hkv=8 N=4096 d=128 causal, every element")
    G = w["Hq"] // w["Hkv"]
    rows = np.arange(w["N"])
    for hq in range(w["Hq"]):
        g = hq // G
        O, L = oracle.attention_rows(q[0, hq].cpu(), rows, k[0, g].cpu(), v[0, g].cpu(),
                                     scale_of(w["d"]), True)
        check(o[0, hq], O, lse[0, hq], L, "bf16", f"head {hq}")


def test_causal_gqa_prefill_32k_every_head_and_block():
    """The 32k causal GQA workload in the launch the bench times: all 32 heads;
    in each head the first row of every 64-row query block, one random row
    inside every block, and the last row (1025 rows per head, 8.2 M outputs)."""
    dev = need_gpu()
    name = "causal_gqa_prefill_32k"
    w, q, k, v, o, lse = _workload_on_gpu(dev, name)
    N = w["N"]
    announce(f"prefill workload {name}: B=1 Hq=32 Hkv=8 N={N} d=128 causal, every head, "
             "two rows of every 64-row block")
    G = w["Hq"] // w["Hkv"]
    rng = np.random.default_rng(1)
    for hq in range(w["Hq"]):
        g = hq // G
        starts = np.arange(0, N, 64)
        rows = np.unique(np.concatenate([starts, starts + rng.integers(1, 64, starts.size),
                                         [N - 1]]))
        K, V = k[0, g].cpu(), v[0, g].cpu()
        O, L = oracle.attention_rows(q[0, hq, rows].cpu(), rows, K, V, scale_of(w["d"]), True)
        check(o[0, hq, rows], O, lse[0, hq, rows], L, "bf16", f"head {hq} ({rows.size} rows)")


def test_deterministic_and_guard_bands():
    dev = need_gpu()
    announce("prefill determinism + NaN guard bands, B=1 Hq=8 Hkv=2 N=700 d=128 causal")
    q, k, v = inputs.prefill_inputs(13, 1, 8, 2, 700, 700, 128, "bf16", dev)
    buf_o, o = nan_guarded(q.shape, torch.bfloat16, dev)
    buf_l, lse = nan_guarded((1, 8, 700), torch.float32, dev)
    eta.attn_prefill(q, k, v, causal=True, out=o, lse=lse)
    first_o, first_l = o.clone(), lse.clone()
    for _ in range(9):
        eta.attn_prefill(q, k, v, causal=True, out=o, lse=lse)
        assert torch.equal(o.view(torch.int16), first_o.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), first_l.view(torch.int32))
    torch.cuda.synchronize()
    assert guards_intact(buf_o) and guards_intact(buf_l)
    assert bool(torch.isfinite(o).all())
