"""Bit-exact checks of kv_append and the page-table gather on the GPU.

The library's gather uses the same address helper as the decode kernel, so
comparing it with the oracle's gather checks the page-table walk itself.
"""

import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, need_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.contiguous().cpu()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_paged_append_and_gather_bit_exact(dtype, d):
    dev = need_gpu()
    announce(f"paged kv_append + gather {dtype} d={d} B=6 Hkv=2 Nnew=5")
    inp = inputs.paged_inputs(31, 6, 4, 2, 5, d, 1, 90, spare_blocks=7, dtype=dtype)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    eta.kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["cache_lens"],
                  block_table=g["block_table"])
    L = inp["block_table"].shape[1] * 16
    out = eta.attn_gather_paged(g["k_pool"], g["seq_lens"], g["block_table"], L)
    torch.cuda.synchronize()
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    assert torch.equal(_bits(g["k_pool"]), _bits(kp))
    assert torch.equal(_bits(g["v_pool"]), _bits(vp))
    for b in range(6):
        n = int(inp["seq_lens"][b])
        ref = oracle.gather_paged(kp, inp["block_table"][b], n)
        assert torch.equal(_bits(out[b, :n]), _bits(ref))
        assert bool((out[b, n:] == 0).all())  # rows past seq_len untouched (zero-filled out)


def test_contiguous_append_bit_exact_and_bounds():
    dev = need_gpu()
    announce("contiguous kv_append bf16 d=128 B=3 L=40 Nnew=4, one sequence overflowing")
    B, L, Hkv, d, Nnew = 3, 40, 2, 128, 4
    cache_k = torch.randn(B, L, Hkv, d).to(torch.bfloat16)
    cache_v = torch.randn(B, L, Hkv, d).to(torch.bfloat16)
    k_new = torch.randn(B, Nnew, Hkv, d).to(torch.bfloat16)
    v_new = torch.randn(B, Nnew, Hkv, d).to(torch.bfloat16)
    lens = torch.tensor([0, 17, 38], dtype=torch.int32)  # the last one runs past L
    gk, gv = cache_k.to(dev), cache_v.to(dev)
    eta.kv_append(k_new.to(dev), v_new.to(dev), gk, gv, lens.to(dev))
    torch.cuda.synchronize()
    ref_k = cache_k.clone()
    ref_v = cache_v.clone()
    for b in range(B):
        for r in range(Nnew):
            t = int(lens[b]) + r
            if t < L:
                ref_k[b, t] = k_new[b, r]
                ref_v[b, t] = v_new[b, r]
    assert torch.equal(_bits(gk), _bits(ref_k))
    assert torch.equal(_bits(gv), _bits(ref_v))
