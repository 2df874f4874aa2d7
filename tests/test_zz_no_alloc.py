"""The allocation-free decode entry point (attn_decode_paged_noalloc, partial
results in the library's static device array) against attn_decode_paged with
a caller workspace, through the C ABI, on two calls in a row, the second
with a smaller input, and both against the fp64 oracle.

The two entry points launch the same kernels with the same worker split, so
their outputs must agree bit for bit; each is also within the bf16 tolerance
of the oracle.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, check, need_gpu, scale_of

pytestmark = pytest.mark.gpu


def _both(dev, q, kc, vc, sl, table):
    o1, l1 = eta.attn_decode_paged(q, kc, vc, sl, block_table=table, causal=True)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    eta.attn_decode_paged_noalloc(q, kc, vc, sl, block_table=table, causal=True, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    return o2, l2


def test_noalloc_matches_workspace_entry_on_two_calls():
    dev = need_gpu()
    # call 1: paged 4-token decode, 12 sequences of up to 3000 cached tokens
    announce("noalloc decode call 1: paged B=12 Hq=32 Hkv=8 Nq=4 d=128 cached[500,3000]")
    inp = inputs.paged_inputs(81, 12, 32, 8, 4, 128, 500, 3000)
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    eta.kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["cache_lens"],
                  block_table=g["block_table"])
    o, lse = _both(dev, g["q"], g["k_pool"], g["v_pool"], g["seq_lens"], g["block_table"])
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(128), True,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "noalloc call 1")

    # call 2, smaller: contiguous single-token decode, 3 sequences, d = 64
    announce("noalloc decode call 2: contiguous B=3 Hq=8 Hkv=2 Nq=1 d=64 lens [1, 200, 77]")
    q, kc, vc, sl = inputs.decode_contig_inputs(82, 3, 8, 2, 1, 64, 200, [1, 200, 77])
    o, lse = _both(dev, q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev), None)
    O, L = oracle.decode_attention(q, kc, vc, sl, scale_of(64), True)
    check(o, O, lse, L, "bf16", "noalloc call 2")


def test_noalloc_rejects_calls_past_its_array():
    dev = need_gpu()
    announce("noalloc decode rejects a call needing more than its static array")
    B, Hq, Hkv, Nq, d = 400, 32, 8, 4, 128
    assert eta.attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, 64) > eta.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Nq, Hq, d), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((B, 64, Hkv, d), dtype=torch.bfloat16, device=dev)
    sl = torch.full((B,), 64, dtype=torch.int32, device=dev)
    with pytest.raises(eta.AttnError, match="workspace"):
        eta.attn_decode_paged_noalloc(q, kc, kc, sl, causal=True)
