"""GPU parity of both workgroup widths of the bf16 prefill kernel, element by
element against the fp64 oracle, on every instantiation: head dim 64 and 128,
causal and not, slabs ([B, H, N, d]) and the token-major cache, 4 and 8 waves
(16 kernels).

The library picks 8 waves only for launches that fill the chip (one such
workgroup per compute unit, two under a causal mask), so at test-sized
shapes the width is forced through the test entry points; the cases then
cover, for each kernel, query-head groups of 1, 2, 3, 4 and 8 (8 = two
workgroups per K/V head and query block), ragged key counts, the offset mask
("Effizienz", "Der wichtige Maskenfehler beim Cache") with q_offset 0,
Nk - Nq and negative (rows that see no key), and for the cache, paged and
contiguous layouts, empty prefixes and sequences past the 64-block lookup
window. A last test checks which width the library chooses on its own.
"""

import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, check, need_gpu, scale_of

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Nq, Nk, q_offset under a causal mask)
SLABS = [
    (1, 8, 1, 300, 333, 33),     # G = 8: two workgroups per K/V head; bottom-right aligned
    (2, 6, 2, 257, 700, 443),    # G = 3: one head per workgroup slot
    (1, 4, 2, 200, 190, -20),    # G = 2; rows 0..19 see no key; ragged Nk
    (1, 3, 3, 130, 129, 0),      # G = 1
    (1, 4, 1, 520, 520, 0),      # G = 4, several query blocks at either width
]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,off", SLABS)
def test_slab_kernel_widths(B, Hq, Hkv, Nq, Nk, off, d, causal, waves):
    dev = need_gpu()
    q_offset = off if causal else 0
    announce(f"prefill bf16 waves={waves} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
             f"causal={causal} q_offset={q_offset}")
    q, k, v = inputs.prefill_inputs(50 + Nq, B, Hq, Hkv, Nq, Nk, d, "bf16")
    o, lse = eta.attn_prefill(q.to(dev), k.to(dev), v.to(dev), scale=scale_of(d), causal=causal,
                              q_offset=q_offset, waves=waves)
    torch.cuda.synchronize()
    O, L = oracle.prefill_attention(q, k, v, scale_of(d), causal, q_offset)
    check(o, O, lse, L, "bf16", f"waves={waves}")


# (B, Hq, Hkv, Nq, cached lengths lo, hi) for a paged cache, or a contiguous
# one when the last item is a list of sequence lengths
CACHES = [
    (3, 8, 2, 100, 20, 300),            # G = 4
    (2, 8, 1, 64, 0, 200),              # G = 8; a sequence may have an empty prefix
    (2, 4, 2, 33, 1100, 1400),          # G = 2; past the 64-block lookup window
    (2, 6, 2, 70, None, [400, 70]),     # G = 3, contiguous cache of 400 rows
    (3, 3, 3, 50, None, [120, 50, 77]),  # G = 1, contiguous
]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,Nq,lo,hi", CACHES)
def test_cache_kernel_widths(B, Hq, Hkv, Nq, lo, hi, d, causal, waves):
    dev = need_gpu()
    if lo is None:
        L = hi[0]
        announce(f"contiguous-cache prefill waves={waves} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} "
                 f"L={L} lens={hi} causal={causal}")
        q, kc, vc, sl = inputs.decode_contig_inputs(60 + Nq, B, Hq, Hkv, Nq, d, L, hi)
        o, lse = eta.attn_prefill_paged(q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev),
                                        scale=scale_of(d), causal=causal, waves=waves)
        torch.cuda.synchronize()
        O, Lr = oracle.decode_attention(q, kc, vc, sl, scale_of(d), causal)
    else:
        announce(f"paged prefill waves={waves} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} "
                 f"cached[{lo},{hi}] causal={causal}")
        inp = inputs.paged_inputs(70 + Nq, B, Hq, Hkv, Nq, d, lo, hi, spare_blocks=2)
        g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
        eta.kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["cache_lens"],
                      block_table=g["block_table"])
        o, lse = eta.attn_prefill_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                        block_table=g["block_table"], scale=scale_of(d),
                                        causal=causal, waves=waves)
        torch.cuda.synchronize()
        kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"],
                                  inp["cache_lens"])
        vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"],
                                  inp["cache_lens"])
        O, Lr = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(d), causal,
                                        block_table=inp["block_table"])
    check(o, O, lse, Lr, "bf16", f"waves={waves}")


def test_library_width_choice():
    need_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    announce(f"workgroup width choice on a device with {cus} compute units")
    # the 4k and 32k causal GQA workloads fill the chip with 8-wave workgroups
    assert eta.attn_prefill_workgroup_waves(1, 32, 8, 4096, True) == (8 if cus <= 256 else 4)
    assert eta.attn_prefill_workgroup_waves(1, 32, 8, 32768, True) == 8
    # the small test shapes run 4-wave workgroups
    for B, Hq, Hkv, Nq, _, _ in SLABS:
        assert eta.attn_prefill_workgroup_waves(B, Hq, Hkv, Nq, True) == 4


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_widths_ignore_nan_in_unused_rows(d, waves):
    """Both widths read a partly filled 16-token block through a range that
    ends at its last valid row: NaN in the unused slots and spare blocks must
    not reach the output."""
    dev = need_gpu()
    announce(f"paged prefill waves={waves} d={d} with NaN-poisoned unused rows, B=3 Hq=8 Hkv=2 "
             f"Nq=50")
    inp = inputs.paged_inputs(90 + d, 3, 8, 2, 50, d, 30, 200, spare_blocks=16)
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    inp["k_pool"], inp["v_pool"] = kp, vp
    assert inputs.poison_unused(inp) > 0
    g = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}
    o, lse = eta.attn_prefill_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                    block_table=g["block_table"], causal=True, waves=waves)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(d), True,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", f"poisoned pool, waves={waves}")
