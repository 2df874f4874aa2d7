"""GPU parity of attn_prefill_paged (chunked prefill against a K/V cache) with
the fp64 oracle's cache attention (any number of new tokens per sequence).

Covers paged and contiguous caches, chunks of 16..600 tokens, group sizes
1..8, head dims 64/128, causal and not, a first chunk with an empty cache,
chunks that straddle blocks, invalid table entries, NaN-poisoned unused cache
rows, a prompt processed chunk by chunk against a full prefill, bitwise
determinism and output guard bands, and the 8 x 512-token chunked prefill
workload at full size, every output element.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import (announce, check, guards_intact, nan_guarded, need_gpu, scale_of,
                               to_f64)

pytestmark = pytest.mark.gpu


def _dev(inp, dev):
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}


def _append_and_run(inp, dev, causal=True):
    g = _dev(inp, dev)
    eta.kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["cache_lens"],
                  block_table=g["block_table"])
    d = inp["q"].shape[-1]
    o, lse = eta.attn_prefill_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                    block_table=g["block_table"], scale=scale_of(d),
                                    causal=causal)
    torch.cuda.synchronize()
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    return g, o, lse, kp, vp


@pytest.mark.parametrize("B,Hq,Hkv,Nq,d,lo,hi,causal", [
    (2, 8, 2, 16, 128, 20, 300, True),
    (2, 32, 8, 100, 128, 50, 500, True),
    (3, 4, 4, 64, 64, 1, 200, True),        # G=1
    (2, 16, 2, 257, 128, 0, 900, True),     # a sequence may start with an empty cache
    (1, 8, 1, 130, 64, 33, 33, False),      # G=8, not causal
    (2, 6, 3, 48, 128, 10, 100, True),      # G=2
    (1, 32, 8, 600, 128, 0, 0, True),       # first chunk: plain causal prefill through the cache
    (70, 4, 2, 4, 64, 1, 120, True),        # more sequences than lanes: launch order by index
])
def test_paged_chunk(B, Hq, Hkv, Nq, d, lo, hi, causal):
    dev = need_gpu()
    announce(f"paged prefill B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} cached[{lo},{hi}] "
             f"causal={causal}")
    inp = inputs.paged_inputs(31, B, Hq, Hkv, Nq, d, lo, hi, spare_blocks=3)
    g, o, lse, kp, vp = _append_and_run(inp, dev, causal)
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(d), causal,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "paged prefill")


@pytest.mark.parametrize("B,Hq,Hkv,Nq,d,L,lens", [
    (2, 8, 2, 70, 128, 400, [400, 70]),
    (3, 8, 8, 33, 64, 200, [200, 33, 150]),
    (2, 8, 2, 70, 128, 1600, [1537, 1100]),  # more than 64 blocks of 16 tokens
])
def test_contiguous_chunk(B, Hq, Hkv, Nq, d, L, lens):
    dev = need_gpu()
    announce(f"contiguous-cache prefill B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} L={L} lens={lens}")
    q, kc, vc, sl = inputs.decode_contig_inputs(32, B, Hq, Hkv, Nq, d, L, lens)
    o, lse = eta.attn_prefill_paged(q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev), causal=True)
    torch.cuda.synchronize()
    O, Lr = oracle.decode_attention(q, kc, vc, sl, scale_of(d), True)
    check(o, O, lse, Lr, "bf16", "contiguous-cache prefill")


@pytest.mark.parametrize("cached,hidden", [
    (150, ((0, 2), (1, 7))),
    # past the first 64 blocks of a sequence, and at the 64-block boundary
    (1400, ((0, 63), (0, 64), (1, 70))),
])
def test_invalid_table_entries_hide_their_keys(cached, hidden):
    dev = need_gpu()
    announce(f"paged prefill with -1 / out-of-range table entries {hidden}, B=2 Hq=4 Hkv=1 Nq=40 "
             f"d=128 cached={cached}")
    inp = inputs.paged_inputs(33, 2, 4, 1, 40, 128, cached, cached, spare_blocks=0)
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    table = inp["block_table"].clone()
    for i, (b, blk) in enumerate(hidden):
        table[b, blk] = -1 if i % 2 == 0 else inp["num_blocks"] + 3
    o, lse = eta.attn_prefill_paged(inp["q"].to(dev), kp.to(dev), vp.to(dev),
                                    inp["seq_lens"].to(dev), block_table=table.to(dev),
                                    causal=True)
    torch.cuda.synchronize()
    # the oracle sees the same keys minus the hidden blocks, at their positions
    Nq = 40
    O = np.zeros((2, Nq, 4, 128))
    L = np.zeros((2, 4, Nq))
    for b in (0, 1):
        n = int(inp["seq_lens"][b])
        hide = {blk for bb, blk in hidden if bb == b}
        keep = [t for t in range(n) if t // 16 not in hide]
        K = oracle.gather_paged(kp, inp["block_table"][b], n)
        V = oracle.gather_paged(vp, inp["block_table"][b], n)
        for hq in range(4):
            for i in range(Nq):
                pos = n - Nq + i
                vis = [t for t in keep if t <= pos]
                ob, lb = oracle.attention_rows(inp["q"][b, i:i + 1, hq], [len(vis) - 1],
                                               K[vis, 0], V[vis, 0], scale_of(128), True)
                O[b, i, hq] = ob[0]
                L[b, hq, i] = lb[0]
    check(o, O, lse, L, "bf16", "hidden blocks")


def test_nan_in_unused_cache_rows_does_not_leak():
    dev = need_gpu()
    announce("paged prefill with NaN spare blocks and NaN tail slots, B=3 Hq=8 Hkv=2 Nq=50 d=128")
    inp = inputs.paged_inputs(34, 3, 8, 2, 50, 128, 30, 200, spare_blocks=16)
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    inp["k_pool"], inp["v_pool"] = kp, vp
    assert inputs.poison_unused(inp) > 0
    g = _dev(inp, dev)
    o, lse = eta.attn_prefill_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                    block_table=g["block_table"], causal=True)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(128), True,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "poisoned pool")


@pytest.mark.parametrize("cache_lens,waves", [
    ((60, 30), 8), ((60, 30), 4),   # 5 and 4 blocks: the longest row ends 3 blocks into a tile
    ((92, 8, 40), 8),               # 7, 2 and 4 blocks
])
def test_table_row_ends_inside_a_tile(cache_lens, waves):
    """A tile's four table entries are read as one group; where the table row ends
    inside the last tile the reads past it stay inside the row and those blocks
    (past the sequence) hide nothing and read nothing: NaN in every block the
    table does not name must not reach the output."""
    dev = need_gpu()
    B = len(cache_lens)
    announce(f"paged prefill, table rows ending inside a tile, cached {cache_lens}, "
             f"Nq=20, waves={waves}")
    inp = inputs.paged_inputs(35, B, 8, 2, 20, 128, 0, 0, spare_blocks=8, cache_lens=cache_lens)
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    inp["k_pool"], inp["v_pool"] = kp, vp
    assert inputs.poison_unused(inp) > 0
    assert inp["block_table"].shape[1] % 4 != 0
    g = _dev(inp, dev)
    o, lse = eta.attn_prefill_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                    block_table=g["block_table"], causal=True, waves=waves)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(128), True,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "table row ends inside a tile")


def test_prompt_in_chunks_matches_full_prefill():
    """A 700-token prompt processed as chunks of 256, 256, 188 (kv_append, then
    attention against the paged cache) gives the rows of one causal prefill."""
    dev = need_gpu()
    announce("prompt of 700 tokens in chunks of 256 vs one causal prefill, Hq=8 Hkv=2 d=128")
    n, Hq, Hkv, d = 700, 8, 2, 128
    q, k, v = inputs.prefill_inputs(35, 1, Hq, Hkv, n, n, d, "bf16", "cpu")  # [1,H,N,d]
    nblk = (n + 15) // 16
    perm = torch.randperm(nblk + 4, generator=torch.Generator().manual_seed(36)).to(torch.int32)
    table = perm[:nblk].view(1, nblk)
    kp = torch.zeros((nblk + 4, 16, Hkv, d), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    kp_d, vp_d, tab_d = kp.to(dev), vp.to(dev), table.to(dev)
    Ofull, Lfull = oracle.prefill_attention(q, k, v, scale_of(d), True, 0)
    done = 0
    for r in (256, 256, 188):
        kn = k[:, :, done:done + r].transpose(1, 2).contiguous().to(dev)  # [1, r, Hkv, d]
        vn = v[:, :, done:done + r].transpose(1, 2).contiguous().to(dev)
        eta.kv_append(kn, vn, kp_d, vp_d, torch.tensor([done], dtype=torch.int32, device=dev),
                      block_table=tab_d)
        done += r
        qc = q[:, :, done - r:done].transpose(1, 2).contiguous().to(dev)  # [1, r, Hq, d]
        o, lse = eta.attn_prefill_paged(qc, kp_d, vp_d,
                                        torch.tensor([done], dtype=torch.int32, device=dev),
                                        block_table=tab_d, causal=True)
        torch.cuda.synchronize()
        check(o.transpose(1, 2), Ofull[:, :, done - r:done], lse, Lfull[:, :, done - r:done],
              "bf16", f"chunk ending at {done}")


def test_deterministic_and_guard_bands():
    dev = need_gpu()
    announce("paged prefill determinism + guard bands, B=2 Hq=32 Hkv=8 Nq=300 d=128")
    inp = _dev(inputs.paged_inputs(37, 2, 32, 8, 300, 128, 100, 900), dev)
    buf_o, o = nan_guarded(inp["q"].shape, torch.bfloat16, dev)
    buf_l, lse = nan_guarded((2, 32, 300), torch.float32, dev)
    eta.attn_prefill_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                           block_table=inp["block_table"], out=o, lse=lse)
    o1, l1 = o.clone(), lse.clone()
    for _ in range(5):
        eta.attn_prefill_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                               block_table=inp["block_table"], out=o, lse=lse)
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l1.view(torch.int32))
    torch.cuda.synchronize()
    assert guards_intact(buf_o) and guards_intact(buf_l)


def test_chunked_prefill_workload_every_element():
    """The 8 x 512-token chunked prefill at full size, in the launch the bench
    times: every output element and LSE of all 8 sequences x 32 heads."""
    dev = need_gpu()
    w = inputs.WORKLOADS["chunked_prefill_paged"]
    announce(f"workload chunked_prefill_paged: B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} "
             f"Nq={w['Nq']} d={w['d']} cached U[{w['len_lo']},{w['len_hi']}], append then prefill")
    inp = inputs.workload_inputs("chunked_prefill_paged", dev)
    eta.kv_append(inp["k_new"], inp["v_new"], inp["k_pool"], inp["v_pool"], inp["cache_lens"],
                  block_table=inp["block_table"])
    o, lse = eta.attn_prefill_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                                    block_table=inp["block_table"], causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    table = inp["block_table"].cpu()
    seq = inp["seq_lens"].cpu()
    G = w["Hq"] // w["Hkv"]
    Nq = w["Nq"]
    qc = inp["q"].cpu()
    rows = np.arange(Nq)
    for b in range(w["B"]):
        n = int(seq[b])
        nblk = (n + 15) // 16
        blocks = table[b, :nblk].long()
        kb = inp["k_pool"][blocks.to(dev)].cpu()
        vb = inp["v_pool"][blocks.to(dev)].cpu()
        local = torch.arange(nblk, dtype=torch.int32)
        K = oracle.gather_paged(kb, local, n)
        V = oracle.gather_paged(vb, local, n)
        for hq in range(w["Hq"]):
            O, L = oracle.attention_rows(qc[b, :, hq], n - Nq + rows, K[:, hq // G],
                                         V[:, hq // G], scale_of(w["d"]), True)
            check(o[b, :, hq], O, lse[b, hq], L, "bf16", f"b={b} hq={hq}")
