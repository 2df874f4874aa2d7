"""GPU parity of kv_append + attn_decode_paged against the fp64 oracle.

Covers contiguous and paged caches, Nq in {1, 2, 4, 5, 8, 64}, group sizes 1..16
(G*Nq up to 64 rows, in groups of 16),
head dims 64/128, causal and not, explicit and default split counts, ragged
lengths, rows that see no key, invalid table entries, NaN-poisoned unused
cache rows, bitwise determinism and output guard bands; plus the split-KV
decode workload (16 x 32k contiguous) and the paged 4-token workload,
every output element, at full size in the launch the bench times.
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


@pytest.mark.parametrize("B,Hq,Hkv,Nq,d,lo,hi,causal,splits", [
    (3, 8, 2, 4, 128, 20, 300, True, 0),
    (3, 8, 2, 4, 128, 20, 300, False, 0),
    (2, 32, 8, 1, 128, 700, 1500, True, 0),
    (2, 32, 8, 4, 64, 33, 100, True, 3),
    (4, 4, 4, 8, 128, 1, 70, True, 1),       # G=1, Nq=8, one split
    (2, 16, 1, 1, 128, 16, 16, True, 0),     # G=16, block-aligned lengths
    (2, 8, 4, 2, 64, 1, 40, True, 50),       # more splits than 32-key steps
    (1, 4, 2, 4, 128, 3000, 3000, True, 7),
    # more than 16 rows per K/V head: groups of 16 rows
    (2, 32, 4, 4, 128, 100, 700, True, 0),    # G=8, Nq=4: 32 rows, 2 groups
    (2, 16, 1, 4, 64, 40, 300, True, 5),      # G=16, Nq=4: 64 rows, 4 groups
    (3, 8, 2, 5, 128, 5, 200, True, 0),       # G=4, Nq=5: 20 rows, ragged second group
    (2, 2, 2, 64, 128, 64, 400, True, 0),     # G=1, Nq=64: 64 query tokens, causal offsets
    (2, 32, 8, 8, 128, 50, 500, False, 3),    # G=4, Nq=8: 32 rows, not causal
    # more sequences than a wave's 64 lanes: the range search scans B in passes of 64
    (130, 8, 2, 1, 64, 1, 80, True, 0),
    (130, 8, 2, 4, 128, 10, 200, True, 333),
])
def test_paged_small(B, Hq, Hkv, Nq, d, lo, hi, causal, splits):
    dev = need_gpu()
    announce(f"paged decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} len[{lo},{hi}] causal={causal} "
             f"splits={splits}")
    inp = inputs.paged_inputs(21, B, Hq, Hkv, Nq, d, lo, hi, spare_blocks=5)
    g = _dev(inp, dev)
    eta.kv_append(g["k_new"], g["v_new"], g["k_pool"], g["v_pool"], g["cache_lens"],
                  block_table=g["block_table"])
    o, lse = eta.attn_decode_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                   block_table=g["block_table"], scale=scale_of(d), causal=causal,
                                   num_splits=splits)
    torch.cuda.synchronize()
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    # the append is a bit copy
    assert torch.equal(g["k_pool"].cpu().view(torch.int16), kp.view(torch.int16))
    assert torch.equal(g["v_pool"].cpu().view(torch.int16), vp.view(torch.int16))
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(d), causal,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "paged")


@pytest.mark.parametrize("B,Hq,Hkv,Nq,d,L,lens,splits", [
    (2, 8, 2, 1, 128, 500, [500, 37], 0),
    (3, 8, 8, 2, 64, 96, [96, 1, 50], 2),
    (1, 32, 8, 4, 128, 4100, [4100], 0),
])
def test_contiguous_small(B, Hq, Hkv, Nq, d, L, lens, splits):
    dev = need_gpu()
    announce(f"contiguous decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} L={L} lens={lens}")
    q, kc, vc, sl = inputs.decode_contig_inputs(22, B, Hq, Hkv, Nq, d, L, lens)
    o, lse = eta.attn_decode_paged(q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev), causal=True,
                                   num_splits=splits)
    torch.cuda.synchronize()
    O, Lr = oracle.decode_attention(q, kc, vc, sl, scale_of(d), True)
    check(o, O, lse, Lr, "bf16", "contiguous")


def test_invalid_table_entries_hide_their_keys():
    dev = need_gpu()
    announce("paged decode with -1 / out-of-range table entries, B=2 Hq=4 Hkv=1 Nq=1 d=128")
    inp = inputs.paged_inputs(23, 2, 4, 1, 1, 128, 100, 100, spare_blocks=0)
    table = inp["block_table"].clone()
    table[0, 2] = -1
    table[1, 4] = inp["num_blocks"] + 3
    g = _dev(inp, dev)
    o, lse = eta.attn_decode_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                   block_table=table.to(dev), causal=True)
    torch.cuda.synchronize()
    # the oracle sees the same keys minus the hidden blocks
    O = np.zeros((2, 1, 4, 128))
    L = np.zeros((2, 4, 1))
    for b, hide in ((0, 2), (1, 4)):
        n = int(inp["seq_lens"][b])
        keep = [t for t in range(n) if t // 16 != hide]
        K = oracle.gather_paged(inp["k_pool"], inp["block_table"][b], n)[keep]
        V = oracle.gather_paged(inp["v_pool"], inp["block_table"][b], n)[keep]
        for hq in range(4):
            ob, lb = oracle.attention_rows(inp["q"][b, :, hq], [len(keep) - 1], K[:, 0], V[:, 0],
                                           scale_of(128), True)
            O[b, :, hq] = ob
            L[b, hq] = lb
    check(o, O, lse, L, "bf16", "hidden blocks")


def test_nan_in_unused_cache_rows_does_not_leak():
    dev = need_gpu()
    announce("paged decode with NaN spare blocks and NaN tail slots, B=4 Hq=8 Hkv=2 Nq=4 d=128")
    inp = inputs.paged_inputs(24, 4, 8, 2, 4, 128, 30, 200, spare_blocks=16)
    # append first (the new rows are live), then poison every row nobody uses
    kp = oracle.kv_append_ref(inp["k_pool"], inp["k_new"], inp["block_table"], inp["cache_lens"])
    vp = oracle.kv_append_ref(inp["v_pool"], inp["v_new"], inp["block_table"], inp["cache_lens"])
    inp["k_pool"], inp["v_pool"] = kp, vp
    touched = inputs.poison_unused(inp)
    assert touched > 0
    g = _dev(inp, dev)
    o, lse = eta.attn_decode_paged(g["q"], g["k_pool"], g["v_pool"], g["seq_lens"],
                                   block_table=g["block_table"], causal=True)
    torch.cuda.synchronize()
    O, L = oracle.decode_attention(inp["q"], kp, vp, inp["seq_lens"], scale_of(128), True,
                                   block_table=inp["block_table"])
    check(o, O, lse, L, "bf16", "poisoned pool")


def test_decode_deterministic_and_guard_bands():
    dev = need_gpu()
    announce("paged decode determinism + guard bands, B=4 Hq=32 Hkv=8 Nq=4 d=128")
    inp = _dev(inputs.paged_inputs(25, 4, 32, 8, 4, 128, 500, 3000), dev)
    buf_o, o = nan_guarded(inp["q"].shape, torch.bfloat16, dev)
    buf_l, lse = nan_guarded((4, 32, 4), torch.float32, dev)
    eta.attn_decode_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                          block_table=inp["block_table"], out=o, lse=lse)
    o1, l1 = o.clone(), lse.clone()
    for _ in range(9):
        eta.attn_decode_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                              block_table=inp["block_table"], out=o, lse=lse)
        assert torch.equal(o.view(torch.int16), o1.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), l1.view(torch.int32))
    torch.cuda.synchronize()
    assert guards_intact(buf_o) and guards_intact(buf_l)


def test_splitkv_decode_32k_workload_every_element():
    """The 16 x 32k split-KV decode in the launch the bench times: every output
    element and LSE (16 sequences x 32 heads) against the oracle."""
    dev = need_gpu()
    w = inputs.WORKLOADS["splitkv_decode_32k"]
    announce(f"workload splitkv_decode_32k: B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Nq=1 "
             f"L={w['seq_len']} d={w['d']} contiguous, default splits, every element")
    q, kc, vc, sl = inputs.workload_inputs("splitkv_decode_32k", dev)
    o, lse = eta.attn_decode_paged(q, kc, vc, sl, causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    G = w["Hq"] // w["Hkv"]
    qc = q.cpu()
    for b in range(w["B"]):
        for g in range(w["Hkv"]):
            K, V = kc[b, :, g].cpu(), vc[b, :, g].cpu()
            for hq in range(g * G, (g + 1) * G):
                O, L = oracle.attention_rows(qc[b, :, hq], [w["seq_len"] - 1], K, V,
                                             scale_of(w["d"]), True)
                check(o[b, :, hq], O, lse[b, hq], L, "bf16", f"b={b} hq={hq}")


def test_paged_decode_q4_workload_every_element():
    """The paged 4-token decode in the launch the bench times (kv_append, then
    decode): every output element and LSE of all 32 sequences x 32 heads x 4
    rows, and the appended rows bit for bit."""
    dev = need_gpu()
    w = inputs.WORKLOADS["paged_decode_q4"]
    announce(f"workload paged_decode_q4: B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Nq=4 d={w['d']} "
             "kv_append then decode, every element")
    inp = inputs.workload_inputs("paged_decode_q4", dev)
    k_new_cpu = inp["k_new"].cpu()
    v_new_cpu = inp["v_new"].cpu()
    eta.kv_append(inp["k_new"], inp["v_new"], inp["k_pool"], inp["v_pool"], inp["cache_lens"],
                  block_table=inp["block_table"])
    o, lse = eta.attn_decode_paged(inp["q"], inp["k_pool"], inp["v_pool"], inp["seq_lens"],
                                   block_table=inp["block_table"], causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    table = inp["block_table"].cpu()
    seq = inp["seq_lens"].cpu()
    qc = inp["q"].cpu()
    G = w["Hq"] // w["Hkv"]
    for b in range(w["B"]):
        n = int(seq[b])
        nblk = (n + 15) // 16
        blocks = table[b, :nblk].long()
        kb = inp["k_pool"][blocks.to(dev)].cpu()  # this sequence's blocks, in table order
        vb = inp["v_pool"][blocks.to(dev)].cpu()
        local = torch.arange(nblk, dtype=torch.int32)
        K = oracle.gather_paged(kb, local, n)
        V = oracle.gather_paged(vb, local, n)
        # the appended rows are exactly the new ones
        assert torch.equal(K[n - 4:].view(torch.int16), k_new_cpu[b].view(torch.int16))
        assert torch.equal(V[n - 4:].view(torch.int16), v_new_cpu[b].view(torch.int16))
        for hq in range(w["Hq"]):
            O, L = oracle.attention_rows(qc[b, :, hq], n - 4 + np.arange(4), K[:, hq // G],
                                         V[:, hq // G], scale_of(w["d"]), True)
            check(o[b, :, hq], O, lse[b, hq], L, "bf16", f"b={b} hq={hq}")


@pytest.mark.parametrize("workers", [1, 2, 5, 13, 64, 1000])
def test_worker_split_boundaries_with_empty_sequences(workers):
    """Key steps of all (sequence, K/V head) segments are shared out evenly among
    the workers, so pieces start and end inside and across segments. Empty
    sequences contribute no steps; a workspace full of NaN shows any read of a
    piece that no worker wrote."""
    dev = need_gpu()
    lens = [0, 70, 1, 0, 33, 300, 16, 0]
    announce(f"contiguous decode, workers={workers}, lens={lens}, NaN-filled workspace")
    B, Hq, Hkv, Nq, d, L = len(lens), 8, 2, 1, 128, 320
    q, kc, vc, sl = inputs.decode_contig_inputs(26, B, Hq, Hkv, Nq, d, L, lens)
    need = eta.attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, L, workers)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev)
    o, lse = eta.attn_decode_paged(q.to(dev), kc.to(dev), vc.to(dev), sl.to(dev), causal=True,
                                   num_splits=workers, workspace=ws)
    torch.cuda.synchronize()
    O, Lr = oracle.decode_attention(q, kc, vc, sl, scale_of(d), True)
    check(o, O, lse, Lr, "bf16", f"workers={workers}")
