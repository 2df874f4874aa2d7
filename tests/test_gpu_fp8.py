"""GPU parity of the fp8 (E4M3) K/V cache: kv_append_fp8 bit for bit against the
oracle's encoder, and attn_decode_paged_fp8 against the oracle's decode over
the dequantised cache (any Nq, G*Nq up to 64, paged and contiguous, invalid
table entries, NaN codes in unused rows), plus the 32-sequence 4-token decode
over an fp8 cache on sampled (sequence, head) pairs at full size."""

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from exact_tiled_attention_flashattention_amd import inputs
from tests.gpu_helpers import announce, check, guards_intact, nan_guarded, need_gpu, scale_of

pytestmark = pytest.mark.gpu


def _dev(inp, dev):
    return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in inp.items()}


def _np(t):
    return t.detach().cpu().float().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("B,Hkv,Nnew,d,paged", [
    (3, 4, 5, 128, True),
    (2, 2, 33, 64, True),
    (2, 8, 4, 128, False),
])
def test_append_is_bit_exact(B, Hkv, Nnew, d, paged):
    dev = need_gpu()
    announce(f"kv_append_fp8 B={B} Hkv={Hkv} Nnew={Nnew} d={d} paged={paged}")
    inp = inputs.paged_inputs_fp8(41, B, 2 * Hkv, Hkv, Nnew, d, 10, 90, spare_blocks=2)
    # new rows spanning the whole range: normal values, tiny ones, and ones
    # that saturate (|x / scale| > 448)
    g = torch.Generator().manual_seed(42)
    kn = torch.randn((B, Nnew, Hkv, d), generator=g) * 3.0
    kn[..., :4] = torch.tensor([1e-4, -3e-3, 40.0, -1e3])
    vn = torch.randn((B, Nnew, Hkv, d), generator=g) * 0.5
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    ks, vs = inp["k_scale"], inp["v_scale"]
    if paged:
        kp, vp, table = inp["k_pool"].clone(), inp["v_pool"].clone(), inp["block_table"]
        L = table.shape[1] * 16
    else:
        L = int(inp["seq_lens"].max()) + 3
        kp = torch.randint(0, 127, (B, L, Hkv, d), dtype=torch.uint8, generator=g)
        vp = torch.randint(0, 127, (B, L, Hkv, d), dtype=torch.uint8, generator=g)
        table = None
    kd, vd = kp.to(dev), vp.to(dev)
    eta.kv_append_fp8(kn.to(dev), vn.to(dev), kd, vd, ks.to(dev), vs.to(dev),
                      inp["cache_lens"].to(dev),
                      block_table=None if table is None else table.to(dev))
    torch.cuda.synchronize()
    if table is None:  # the contiguous cache is the identity table over [B, L] rows
        nb = L // 16 + 1
        pool_k = torch.zeros((B * nb, 16, Hkv, d), dtype=torch.uint8)
        pool_v = torch.zeros_like(pool_k)
        pool_k.view(B, nb * 16, Hkv, d)[:, :L] = kp
        pool_v.view(B, nb * 16, Hkv, d)[:, :L] = vp
        tab = np.arange(B * nb).reshape(B, nb)
        want_k = oracle.kv_append_ref(pool_k.numpy(), oracle.quantize(_np(kn), _np(ks)), tab,
                                      _np(inp["cache_lens"]))
        want_v = oracle.kv_append_ref(pool_v.numpy(), oracle.quantize(_np(vn), _np(vs)), tab,
                                      _np(inp["cache_lens"]))
        want_k = want_k.reshape(B, nb * 16, Hkv, d)[:, :L]
        want_v = want_v.reshape(B, nb * 16, Hkv, d)[:, :L]
    else:
        want_k = oracle.kv_append_ref(kp.numpy(), oracle.quantize(_np(kn), _np(ks)),
                                      table.numpy(), _np(inp["cache_lens"]))
        want_v = oracle.kv_append_ref(vp.numpy(), oracle.quantize(_np(vn), _np(vs)),
                                      table.numpy(), _np(inp["cache_lens"]))
    assert np.array_equal(kd.cpu().numpy(), want_k)
    assert np.array_equal(vd.cpu().numpy(), want_v)


def _reference(inp, causal, d):
    kq = oracle.dequantize(_np(inp["k_pool"]), _np(inp["k_scale"]))
    vq = oracle.dequantize(_np(inp["v_pool"]), _np(inp["v_scale"]))
    return oracle.decode_attention(inp["q"], kq, vq, inp["seq_lens"], scale_of(d), causal,
                                   block_table=inp["block_table"])


@pytest.mark.parametrize("B,Hq,Hkv,Nq,d,lo,hi,causal,splits", [
    (3, 8, 2, 4, 128, 20, 300, True, 0),
    (2, 32, 8, 1, 128, 700, 1500, True, 0),
    (2, 32, 8, 4, 64, 33, 100, True, 3),
    (4, 4, 4, 8, 128, 1, 70, False, 1),
    (2, 32, 4, 4, 128, 100, 700, True, 0),    # 32 rows per K/V head: two groups
    (2, 16, 1, 4, 64, 40, 300, True, 5),      # 64 rows, four groups
    (130, 8, 2, 4, 128, 10, 120, True, 0),    # more sequences than a wave's 64 lanes
])
def test_decode_matches_dequantised_oracle(B, Hq, Hkv, Nq, d, lo, hi, causal, splits):
    dev = need_gpu()
    announce(f"fp8 decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} d={d} len[{lo},{hi}] causal={causal} "
             f"splits={splits}")
    inp = inputs.paged_inputs_fp8(43, B, Hq, Hkv, Nq, d, lo, hi, spare_blocks=3)
    g = _dev(inp, dev)
    o, lse = eta.attn_decode_paged_fp8(g["q"], g["k_pool"], g["v_pool"], g["k_scale"],
                                       g["v_scale"], g["seq_lens"], block_table=g["block_table"],
                                       scale=scale_of(d), causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    O, L = _reference(inp, causal, d)
    check(o, O, lse, L, "bf16", "fp8 decode")


def test_contiguous_fp8_cache():
    dev = need_gpu()
    announce("fp8 decode, contiguous cache B=2 Hq=8 Hkv=2 Nq=2 d=128 L=300")
    B, Hq, Hkv, Nq, d, L = 2, 8, 2, 2, 128, 300
    g = torch.Generator().manual_seed(44)
    kc = (torch.randn((B, L, Hkv, d), generator=g) * 60).clamp(-448, 448)
    vc = (torch.randn((B, L, Hkv, d), generator=g) * 60).clamp(-448, 448)
    kc = kc.to(torch.float8_e4m3fn).view(torch.uint8)
    vc = vc.to(torch.float8_e4m3fn).view(torch.uint8)
    q = torch.randn((B, Nq, Hq, d), generator=g).to(torch.bfloat16)
    sl = torch.tensor([300, 77], dtype=torch.int32)
    ks = inputs.fp8_scales(Hkv)
    vs = inputs.fp8_scales(Hkv) * 2
    o, lse = eta.attn_decode_paged_fp8(q.to(dev), kc.to(dev), vc.to(dev), ks.to(dev), vs.to(dev),
                                       sl.to(dev), causal=True)
    torch.cuda.synchronize()
    O, Lr = oracle.decode_attention(q, oracle.dequantize(kc.numpy(), ks.numpy()),
                                    oracle.dequantize(vc.numpy(), vs.numpy()), sl, scale_of(d),
                                    True)
    check(o, O, lse, Lr, "bf16", "contiguous fp8")


def test_nan_codes_and_invalid_entries_do_not_leak():
    dev = need_gpu()
    announce("fp8 decode with NaN codes in unused rows and a -1 table entry, B=3 Hq=8 Hkv=2 Nq=4")
    inp = inputs.paged_inputs_fp8(45, 3, 8, 2, 4, 128, 40, 200, spare_blocks=8)
    assert inputs.poison_unused(inp, value=0x7F) > 0  # 0x7F is a NaN code
    table = inp["block_table"].clone()
    table[1, 1] = -1
    g = _dev(inp, dev)
    buf_o, o = nan_guarded(inp["q"].shape, torch.bfloat16, dev)
    o, lse = eta.attn_decode_paged_fp8(g["q"], g["k_pool"], g["v_pool"], g["k_scale"],
                                       g["v_scale"], g["seq_lens"], block_table=table.to(dev),
                                       causal=True, out=o)
    torch.cuda.synchronize()
    assert guards_intact(buf_o)
    # the oracle sees the same cache with sequence 1's block 1 removed
    kq = oracle.dequantize(_np(inp["k_pool"]), _np(inp["k_scale"]))
    vq = oracle.dequantize(_np(inp["v_pool"]), _np(inp["v_scale"]))
    O, L = oracle.decode_attention(inp["q"], kq, vq, inp["seq_lens"], scale_of(128), True,
                                   block_table=inp["block_table"])
    n = int(inp["seq_lens"][1])
    keep = [t for t in range(n) if t // 16 != 1]
    K = oracle.gather_paged(kq, inp["block_table"][1], n)[keep]
    V = oracle.gather_paged(vq, inp["block_table"][1], n)[keep]
    for hq in range(8):
        pos = [len(keep) - 4 + i for i in range(4)]
        ob, lb = oracle.attention_rows(inp["q"][1, :, hq], pos, K[:, hq // 4], V[:, hq // 4],
                                       scale_of(128), True)
        O[1, :, hq] = ob
        L[1, hq] = lb
    check(o, O, lse, L, "bf16", "fp8 with NaN codes and a hidden block")


def test_fp8_workload_every_element():
    """The paged 4-token decode over E4M3 codes at full size: every output
    element and LSE of all 32 sequences x 32 heads, and every appended code."""
    dev = need_gpu()
    w = inputs.WORKLOADS["paged_decode_q4_fp8"]
    announce(f"workload paged_decode_q4_fp8: B={w['B']} Hq={w['Hq']} Hkv={w['Hkv']} Nq=4 "
             f"d={w['d']}, append then decode over E4M3 codes")
    inp = inputs.workload_inputs("paged_decode_q4_fp8", dev)
    eta.kv_append_fp8(inp["k_new"], inp["v_new"], inp["k_pool"], inp["v_pool"], inp["k_scale"],
                      inp["v_scale"], inp["cache_lens"], block_table=inp["block_table"])
    o, lse = eta.attn_decode_paged_fp8(inp["q"], inp["k_pool"], inp["v_pool"], inp["k_scale"],
                                       inp["v_scale"], inp["seq_lens"],
                                       block_table=inp["block_table"], causal=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    table = inp["block_table"].cpu()
    seq = inp["seq_lens"].cpu()
    ks, vs = _np(inp["k_scale"]), _np(inp["v_scale"])
    G = w["Hq"] // w["Hkv"]
    knew = _np(inp["k_new"].cpu())
    qc = inp["q"].cpu()
    vnew = _np(inp["v_new"].cpu())
    for b in range(w["B"]):
        n = int(seq[b])
        nblk = (n + 15) // 16
        blocks = table[b, :nblk].long()
        kb = inp["k_pool"][blocks.to(dev)].cpu().numpy()
        vb = inp["v_pool"][blocks.to(dev)].cpu().numpy()
        local = np.arange(nblk)
        K = oracle.dequantize(oracle.gather_paged(kb, local, n), ks)
        V = oracle.dequantize(oracle.gather_paged(vb, local, n), vs)
        # the appended rows are the oracle's codes of the new rows
        codes = oracle.gather_paged(kb, local, n)[n - 4:]
        assert np.array_equal(codes, oracle.quantize(knew[b], ks))
        assert np.array_equal(oracle.gather_paged(vb, local, n)[n - 4:],
                              oracle.quantize(vnew[b], vs))
        for hq in range(w["Hq"]):
            O, L = oracle.attention_rows(qc[b, :, hq], n - 4 + np.arange(4),
                                         K[:, hq // G], V[:, hq // G], scale_of(w["d"]), True)
            check(o[b, :, hq], O, lse[b, hq], L, "bf16", f"b={b} hq={hq}")
