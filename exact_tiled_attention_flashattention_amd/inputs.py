"""Seeded synthetic inputs, shared by the tests, the bench and the checker.

This module draws random tensors and builds page tables; it holds none of the
attention arithmetic. Values are f32 draws from N(0, 1) cast to bf16 with
round-to-nearest-even (or kept in f32). One ``torch.Generator`` per call,
seeded by the caller, draws every tensor in a fixed order, so a (seed, shape,
device) triple always yields the same bytes.

The five named workloads (``WORKLOADS``) are the shapes the library is
measured on: single-head fp32 attention, causal GQA prefill at 4k and 32k
tokens (32 query heads over 8 K/V heads, head dim 128), split-KV decode of
one token against 16 contiguous 32k-token caches, and 4-token decode against
a 16-token-block paged cache with random block placement and per-sequence
lengths drawn uniformly from [1024, 16384].
"""

import math

import torch

BLOCK = 16  # tokens per physical cache block

WORKLOADS = {
    "single_head_f32": dict(seed=1001, kind="prefill", B=1, Hq=1, Hkv=1, N=256, d=64,
                            dtype="f32", causal=False),
    "causal_gqa_prefill_4k": dict(seed=1002, kind="prefill", B=1, Hq=32, Hkv=8, N=4096,
                                  d=128, dtype="bf16", causal=True),
    "causal_gqa_prefill_32k": dict(seed=1003, kind="prefill", B=1, Hq=32, Hkv=8, N=32768,
                                   d=128, dtype="bf16", causal=True),
    "splitkv_decode_32k": dict(seed=1004, kind="decode_contig", B=16, Hq=32, Hkv=8, Nq=1,
                               d=128, seq_len=32768, dtype="bf16"),
    "paged_decode_q4": dict(seed=1005, kind="decode_paged", B=32, Hq=32, Hkv=8, Nq=4, d=128,
                            len_lo=1024, len_hi=16384, dtype="bf16"),
    # the paged 4-token decode over an E4M3 cache with per-head scales
    "paged_decode_q4_fp8": dict(seed=1007, kind="decode_paged_fp8", B=32, Hq=32, Hkv=8, Nq=4,
                                d=128, len_lo=1024, len_hi=16384, dtype="bf16"),
    # the paged 4-token decode at head dim 64 (its byte counters show that
    # only the heads' own rows are read)
    "paged_decode_q4_d64": dict(seed=1010, kind="decode_paged", B=32, Hq=32, Hkv=8, Nq=4, d=64,
                                len_lo=1024, len_hi=16384, dtype="bf16"),
    # chunked prefill: a 512-token chunk per sequence appended after a cached
    # prefix, then attending to the whole paged cache
    "chunked_prefill_paged": dict(seed=1006, kind="prefill_paged", B=8, Hq=32, Hkv=8, Nq=512,
                                  d=128, len_lo=1024, len_hi=8192, dtype="bf16"),
    # the backward pass of the 4k causal GQA prefill (q, k, v, then dO)
    "causal_gqa_backward_4k": dict(seed=1009, kind="backward", B=1, Hq=32, Hkv=8, N=4096,
                                   d=128, dtype="bf16", causal=True),
}

# 1000 chat completions served from a cache of 65536 token positions (8 GiB
# for a 32-layer model with 8 K/V heads of dim 128 in bf16: 128 KiB per
# token); prompt and output lengths uniform on [32, 2048]; a contiguous
# allocator that cannot know the output length reserves 2048 new tokens
CHAT_SIM = dict(seed=1008, chats=1000, prompt_lo=32, prompt_hi=2048, output_lo=32,
                output_hi=2048, capacity_tokens=65536, max_new_tokens=2048)


def chat_lengths(seed, chats, prompt_lo, prompt_hi, output_lo, output_hi, **_):
    """Prompt and output lengths of `chats` chat completions, each uniform on
    its inclusive integer range, drawn prompts first. Returns two int lists."""
    g = _gen(seed, "cpu")
    p = torch.randint(prompt_lo, prompt_hi + 1, (chats,), generator=g)
    r = torch.randint(output_lo, output_hi + 1, (chats,), generator=g)
    return [int(x) for x in p], [int(x) for x in r]


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, dtype, device):
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    return x if dtype == torch.float32 else x.to(dtype)


def backward_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype="bf16", device="cpu"):
    """q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d], dout [B,Hq,Nq,d] (the gradient of
    the loss with respect to O), drawn in that order from one generator."""
    g = _gen(seed, device)
    dt = torch_dtype(dtype)
    q = _normal((B, Hq, Nq, d), g, dt, device)
    k = _normal((B, Hkv, Nk, d), g, dt, device)
    v = _normal((B, Hkv, Nk, d), g, dt, device)
    dout = _normal((B, Hq, Nq, d), g, dt, device)
    return q, k, v, dout


def prefill_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype="bf16", device="cpu"):
    """q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d], drawn in that order."""
    dt = torch_dtype(dtype)
    g = _gen(seed, device)
    q = _normal((B, Hq, Nq, d), g, dt, device)
    k = _normal((B, Hkv, Nk, d), g, dt, device)
    v = _normal((B, Hkv, Nk, d), g, dt, device)
    return q, k, v


def decode_contig_inputs(seed, B, Hq, Hkv, Nq, d, max_len, seq_lens=None, dtype="bf16",
                         device="cpu"):
    """q [B,Nq,Hq,d]; caches [B,max_len,Hkv,d]; seq_lens [B] int32 (default: all full).

    Draw order: k_cache, v_cache, q.
    """
    dt = torch_dtype(dtype)
    g = _gen(seed, device)
    k = _normal((B, max_len, Hkv, d), g, dt, device)
    v = _normal((B, max_len, Hkv, d), g, dt, device)
    q = _normal((B, Nq, Hq, d), g, dt, device)
    if seq_lens is None:
        seq_lens = [max_len] * B
    sl = torch.tensor(list(seq_lens), dtype=torch.int32, device=device)
    return q, k, v, sl


def paged_inputs(seed, B, Hq, Hkv, Nq, d, len_lo, len_hi, spare_blocks=0, dtype="bf16",
                 device="cpu", cache_lens=None):
    """A paged cache with random block placement, plus the Nq new tokens.

    Draw order on one CPU generator (seed): cached lengths c_b uniform on the
    integers [len_lo, len_hi] (unless ``cache_lens`` is given), a random
    permutation of the pool's blocks. Then on the target device's generator
    (same seed): the K and V pools, the new K/V rows, the queries.
    Sequence b ends up with seq_len_b = c_b + Nq tokens after the append and
    owns ceil(seq_len_b / 16) blocks, taken in order from the permutation;
    unused table entries are -1. ``spare_blocks`` extra blocks that no table
    references are added to the pool.

    Returns a dict: q [B,Nq,Hq,d], k_pool/v_pool [P,16,Hkv,d],
    k_new/v_new [B,Nq,Hkv,d], block_table [B,max_blocks] int32,
    cache_lens [B] int32, seq_lens [B] int32, num_blocks P.
    """
    dt = torch_dtype(dtype)
    gc = _gen(seed, "cpu")
    if cache_lens is None:
        c = torch.randint(len_lo, len_hi + 1, (B,), generator=gc, dtype=torch.int64)
    else:
        c = torch.tensor(list(cache_lens), dtype=torch.int64)
    seq = c + Nq
    nblk = [(int(s) + BLOCK - 1) // BLOCK for s in seq]
    used = sum(nblk)
    P = used + spare_blocks
    perm = torch.randperm(P, generator=gc)
    max_blocks = max(nblk) if nblk else 1
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    at = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[at : at + nblk[b]].to(torch.int32)
        at += nblk[b]
    g = _gen(seed, device)
    k_pool = _normal((P, BLOCK, Hkv, d), g, dt, device)
    v_pool = _normal((P, BLOCK, Hkv, d), g, dt, device)
    k_new = _normal((B, Nq, Hkv, d), g, dt, device)
    v_new = _normal((B, Nq, Hkv, d), g, dt, device)
    q = _normal((B, Nq, Hq, d), g, dt, device)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new,
                block_table=table.to(device), cache_lens=c.to(torch.int32).to(device),
                seq_lens=seq.to(torch.int32).to(device), num_blocks=P)


def fp8_scales(Hkv, device="cpu"):
    """Per-K/V-head scales of a synthetic E4M3 cache: head h's codes stand for
    values of standard deviation about 0.5 + h / Hkv."""
    return torch.tensor([(6.0 / 448.0) * (0.5 + h / Hkv) for h in range(Hkv)],
                        dtype=torch.float32, device=device)


def paged_inputs_fp8(seed, B, Hq, Hkv, Nq, d, len_lo, len_hi, spare_blocks=0, device="cpu",
                     cache_lens=None):
    """``paged_inputs`` with an E4M3 cache: the same lengths, table, new bf16
    K/V rows and bf16 queries, while the pools hold codes. The codes are
    standard normal draws times 448/6, clamped to the finite range and cast to
    float8_e4m3fn, so with ``fp8_scales`` head h's cached values are about
    N(0, (0.5 + h/Hkv)^2). Adds k_scale, v_scale [Hkv] f32."""
    inp = paged_inputs(seed, B, Hq, Hkv, Nq, d, len_lo, len_hi, spare_blocks, "bf16", device,
                       cache_lens)
    g = _gen(seed + 7919, device)
    P = inp["num_blocks"]
    for name in ("k_pool", "v_pool"):
        x = torch.randn((P, BLOCK, Hkv, d), generator=g, dtype=torch.float32, device=device)
        x = (x * (448.0 / 6.0)).clamp_(-448.0, 448.0)
        inp[name] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        del x
    inp["k_scale"] = fp8_scales(Hkv, device)
    inp["v_scale"] = fp8_scales(Hkv, device)
    return inp


def poison_unused(inp, value=float("nan")):
    """Fill every pool row that no sequence uses (spare blocks, tail slots past
    seq_len) with ``value``; returns the number of rows touched."""
    table = inp["block_table"].cpu()
    seq = inp["seq_lens"].cpu()
    P = inp["num_blocks"]
    live = torch.zeros((P, BLOCK), dtype=torch.bool)
    for b in range(table.shape[0]):
        n = int(seq[b])
        for i in range(math.ceil(n / BLOCK)):
            blk = int(table[b, i])
            live[blk, : min(BLOCK, n - i * BLOCK)] = True
    dead = (~live).to(inp["k_pool"].device)
    for key in ("k_pool", "v_pool"):
        inp[key][dead] = value
    return int((~live).sum())


def workload_inputs(name, device="cpu"):
    """Inputs of one named workload (see ``WORKLOADS``)."""
    w = WORKLOADS[name]
    if w["kind"] == "prefill":
        return prefill_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["N"], w["d"],
                              w["dtype"], device)
    if w["kind"] == "backward":
        return backward_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["N"], w["d"],
                               w["dtype"], device)
    if w["kind"] == "decode_contig":
        return decode_contig_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["Nq"], w["d"],
                                    w["seq_len"], None, w["dtype"], device)
    if w["kind"] == "decode_paged_fp8":
        return paged_inputs_fp8(w["seed"], w["B"], w["Hq"], w["Hkv"], w["Nq"], w["d"],
                                w["len_lo"], w["len_hi"], 0, device)
    return paged_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["Nq"], w["d"], w["len_lo"],
                        w["len_hi"], 0, w["dtype"], device)
