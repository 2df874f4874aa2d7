"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE, not the product.

This package is the independent checker of the HIP path. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (the C-ABI library and its Python binding) never
imports, links or calls anything here, and this package imports nothing from
the product: the two share no kernels, helpers, constants or pre/post
processing. Inputs reach both sides from the seeded generators, which hold none
of the method's arithmetic.

What it computes is the plain definition of attention (no tiling, no online
softmax): every entry of a query row's score vector and probability vector
exists at once in fp64 and the softmax sees the whole row. Sources:

* "Phase 07 · 12: KV cache, Flash Attention and inference optimisation"
  (AI Engineering from Scratch), section "tiling trick": standard attention is
  S = Q Kᵀ, P = softmax(S), O = P V; section "Paged attention": 16-token
  blocks with a page table; "Build it, step 1": the per-layer/per-head cache
  with append/read; "Build it, step 2": the running (max, sum) loop.
* "大模型面试笔记——Attention篇" (juejin), §2 (online safe softmax) and §4
  (decode step: softmax(t_Q x_Kᵀ/√h)·x_V with x_K, x_V grown by concatenation).
* "[BEE-30062] FlashAttention 與高效注意力核心", section "Background"
  (Flash-Decoding's split of K/V along the sequence with a stable reduction of
  the partial softmax results) and section "為長上下文推論啟用 FlashDecoding"
  (cache layout (batch, seqlen, n_kv_heads, head_dim), per-sequence lengths).
* "Effizienz" (tokenwerk), sections "GQA im leicht lesbaren Code" (query head
  groups share a K/V head, repeat_interleave along the head axis),
  "Cachebedarf berechnen" (M_KV = 2·L·B·T·Hkv·d·e) and "Der wichtige
  Maskenfehler beim Cache" (the causal mask must carry a position offset when
  the query is shorter than the keys).
* backward.py: the gradients dQ, dK, dV of the same definition (the chain
  rule through S, softmax and P V; "Phase 07 · 12", section "tiling trick",
  notes that the backward pass recomputes forward values instead of storing
  them).
* pool.py: the paged cache's block pool as a plain set, and the chat-serving
  schedule of "Phase 07 · 12", section "Exercises" (item 3).
* fp8.py: the E4M3 encoding of a quantised K/V cache with per-head scales
  (the fp8 cache option of "Phase 07 · 12", section "Paged attention"; the
  encoding is the OCP 8-bit format, a reading stated in that module).

Every function here is pinned by CPU tests against values and identities that
the pages and the mathematics fix (tests/test_oracle_*.py); none is marked
"parity unpinned".
"""

from .attention import (
    NEG_INF,
    attention_rows,
    prefill_attention,
    decode_attention,
    combine_partials,
)
from .paged import gather_paged, gather_contiguous, kv_append_ref
from .online import online_attention_rows
from .counts import kv_cache_bytes, visible_pairs, naive_vs_cached_kv_states
from .fp8 import E4M3_MAX, e4m3_decode, e4m3_encode, quantize, dequantize
from .backward import attention_backward_rows, prefill_backward

__all__ = [
    "NEG_INF",
    "attention_rows",
    "prefill_attention",
    "decode_attention",
    "combine_partials",
    "gather_paged",
    "gather_contiguous",
    "kv_append_ref",
    "online_attention_rows",
    "kv_cache_bytes",
    "visible_pairs",
    "naive_vs_cached_kv_states",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "quantize",
    "dequantize",
    "attention_backward_rows",
    "prefill_backward",
]
