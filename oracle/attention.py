"""Plain fp64 attention: the definition written out (test infrastructure only).

Nothing here is tiled or streamed. For each query row the whole score row and
the whole probability row exist at once; rows are processed in blocks of at
most ``ROW_BLOCK`` only so that a 32k-key problem fits in host memory.
"""

import numpy as np

NEG_INF = -np.inf
ROW_BLOCK = 2048


def _f64(x):
    """Exact upcast of stored inputs (f32, bf16 via torch, or numpy) to fp64."""
    if hasattr(x, "detach"):  # a torch tensor: bf16 has no numpy dtype
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, pos, k, v, scale, causal):
    """Exact attention for a set of query rows against one key/value head.

    Definition ("Phase 07 · 12 … Flash Attention", section "tiling trick":
    S = Q Kᵀ, P = softmax(S), O = P V; "大模型面试笔记——Attention篇" §4: the
    scores are scaled by 1/√h before the softmax, here the explicit ``scale``).

    q     [R, d]  query rows
    pos   [R]     absolute position of each row; with ``causal`` row i sees
                  key j iff j <= pos[i] ("Effizienz", section "Der wichtige
                  Maskenfehler beim Cache": a query that is shorter than the
                  keys needs the offset, not a top-left triangle)
    k, v  [n, d]  keys and values
    Returns O [R, d] and LSE [R] (natural log of the sum of exp over the
    visible scaled scores). A row that sees no key gets O = 0, LSE = -inf.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    pos = np.asarray(pos, dtype=np.int64)
    R, d = q.shape
    n = k.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full((R,), NEG_INF, dtype=np.float64)
    if n == 0 or R == 0:
        return out, lse
    for r0 in range(0, R, ROW_BLOCK):
        r1 = min(R, r0 + ROW_BLOCK)
        # S: every score of these rows, in full.
        S = scale * (q[r0:r1] @ k.T)
        if causal:
            hidden = np.arange(n)[None, :] > pos[r0:r1, None]
            S[hidden] = NEG_INF
        # Safe softmax over the whole row ("大模型面试笔记" §2): subtract the
        # row maximum before exponentiating.
        m = S.max(axis=1)
        seen = np.isfinite(m)
        E = np.exp(S - np.where(seen, m, 0.0)[:, None])  # exp(-inf) = 0
        lsum = E.sum(axis=1)
        P = np.zeros_like(E)
        P[seen] = E[seen] / lsum[seen, None]
        out[r0:r1] = P @ v
        lse[r0:r1] = np.where(seen, m + np.log(np.where(seen, lsum, 1.0)), NEG_INF)
    return out, lse


def prefill_attention(q, k, v, scale, causal, q_offset=0, heads=None, rows=None):
    """Prefill over whole prompts, layout (batch, heads, seq, head_dim).

    The layout is the one the SDPA call on "[BEE-30062]" (section
    "為所有 GPU 訓練和推論啟用 FlashAttention-2") documents. Query head hq reads
    K/V head hq // (Hq/Hkv): the grouping that repeat_interleave along the head
    axis produces ("Effizienz", section "GQA im leicht lesbaren Code").

    q [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d]. Row i of a head sits at absolute
    position i + q_offset. ``heads`` (list of (b, hq)) and ``rows`` (index
    array into Nq) restrict the work to a sample; the returned arrays then hold
    NaN everywhere else.
    Returns O [B, Hq, Nq, d] and LSE [B, Hq, Nq] in fp64.
    """
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sample = heads is not None or rows is not None
    fill = np.nan if sample else 0.0
    O = np.full((B, Hq, Nq, v.shape[3]), fill, dtype=np.float64)
    LSE = np.full((B, Hq, Nq), fill, dtype=np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    for b, hq in heads:
        g = hq // G
        o, l = attention_rows(q[b, hq][idx], idx + q_offset, k[b, g], v[b, g], scale, causal)
        O[b, hq, idx] = o
        LSE[b, hq, idx] = l
    return O, LSE


def decode_attention(q, k_cache, v_cache, seq_lens, scale, causal, block_table=None,
                     block_size=16, heads=None):
    """Decode of Nq new tokens per sequence against a (paged or contiguous) cache.

    q [B, Nq, Hq, d] ("[BEE-30062]", section "為長上下文推論啟用 FlashDecoding":
    query (batch, 1, n_heads, head_dim) and caches (batch, seqlen_cache,
    n_kv_heads, head_dim) with per-sequence real lengths). ``seq_lens[b]``
    counts every visible key, the Nq new ones included. Query row i of
    sequence b sits at position seq_lens[b] - Nq + i ("Effizienz", section
    "Der wichtige Maskenfehler beim Cache").

    With ``block_table`` the caches are pools [num_blocks, 16, Hkv, d] and the
    keys of sequence b are gathered through its table row by this package's
    own gather ("Phase 07 · 12", section "Paged attention"); without it the
    caches are contiguous [B, max_len, Hkv, d].
    Returns O [B, Nq, Hq, d] and LSE [B, Hq, Nq] in fp64 (NaN outside a
    ``heads`` sample of (b, hq) pairs).
    """
    from .paged import gather_contiguous, gather_paged

    B, Nq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sample = heads is not None
    fill = np.nan if sample else 0.0
    O = np.full((B, Nq, Hq, v_cache.shape[3]), fill, dtype=np.float64)
    LSE = np.full((B, Hq, Nq), fill, dtype=np.float64)
    want = {}
    for b, hq in (heads if sample else [(b, h) for b in range(B) for h in range(Hq)]):
        want.setdefault(b, []).append(hq)
    seq_lens = [int(x) for x in np.asarray(_f64(seq_lens)).reshape(-1)]
    for b, hqs in want.items():
        n = seq_lens[b]
        if block_table is None:
            K = gather_contiguous(k_cache, b, n)
            V = gather_contiguous(v_cache, b, n)
        else:
            K = gather_paged(k_cache, block_table[b], n, block_size)
            V = gather_paged(v_cache, block_table[b], n, block_size)
        pos = n - Nq + np.arange(Nq)
        for hq in hqs:
            g = hq // G
            o, l = attention_rows(q[b, :, hq, :], pos, K[:, g, :], V[:, g, :], scale, causal)
            O[b, :, hq, :] = o
            LSE[b, hq, :] = l
    return O, LSE


def combine_partials(O_parts, LSE_parts):
    """Merge attention results computed over disjoint key chunks.

    "[BEE-30062]", section "Background": Flash-Decoding splits K/V along the
    sequence, processes the chunks in parallel and reduces the partial softmax
    results in a numerically stable way. Chunk s holds its own normalised
    output O_s and log-sum-exp LSE_s; the whole-row result is
        LSE = log Σ_s exp(LSE_s),   O = Σ_s exp(LSE_s - LSE) · O_s,
    evaluated after subtracting max_s LSE_s. Empty chunks (LSE_s = -inf) add
    nothing. O_parts [S, R, d], LSE_parts [S, R] -> O [R, d], LSE [R].
    """
    O_parts = _f64(O_parts)
    LSE_parts = _f64(LSE_parts)
    top = LSE_parts.max(axis=0)
    seen = np.isfinite(top)
    shift = np.where(seen, top, 0.0)
    w = np.exp(LSE_parts - shift[None, :])  # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=0)
    lse = np.where(seen, shift + np.log(np.where(seen, tot, 1.0)), NEG_INF)
    coef = np.zeros_like(w)
    coef[:, seen] = w[:, seen] / tot[None, seen]
    O = np.einsum("sr,srd->rd", coef, O_parts)
    return O, lse
