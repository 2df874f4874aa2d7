"""Counting helpers of the oracle (test infrastructure).

* KV-cache size: "Effizienz" (tokenwerk), section "Cachebedarf berechnen":
  M_KV = 2 · L · B · T · Hkv · d · e bytes (the 2 for the separate K and V
  arrays). The same product appears per token and layer on "Phase 07 · 12",
  section "Concept / pre-computation", and on "[BEE-30062]", section
  "部署使用 GQA 的模型以減輕 KV 快取記憶體壓力".
* Visible query-key pairs: counted by brute force over the mask, the quantity
  behind "step t compares against t tokens" ("Phase 07 · 12", "Build it,
  step 3").
* K/V states computed by a naive decoder (recomputes the whole prefix at every
  step) and by a cached decoder (computes each token once), same section.
"""


def kv_cache_bytes(L, B, T, Hkv, d, e):
    """Bytes of a K/V cache for L layers, batch B, T stored positions."""
    return 2 * L * B * T * Hkv * d * e


def visible_pairs(nq, nk, causal, q_offset=0):
    """Number of (query row, key) pairs the mask lets through, counted one by one."""
    total = 0
    for i in range(nq):
        for j in range(nk):
            if not causal or j <= i + q_offset:
                total += 1
    return total


def naive_vs_cached_kv_states(n_tokens, d=8, seed=0):
    """Run a one-head toy decoder twice: recomputing K/V, and with a K/V cache.

    Each step t (1-based) takes the t-th input vector, projects a query, and
    attends over the keys/values of tokens 1..t ("大模型面试笔记——Attention篇"
    §4). The naive decoder projects K and V again for the whole prefix at
    every step; the cached one appends only the new token's K and V
    ("Phase 07 · 12", "Build it, step 1/3"). Projections are counted as they
    are made.
    Returns (naive_states, cached_states, naive_outputs, cached_outputs);
    the outputs are [n_tokens, d] fp64 arrays that must agree.
    """
    import numpy as np

    from .attention import attention_rows

    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_tokens, d))
    wq, wk, wv = (rng.standard_normal((d, d)) for _ in range(3))
    scale = 1.0 / np.sqrt(d)

    naive_states = 0
    naive_out = np.zeros((n_tokens, d))
    for t in range(n_tokens):
        ks, vs = [], []
        for s in range(t + 1):  # recompute every prefix state
            ks.append(x[s] @ wk)
            vs.append(x[s] @ wv)
            naive_states += 1
        o, _ = attention_rows((x[t] @ wq)[None], [t], np.array(ks), np.array(vs), scale, True)
        naive_out[t] = o[0]

    cached_states = 0
    cache_k, cache_v = [], []
    cached_out = np.zeros((n_tokens, d))
    for t in range(n_tokens):
        cache_k.append(x[t] @ wk)  # the only new projection this step
        cache_v.append(x[t] @ wv)
        cached_states += 1
        o, _ = attention_rows((x[t] @ wq)[None], [t], np.array(cache_k), np.array(cache_v),
                              scale, True)
        cached_out[t] = o[0]
    return naive_states, cached_states, naive_out, cached_out
