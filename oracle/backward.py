"""Gradients of exact attention, plain fp64 — TEST INFRASTRUCTURE.

What is differentiated is the definition the forward oracle writes out
("Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
section "tiling trick": S = Q Kᵀ scaled, P = softmax(S) row by row, O = P V;
the same section says the backward pass recomputes the forward's
intermediate values instead of storing them, so a tiled backward needs only
Q, K, V, O, the per-row log-sum-exp and dO). With a loss whose gradient with
respect to O is dO, the chain rule through those three steps gives, for one
query head against its K/V head (masked entries have P = 0):

    dV  = Pᵀ dO
    dP  = dO Vᵀ
    dS  = P ∘ (dP − D),   D_i = Σ_j P_ij dP_ij     (softmax Jacobian, row i)
    dQ  = scale · dS K
    dK  = scale · dSᵀ Q

D_i is written here as its definition; it equals dO_i · O_i because
O_i = Σ_j P_ij V_j. Under grouped-query attention a K/V head serves G query
heads ("Effizienz", "GQA im leicht lesbaren Code": repeat_interleave along
the head axis), so its dK and dV are the sums over those heads.

Every score row and probability row exists in full (no tiling); rows are
processed in blocks only to bound host memory.

With ``magnitudes=True`` the same loop also returns, per gradient element,
the sum of the absolute values of the terms it adds up (|dS| widened by the
error a once-rounded O puts into D): the scale against which the roundings of
a bf16 kernel (P and dS rounded for the matrix products, O stored in bf16)
are measured.
"""

import numpy as np

from .attention import NEG_INF, ROW_BLOCK, _f64


def attention_backward_rows(q, pos, k, v, dout, scale, causal, magnitudes=False):
    """Gradients for one query head's rows against one key/value head.

    q [R, d] at absolute positions pos [R] (causal: row i sees key j iff
    j <= pos[i]); k, v [n, d]; dout [R, dv] = dLoss/dO.
    Returns dq [R, d], dk [n, d], dv [n, dv] in fp64; with ``magnitudes``
    also (Mq, Mk, Mv) of the same shapes:
        Mv = Pᵀ |dO|,  Mq = scale (|dS| + P ∘ E) |K|,  Mk = scale (|dS| + P ∘ E)ᵀ |Q|,
    where E_i = Σ_d |dO_id| |O_id| (the size of D's terms).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    dout = _f64(dout)
    pos = np.asarray(pos, dtype=np.int64)
    R, d = q.shape
    n = k.shape[0]
    dq = np.zeros((R, d), dtype=np.float64)
    dk = np.zeros((n, d), dtype=np.float64)
    dv = np.zeros((n, v.shape[1]), dtype=np.float64)
    mq, mk, mv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    if n == 0 or R == 0:
        return (dq, dk, dv, (mq, mk, mv)) if magnitudes else (dq, dk, dv)
    for r0 in range(0, R, ROW_BLOCK):
        r1 = min(R, r0 + ROW_BLOCK)
        S = scale * (q[r0:r1] @ k.T)
        if causal:
            S[np.arange(n)[None, :] > pos[r0:r1, None]] = NEG_INF
        m = S.max(axis=1)
        seen = np.isfinite(m)
        E = np.exp(S - np.where(seen, m, 0.0)[:, None])
        P = np.zeros_like(E)
        P[seen] = E[seen] / E[seen].sum(axis=1, keepdims=True)
        dv += P.T @ dout[r0:r1]
        dP = dout[r0:r1] @ v.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        dq[r0:r1] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r0:r1])
        if magnitudes:
            Ei = (np.abs(dout[r0:r1]) * np.abs(P @ v)).sum(axis=1)
            W = np.abs(dS) + P * Ei[:, None]
            mv += P.T @ np.abs(dout[r0:r1])
            mq[r0:r1] = scale * (W @ np.abs(k))
            mk += scale * (W.T @ np.abs(q[r0:r1]))
    return (dq, dk, dv, (mq, mk, mv)) if magnitudes else (dq, dk, dv)


def prefill_backward(q, k, v, dout, scale, causal, q_offset=0, kv_heads=None, magnitudes=False):
    """Gradients of the prefill (layout (batch, heads, seq, head_dim)).

    q, dout [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d]; row i of a head sits at
    position i + q_offset. ``kv_heads`` (list of (b, g)) restricts the work to
    those K/V heads and their G query heads; everything else is NaN.
    Returns dQ [B, Hq, Nq, d], dK, dV [B, Hkv, Nk, d] in fp64 (and, with
    ``magnitudes``, their magnitude tensors as a fourth item).
    """
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    fill = np.nan if kv_heads is not None else 0.0
    dQ = np.full((B, Hq, Nq, d), fill, dtype=np.float64)
    dK = np.full((B, Hkv, Nk, d), fill, dtype=np.float64)
    dV = np.full((B, Hkv, Nk, v.shape[3]), fill, dtype=np.float64)
    if kv_heads is None:
        kv_heads = [(b, g) for b in range(B) for g in range(Hkv)]
    M = (np.full_like(dQ, fill), np.full_like(dK, fill), np.full_like(dV, fill))
    pos = np.arange(Nq) + q_offset
    for b, g in kv_heads:
        dK[b, g] = 0.0
        dV[b, g] = 0.0
        M[1][b, g] = 0.0
        M[2][b, g] = 0.0
        for hq in range(g * G, (g + 1) * G):
            res = attention_backward_rows(q[b, hq], pos, k[b, g], v[b, g], dout[b, hq], scale,
                                          causal, magnitudes)
            dQ[b, hq] = res[0]
            dK[b, g] += res[1]
            dV[b, g] += res[2]
            if magnitudes:
                M[0][b, hq] = res[3][0]
                M[1][b, g] += res[3][1]
                M[2][b, g] += res[3][2]
    return (dQ, dK, dV, M) if magnitudes else (dQ, dK, dV)
