"""Pins of the oracle's attention gradients (CPU only).

The gradients are pinned to things other than the oracle's own formulas:
central finite differences of the forward oracle (a different code path: it
never forms dS), torch autograd through an independently written fp64
softmax-attention expression with an explicit bottom-right mask, closed
forms (one key; equal values), exact identities of the softmax Jacobian
(each row of dS sums to zero, so the keys' dK sum to zero; the keys' dV sum
to the visible rows' dO), the causal horizon, and the GQA sum over a group.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, dout, scale, causal, q_offset):
    """Σ dO ∘ O through the forward oracle: its gradient is (dQ, dK, dV)."""
    B, Hq, Nq, d = q.shape
    O, _ = oracle.prefill_attention(q, k, v, scale, causal, q_offset)
    return float((O * dout).sum())


@pytest.mark.parametrize("causal,q_offset,G", [(False, 0, 1), (True, 0, 2), (True, 3, 3)])
def test_finite_differences(causal, q_offset, G):
    rng = np.random.default_rng(5)
    B, Hkv, Nq, Nk, d = 1, 2, 5, 7, 3
    Hq = Hkv * G
    q = _rand(rng, B, Hq, Nq, d)
    k = _rand(rng, B, Hkv, Nk, d)
    v = _rand(rng, B, Hkv, Nk, d)
    do = _rand(rng, B, Hq, Nq, d)
    scale = 0.7
    dQ, dK, dV = ob.prefill_backward(q, k, v, do, scale, causal, q_offset)
    h = 1e-6
    for name, x, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = _loss(q, k, v, do, scale, causal, q_offset)
            x[idx] = old - h
            fm = _loss(q, k, v, do, scale, causal, q_offset)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(grad).max()), name


def _torch_grads(q, k, v, do, scale, causal, q_offset):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kk = tk.repeat_interleave(G, dim=1)
    vv = tv.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2))
    if causal:
        i = torch.arange(Nq)[:, None] + q_offset
        j = torch.arange(Nk)[None, :]
        s = s.masked_fill(j > i, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.matmul(p, vv)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal,q_offset", [(False, 0), (True, 0), (True, 37)])
def test_matches_torch_autograd(causal, q_offset):
    rng = np.random.default_rng(8)
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 29, 66, 16
    q = _rand(rng, B, Hq, Nq, d)
    k = _rand(rng, B, Hkv, Nk, d)
    v = _rand(rng, B, Hkv, Nk, d)
    do = _rand(rng, B, Hq, Nq, d)
    got = ob.prefill_backward(q, k, v, do, 0.25, causal, q_offset)
    ref = _torch_grads(q, k, v, do, 0.25, causal, q_offset)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())


def test_one_key_closed_form():
    # one key: P = 1 for every row, so O = V0 whatever Q, K are
    rng = np.random.default_rng(1)
    q = _rand(rng, 9, 4)
    k = _rand(rng, 1, 4)
    v = _rand(rng, 1, 4)
    do = _rand(rng, 9, 4)
    dq, dk, dv = ob.attention_backward_rows(q, np.arange(9), k, v, do, 0.5, False)
    assert np.abs(dq).max() == 0.0 and np.abs(dk).max() <= 1e-15
    assert np.allclose(dv[0], do.sum(axis=0), rtol=0, atol=1e-14)


def test_equal_values_closed_form():
    # every V row equal: O does not depend on the scores, so dQ = dK = 0
    rng = np.random.default_rng(2)
    q = _rand(rng, 6, 5)
    k = _rand(rng, 8, 5)
    v = np.tile(_rand(rng, 1, 5), (8, 1))
    do = _rand(rng, 6, 5)
    dq, dk, dv = ob.attention_backward_rows(q, np.arange(6) + 2, k, v, do, 0.9, True)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_jacobian_identities(causal):
    rng = np.random.default_rng(3)
    R, n, d = 40, 55, 8
    q = _rand(rng, R, d)
    k = _rand(rng, n, d)
    v = _rand(rng, n, d)
    do = _rand(rng, R, d)
    pos = np.arange(R) + (n - R)
    dq, dk, dv = ob.attention_backward_rows(q, pos, k, v, do, 0.3, causal)
    # each row of dS sums to zero, so Σ_j dK_j = scale Σ_i (Σ_j dS_ij) q_i = 0
    assert np.abs(dk.sum(axis=0)).max() <= 1e-12 * np.abs(dk).sum()
    # rows of P sum to one, so Σ_j dV_j = Σ_i dO_i (every row sees a key here)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-12)


def test_causal_horizon():
    # keys past every row's horizon get no gradient; a row's dQ ignores them
    rng = np.random.default_rng(4)
    R, n, d = 10, 30, 6
    q = _rand(rng, R, d)
    k = _rand(rng, n, d)
    v = _rand(rng, n, d)
    do = _rand(rng, R, d)
    pos = np.arange(R) + 5            # rows see keys 0..14 at most
    dq, dk, dv = ob.attention_backward_rows(q, pos, k, v, do, 0.4, True)
    assert np.abs(dk[15:]).max() == 0.0 and np.abs(dv[15:]).max() == 0.0
    dq2, dk2, dv2 = ob.attention_backward_rows(q, pos, k[:15], v[:15], do, 0.4, True)
    assert np.abs(dq - dq2).max() <= 1e-14
    assert np.abs(dk[:15] - dk2).max() <= 1e-14 and np.abs(dv[:15] - dv2).max() <= 1e-14


def test_gqa_sums_over_the_group():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, N, d = 1, 6, 2, 12, 4
    q = _rand(rng, B, Hq, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    do = _rand(rng, B, Hq, N, d)
    dQ, dK, dV = ob.prefill_backward(q, k, v, do, 0.5, True)
    # the same problem as MHA on repeated K/V heads, then summed per group
    kr = np.repeat(k, 3, axis=1)
    vr = np.repeat(v, 3, axis=1)
    mQ, mK, mV = ob.prefill_backward(q, kr, vr, do, 0.5, True)
    assert np.abs(dQ - mQ).max() <= 1e-14
    assert np.abs(dK - mK.reshape(B, Hkv, 3, N, d).sum(axis=2)).max() <= 1e-13
    assert np.abs(dV - mV.reshape(B, Hkv, 3, N, d).sum(axis=2)).max() <= 1e-13


def test_magnitudes_bound_the_gradients():
    # each magnitude is a sum of the absolute values of the gradient's terms,
    # so it bounds the gradient; it is zero exactly where every term is
    rng = np.random.default_rng(12)
    q = _rand(rng, 1, 4, 33, 8)
    k = _rand(rng, 1, 2, 40, 8)
    v = _rand(rng, 1, 2, 40, 8)
    do = _rand(rng, 1, 4, 33, 8)
    dQ, dK, dV, (mq, mk, mv) = ob.prefill_backward(q, k, v, do, 0.4, True, 0, magnitudes=True)
    for g, m in ((dQ, mq), (dK, mk), (dV, mv)):
        assert (np.abs(g) <= m * (1 + 1e-12) + 1e-300).all()
    assert (mk[:, :, 33:] == 0).all() and (mv[:, :, 33:] == 0).all()  # keys no row sees


def _brute_magnitudes(q, pos, k, v, do, scale, causal):
    """Every gradient element as an explicit list of its terms, with Python
    floats and math.exp; the magnitude is the sum of the terms' absolute
    values. dV_jc = Σ_i P_ij dO_ic; dQ_ic = scale Σ_j dS_ij K_jc and
    dK_jc = scale Σ_i dS_ij Q_ic, each term widened by P_ij E_i with
    E_i = Σ_c |dO_ic| |O_ic| (the size of the terms of D_i = dO_i · O_i)."""
    R, d = len(q), len(q[0])
    n, dv_ = len(k), len(v[0])
    vis = [[(not causal) or j <= pos[i] for j in range(n)] for i in range(R)]
    P = []
    for i in range(R):
        s = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in range(n)]
        seen = [s[j] for j in range(n) if vis[i][j]]
        if not seen:
            P.append([0.0] * n)
            continue
        mx = max(seen)
        e = [math.exp(s[j] - mx) if vis[i][j] else 0.0 for j in range(n)]
        tot = sum(e)
        P.append([x / tot for x in e])
    O = [[sum(P[i][j] * v[j][c] for j in range(n)) for c in range(dv_)] for i in range(R)]
    dP = [[sum(do[i][c] * v[j][c] for c in range(dv_)) for j in range(n)] for i in range(R)]
    D = [sum(P[i][j] * dP[i][j] for j in range(n)) for i in range(R)]
    dS = [[P[i][j] * (dP[i][j] - D[i]) for j in range(n)] for i in range(R)]
    E = [sum(abs(do[i][c]) * abs(O[i][c]) for c in range(dv_)) for i in range(R)]
    mv = [[sum(abs(P[i][j] * do[i][c]) for i in range(R)) for c in range(dv_)] for j in range(n)]
    mq = [[sum(abs(scale * dS[i][j] * k[j][c]) + scale * P[i][j] * E[i] * abs(k[j][c])
               for j in range(n)) for c in range(d)] for i in range(R)]
    mk = [[sum(abs(scale * dS[i][j] * q[i][c]) + scale * P[i][j] * E[i] * abs(q[i][c])
               for i in range(R)) for c in range(d)] for j in range(n)]
    return np.array(mq), np.array(mk), np.array(mv)


@pytest.mark.parametrize("causal,off", [(False, 0), (True, 1), (True, -1)])
def test_magnitudes_brute_force(causal, off):
    # exact from both sides: an inflated or deflated magnitude fails
    rng = np.random.default_rng(21)
    R, n, d = 4, 5, 3
    q, k, v, do = (_rand(rng, R, d), _rand(rng, n, d), _rand(rng, n, d), _rand(rng, R, d))
    pos = np.arange(R) + off
    *_, (mq, mk, mv) = ob.attention_backward_rows(q, pos, k, v, do, 0.7, causal, magnitudes=True)
    bq, bk, bv = _brute_magnitudes(q.tolist(), pos.tolist(), k.tolist(), v.tolist(),
                                   do.tolist(), 0.7, causal)
    for got, ref in ((mq, bq), (mk, bk), (mv, bv)):
        assert np.abs(got - ref).max() <= 1e-13 * max(1.0, np.abs(ref).max())


def test_magnitudes_one_key_closed_form():
    # one key: P = 1, O_i = V_0 and dS = 0, so every magnitude is a closed form:
    # Mv_0 = Σ_i |dO_i|, Mq_i = scale E_i |K_0|, Mk_0 = scale Σ_i E_i |Q_i| with
    # E_i = Σ_c |dO_ic| |V_0c|
    rng = np.random.default_rng(22)
    R, d, scale = 6, 4, 0.3
    q, k, v, do = (_rand(rng, R, d), _rand(rng, 1, d), _rand(rng, 1, d), _rand(rng, R, d))
    *_, (mq, mk, mv) = ob.attention_backward_rows(q, np.arange(R), k, v, do, scale, False,
                                                  magnitudes=True)
    E = np.abs(do) @ np.abs(v[0])
    assert np.allclose(mv[0], np.abs(do).sum(axis=0), rtol=1e-14, atol=0)
    assert np.allclose(mq, scale * E[:, None] * np.abs(k[0])[None, :], rtol=1e-14, atol=0)
    assert np.allclose(mk[0], scale * (E[:, None] * np.abs(q)).sum(axis=0), rtol=1e-14, atol=0)


def test_magnitudes_equal_the_gradient_when_terms_share_a_sign():
    # dO >= 0: every term of dV_jc = Σ_i P_ij dO_ic is >= 0, so Mv equals dV
    rng = np.random.default_rng(23)
    R, n, d = 7, 9, 5
    q, k, v = _rand(rng, R, d), _rand(rng, n, d), _rand(rng, n, d)
    do = np.abs(_rand(rng, R, d))
    dq, dk, dv, (mq, mk, mv) = ob.attention_backward_rows(q, np.arange(R) + 2, k, v, do, 0.5,
                                                          True, magnitudes=True)
    assert np.allclose(mv, dv, rtol=1e-13, atol=0)
    # V = 0: O = 0 and dP = 0, so dS = 0, E = 0 and Mq = Mk = 0 exactly
    *_, (mq0, mk0, _) = ob.attention_backward_rows(q, np.arange(R), k, 0 * v, do, 0.5, True,
                                                   magnitudes=True)
    assert (mq0 == 0).all() and (mk0 == 0).all()


def test_kv_head_sample_matches_full():
    rng = np.random.default_rng(9)
    q = _rand(rng, 2, 4, 9, 4)
    k = _rand(rng, 2, 2, 9, 4)
    v = _rand(rng, 2, 2, 9, 4)
    do = _rand(rng, 2, 4, 9, 4)
    full = ob.prefill_backward(q, k, v, do, 0.5, True)
    part = ob.prefill_backward(q, k, v, do, 0.5, True, kv_heads=[(1, 0)])
    assert np.array_equal(part[0][1, 0:2], full[0][1, 0:2])
    assert np.array_equal(part[1][1, 0], full[1][1, 0])
    assert np.isnan(part[1][0, 0]).all()


# ---- planted mistakes: each edit of the gradient code must fail a pin above ----

def _mutant(old, new):
    import os
    import types

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                        "backward.py")
    src = open(path).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle._bwd_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


BWD_MUTANTS = [
    ("D sign", "dS = P * (dP - D[:, None])", "dS = P * (dP + D[:, None])"),
    ("D without P", "D = (P * dP).sum(axis=1)", "D = dP.sum(axis=1) / dP.shape[1]"),
    ("dK scale dropped", "dk += scale * (dS.T @ q[r0:r1])", "dk += (dS.T @ q[r0:r1])"),
    ("dQ from V", "dq[r0:r1] = scale * (dS @ k)", "dq[r0:r1] = scale * (dS @ v)"),
    ("dV from the scores", "dv += P.T @ dout[r0:r1]", "dv += E.T @ dout[r0:r1]"),
    ("mask off by one", "S[np.arange(n)[None, :] > pos[r0:r1, None]] = NEG_INF",
     "S[np.arange(n)[None, :] >= pos[r0:r1, None]] = NEG_INF"),
    ("GQA group overwritten", "dK[b, g] += res[1]", "dK[b, g] = res[1]"),
]


@pytest.mark.parametrize("what,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, what, old, new):
    mod = _mutant(old, new)
    monkeypatch.setattr(ob, "attention_backward_rows", mod.attention_backward_rows)
    monkeypatch.setattr(ob, "prefill_backward", mod.prefill_backward)
    pins = [lambda: test_matches_torch_autograd(True, 37),
            lambda: test_matches_torch_autograd(False, 0),
            lambda: test_finite_differences(True, 3, 3)]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {what}"


MAG_MUTANTS = [
    ("W inflated x10", "W = np.abs(dS) + P * Ei[:, None]", "W = 10.0 * (np.abs(dS) + P * Ei[:, None])"),
    ("Mv inflated x4", "mv += P.T @ np.abs(dout[r0:r1])", "mv += 4.0 * (P.T @ np.abs(dout[r0:r1]))"),
    ("Mq inflated x2", "mq[r0:r1] = scale * (W @ np.abs(k))", "mq[r0:r1] = 2.0 * scale * (W @ np.abs(k))"),
    ("Mk inflated x2", "mk += scale * (W.T @ np.abs(q[r0:r1]))",
     "mk += 2.0 * scale * (W.T @ np.abs(q[r0:r1]))"),
    ("E term dropped", "W = np.abs(dS) + P * Ei[:, None]", "W = np.abs(dS)"),
    ("E from |V| not |O|", "Ei = (np.abs(dout[r0:r1]) * np.abs(P @ v)).sum(axis=1)",
     "Ei = (np.abs(dout[r0:r1]) * (P @ np.abs(v))).sum(axis=1)"),
    ("|dS| replaced by dS", "W = np.abs(dS) + P * Ei[:, None]", "W = dS + P * Ei[:, None]"),
]


@pytest.mark.parametrize("what,old,new", MAG_MUTANTS, ids=[m[0] for m in MAG_MUTANTS])
def test_planted_magnitude_mistake_is_caught(monkeypatch, what, old, new):
    mod = _mutant(old, new)
    monkeypatch.setattr(ob, "attention_backward_rows", mod.attention_backward_rows)
    monkeypatch.setattr(ob, "prefill_backward", mod.prefill_backward)
    pins = [lambda: test_magnitudes_brute_force(True, 1),
            lambda: test_magnitudes_one_key_closed_form(),
            lambda: test_magnitudes_equal_the_gradient_when_terms_share_a_sign()]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {what}"
