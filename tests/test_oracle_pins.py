"""Pins of the fp64 oracle against what the pages and the mathematics fix.

CPU only. Each test names the passage it follows. None of these compares the
oracle with itself: the pins are worked values printed on the pages, closed
forms, invariants, brute force with Python scalars, and library routines
(torch's SDPA in fp64 with an explicit mask, torch.logsumexp,
repeat_interleave) on inputs where they compute the same thing.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_flashattention_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked values printed on the pages
# ---------------------------------------------------------------------------

def test_kv_cache_formula_worked_values():
    # "Effizienz", "Cachebedarf berechnen"; "Phase 07 · 12" concept section;
    # "[BEE-30062]" GQA deployment section.
    for c in _load("kv_cache_sizes.json")["cases"]:
        got = oracle.kv_cache_bytes(c["L"], c["B"], c["T"], c["Hkv"], c["d"], c["e"])
        assert got == c["bytes"], c["cite"]
    assert oracle.kv_cache_bytes(6, 1, 1024, 2, 64, 2) == 3 * 1024 * 1024


def test_pair_counts_match_pages():
    # "Phase 07 · 12", "Build it, step 3": step t compares against t tokens.
    for c in _load("decode_counts.json")["query_key_comparisons"]:
        n = c["n_tokens"]
        assert oracle.visible_pairs(n, n, causal=True) == c["pairs"]
    assert oracle.visible_pairs(7, 7, causal=False) == 49
    # offset mask: 4 new rows after 16 cached keys see 17, 18, 19, 20 keys
    assert oracle.visible_pairs(4, 20, causal=True, q_offset=16) == 17 + 18 + 19 + 20


def test_naive_and_cached_decoders_agree_and_count():
    # "Phase 07 · 12", "Build it, step 3" and exercise 1: same outputs, and
    # 5050 vs 100 K/V states for 100 tokens.
    for c in _load("decode_counts.json")["kv_states"]:
        naive, cached, out_naive, out_cached = oracle.naive_vs_cached_kv_states(c["n_tokens"])
        assert naive == c["naive"] and cached == c["cached"]
        np.testing.assert_allclose(out_cached, out_naive, rtol=0, atol=1e-13)
    naive, cached, _, _ = oracle.naive_vs_cached_kv_states(10)
    assert (naive, cached) == (55, 10)


# ---------------------------------------------------------------------------
# Invariants of the softmax
# ---------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal,off", [(False, 0), (True, 0), (True, 5)])
def test_probability_rows(causal, off):
    # With V = identity the output row IS the probability row P_i
    # ("大模型面试笔记" §2; "Attention éclair" FAQ): P >= 0, rows sum to 1,
    # masked entries exactly 0.
    n, R, d = 13, 8, 6
    q = _rand((R, d), 1)
    k = _rand((n, d), 2)
    pos = np.arange(R) + off
    P, _ = oracle.attention_rows(q, pos, k, np.eye(n), 0.7, causal)
    assert (P >= 0).all()
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14 * n)
    if causal:
        for i in range(R):
            assert (P[i, pos[i] + 1:] == 0).all()
            assert (P[i, : pos[i] + 1] > 0).all()


def test_online_equals_full_for_every_tile_size():
    # "Phase 07 · 12" step 2 / "大模型面试笔记" §2: the running (max, sum)
    # loop gives the full-softmax result. Every tile size 1..n, including
    # sizes that do not divide n.
    n, R, d = 23, 5, 4
    q = _rand((R, d), 3)
    k = _rand((n, d), 4)
    v = _rand((n, d), 5)
    pos = np.array([0, 3, 11, 17, 22])
    for causal in (False, True):
        O, L = oracle.attention_rows(q, pos, k, v, 0.5, causal)
        for tile in range(1, n + 1):
            Ot, Lt = oracle.online_attention_rows(q, pos, k, v, 0.5, causal, tile)
            np.testing.assert_allclose(Ot, O, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Lt, L, rtol=1e-12, atol=1e-13)


def test_online_equals_full_when_max_rises_every_tile():
    # Scores increasing in j (and scaled x10) make every tile raise the
    # running max, so every rescale factor is exercised.
    n, d = 40, 3
    q = np.array([[1.0, 0.0, 0.0]])
    k = np.zeros((n, d))
    k[:, 0] = 10.0 * np.arange(n) / n
    v = _rand((n, d), 6)
    O, L = oracle.attention_rows(q, [n - 1], k, v, 1.0, False)
    for tile in (1, 2, 3, 7, 40):
        Ot, Lt = oracle.online_attention_rows(q, [n - 1], k, v, 1.0, False, tile)
        np.testing.assert_allclose(Ot, O, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(Lt, L, rtol=1e-12)


# ---------------------------------------------------------------------------
# Library routines and brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("Nq,Nk,causal", [(9, 9, True), (9, 9, False), (3, 11, True), (1, 6, True)])
def test_matches_torch_sdpa_fp64_with_explicit_mask(Nq, Nk, causal):
    # "[BEE-30062]" SDPA call, layout (batch, heads, seq, head_dim); the mask
    # is given explicitly with the bottom-right offset, because SDPA's
    # is_causal is aligned top-left ("Effizienz", "Der wichtige Maskenfehler").
    B, Hq, Hkv, d = 2, 6, 2, 5
    g = torch.Generator().manual_seed(7)
    q = torch.randn(B, Hq, Nq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    off = Nk - Nq
    scale = 0.37
    O, L = oracle.prefill_attention(q.numpy(), k.numpy(), v.numpy(), scale, causal, off)
    kr = k.repeat_interleave(Hq // Hkv, dim=1)
    vr = v.repeat_interleave(Hq // Hkv, dim=1)
    mask = torch.ones(Nq, Nk, dtype=torch.bool)
    if causal:
        mask = torch.arange(Nk)[None, :] <= (torch.arange(Nq)[:, None] + off)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = scale * (q @ kr.transpose(-1, -2))
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12, atol=1e-12)


def test_brute_force_python_scalars():
    # The plain definition with Python floats and math.exp, tiny shapes.
    rng = np.random.default_rng(11)
    for Nq, Nk, d in [(1, 1, 1), (2, 3, 2), (6, 6, 4), (3, 6, 3), (5, 2, 4)]:
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, d))
        scale = 0.9
        for causal in (False, True):
            off = Nk - Nq
            pos = np.arange(Nq) + off
            O, L = oracle.attention_rows(q, pos, k, v, scale, causal)
            for i in range(Nq):
                vis = [j for j in range(Nk) if (not causal) or j <= i + off]
                if not vis:
                    assert L[i] == -math.inf and (O[i] == 0).all()
                    continue
                sc = {j: scale * sum(float(q[i, t]) * float(k[j, t]) for t in range(d)) for j in vis}
                top = max(sc.values())
                w = {j: math.exp(s - top) for j, s in sc.items()}
                z = sum(w.values())
                for t in range(d):
                    ref = sum(w[j] / z * float(v[j, t]) for j in vis)
                    assert abs(O[i, t] - ref) <= 1e-13
                assert abs(L[i] - (top + math.log(z))) <= 1e-13


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def test_closed_form_single_key():
    q = _rand((4, 5), 12)
    k = _rand((1, 5), 13)
    v = _rand((1, 5), 14)
    O, L = oracle.attention_rows(q, np.arange(4), k, v, 0.3, True)
    np.testing.assert_allclose(O, np.repeat(v, 4, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L, 0.3 * (q @ k[0]), rtol=1e-14)


@pytest.mark.parametrize("off", [0, 1, 4, 9])
def test_closed_form_zero_query_pins_mask_offset(off):
    # Q = 0: all visible scores are 0, so P is uniform over the visible keys:
    # O = mean of the visible V rows and LSE = ln(#visible) exactly.
    n, R, d = 12, 3, 4
    v = _rand((n, d), 15)
    k = _rand((n, d), 16)
    pos = np.arange(R) + off
    O, L = oracle.attention_rows(np.zeros((R, d)), pos, k, v, 1.0, True)
    for i in range(R):
        cnt = min(n, pos[i] + 1)
        np.testing.assert_allclose(O[i], v[:cnt].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(L[i] - math.log(cnt)) < 1e-14


def test_closed_form_two_keys_is_sigmoid():
    q = _rand((6, 3), 17)
    k = _rand((2, 3), 18)
    v = _rand((2, 3), 19)
    scale = 1.3
    O, L = oracle.attention_rows(q, np.full(6, 1), k, v, scale, True)
    s = scale * (q @ k.T)
    p0 = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    np.testing.assert_allclose(O, p0[:, None] * v[0] + (1 - p0)[:, None] * v[1], atol=1e-14)
    np.testing.assert_allclose(L, np.logaddexp(s[:, 0], s[:, 1]), atol=1e-14)


def test_row_with_no_visible_key():
    # No page covers it; the m = -inf guard of the tiled loop leaves the row
    # empty: O = 0, LSE = -inf, no NaN.
    O, L = oracle.attention_rows(_rand((2, 3), 20), [-1, 0], _rand((4, 3), 21),
                                 _rand((4, 3), 22), 1.0, True)
    assert (O[0] == 0).all() and L[0] == -math.inf
    assert np.isfinite(O).all() and np.isfinite(L[1])


# ---------------------------------------------------------------------------
# Mask offset, cached decode, GQA, split combine
# ---------------------------------------------------------------------------

def test_decode_rows_equal_last_rows_of_full_prefill():
    # "Effizienz", "Der wichtige Maskenfehler beim Cache".
    n, Nq, d = 30, 4, 8
    q = _rand((1, 2, n, d), 23)
    k = _rand((1, 1, n, d), 24)
    v = _rand((1, 1, n, d), 25)
    Ofull, Lfull = oracle.prefill_attention(q, k, v, 0.4, True, 0)
    Odec, Ldec = oracle.prefill_attention(q[:, :, n - Nq:], k, v, 0.4, True, n - Nq)
    np.testing.assert_allclose(Odec, Ofull[:, :, n - Nq:], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Ldec, Lfull[:, :, n - Nq:], rtol=1e-13, atol=1e-14)
    # the top-left triangle (offset 0) is the pitfall: a different answer
    Owrong, _ = oracle.prefill_attention(q[:, :, n - Nq:], k, v, 0.4, True, 0)
    assert np.abs(Owrong - Ofull[:, :, n - Nq:]).max() > 1e-3


@pytest.mark.parametrize("step", [1, 4, 17, 40])
def test_cached_paged_decode_equals_full_recompute(step):
    # "Phase 07 · 12" exercise 1 and "Effizienz" extension plan: decode with a
    # growing (here paged) cache, each K/V appended once, and compare every
    # position with a full causal recompute. Steps of 17 (chunks that straddle
    # 16-token blocks, ragged last chunk) and 40 (the whole prompt as one
    # chunk) are chunked prefill against the paged cache.
    n, Hq, Hkv, d = 40, 4, 2, 8
    q = _rand((1, Hq, n, d), 26)
    k = _rand((1, Hkv, n, d), 27)
    v = _rand((1, Hkv, n, d), 28)
    Ofull, Lfull = oracle.prefill_attention(q, k, v, 0.35, True, 0)
    nblk = 4
    perm = np.random.default_rng(29).permutation(nblk + 2)
    table = perm[:nblk][None, :]
    kp = np.full((nblk + 2, 16, Hkv, d), np.nan)
    vp = np.full((nblk + 2, 16, Hkv, d), np.nan)
    filled = 0
    while filled < n:
        r = min(step, n - filled)
        newk = k[:, :, filled:filled + r].transpose(0, 2, 1, 3)
        newv = v[:, :, filled:filled + r].transpose(0, 2, 1, 3)
        kp = oracle.kv_append_ref(kp, newk, table, [filled])
        vp = oracle.kv_append_ref(vp, newv, table, [filled])
        filled += r
        qd = q[:, :, filled - r:filled].transpose(0, 2, 1, 3)  # [1, r, Hq, d]
        Od, Ld = oracle.decode_attention(qd, kp, vp, [filled], 0.35, True, block_table=table)
        np.testing.assert_allclose(Od.transpose(0, 2, 1, 3), Ofull[:, :, filled - r:filled],
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Ld, Lfull[:, :, filled - r:filled], rtol=1e-13, atol=1e-14)


def test_gqa_equals_mha_on_repeat_interleaved_kv():
    # "Effizienz", "GQA im leicht lesbaren Code".
    B, Hq, Hkv, N, d = 2, 8, 2, 10, 4
    q = _rand((B, Hq, N, d), 30)
    k = _rand((B, Hkv, N, d), 31)
    v = _rand((B, Hkv, N, d), 32)
    O, L = oracle.prefill_attention(q, k, v, 0.5, True)
    kr = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1).numpy()
    vr = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1).numpy()
    O2, L2 = oracle.prefill_attention(q, kr, vr, 0.5, True)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    # and it is not the modulo mapping
    kw = np.stack([k[:, h % Hkv] for h in range(Hq)], axis=1)
    vw = np.stack([v[:, h % Hkv] for h in range(Hq)], axis=1)
    O3, _ = oracle.prefill_attention(q, kw, vw, 0.5, True)
    assert np.abs(O3 - O).max() > 1e-3


def test_split_combine_equals_unsplit():
    # "[BEE-30062]" Background: Flash-Decoding splits along the key sequence
    # and reduces the partial softmax results stably.
    rng = np.random.default_rng(33)
    n, R, d = 37, 6, 5
    q = rng.standard_normal((R, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    pos = np.array([0, 5, 16, 20, 35, 36])
    O, L = oracle.attention_rows(q, pos, k, v, 0.8, True)
    for trial in range(20):
        cuts = sorted(rng.choice(np.arange(0, n + 1), size=rng.integers(1, 6)))
        edges = [0] + list(cuts) + [n]
        Os, Ls = [], []
        for a, b in zip(edges[:-1], edges[1:]):  # may include empty chunks
            # chunk of keys a..b-1: keys keep their absolute positions
            o, l = oracle.attention_rows(q, pos - a, k[a:b], v[a:b], 0.8, True)
            Os.append(o)
            Ls.append(l)
        Oc, Lc = oracle.combine_partials(np.array(Os), np.array(Ls))
        np.testing.assert_allclose(Oc, O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Lc, L, rtol=1e-12, atol=1e-13)
    # all chunks empty -> empty row
    Oe, Le = oracle.combine_partials(np.zeros((3, 1, d)), np.full((3, 1), -np.inf))
    assert (Oe == 0).all() and Le[0] == -np.inf


# ---------------------------------------------------------------------------
# Paged gather and append, bit-exact
# ---------------------------------------------------------------------------

def _bits(t):
    return t.contiguous().view(torch.int16).numpy()


def test_paged_gather_is_bit_exact():
    # "Phase 07 · 12", "Paged attention": 16-token blocks + page table.
    inp = inputs.paged_inputs(40, B=5, Hq=4, Hkv=2, Nq=2, d=8, len_lo=1, len_hi=70)
    pool = inp["k_pool"]
    table = inp["block_table"]
    for b in range(5):
        n = int(inp["seq_lens"][b])
        got = oracle.gather_paged(pool, table[b], n)
        # the same rows addressed one by one: position t -> (table[t//16], t%16)
        ref = torch.stack([pool[int(table[b, t // 16]), t % 16] for t in range(n)])
        np.testing.assert_array_equal(_bits(got), _bits(ref))


def test_contiguous_cache_is_the_identity_table_case():
    B, L, Hkv, d = 2, 48, 2, 4
    cache = torch.randn(B, L, Hkv, d).to(torch.bfloat16)
    pool = cache.reshape(B * L // 16, 16, Hkv, d)
    table = torch.arange(B * L // 16, dtype=torch.int32).reshape(B, L // 16)
    for b in range(B):
        np.testing.assert_array_equal(_bits(oracle.gather_paged(pool, table[b], 37)),
                                      _bits(oracle.gather_contiguous(cache, b, 37)))


def test_kv_append_round_trip_and_untouched_bytes():
    inp = inputs.paged_inputs(41, B=4, Hq=4, Hkv=2, Nq=3, d=8, len_lo=5, len_hi=60,
                              spare_blocks=3)
    pool = inp["k_pool"]
    out = oracle.kv_append_ref(pool, inp["k_new"], inp["block_table"], inp["cache_lens"])
    touched = torch.zeros(pool.shape[:2], dtype=torch.bool)
    for b in range(4):
        c = int(inp["cache_lens"][b])
        got = oracle.gather_paged(out, inp["block_table"][b], c + 3)
        np.testing.assert_array_equal(_bits(got[c:]), _bits(inp["k_new"][b]))
        np.testing.assert_array_equal(_bits(got[:c]),
                                      _bits(oracle.gather_paged(pool, inp["block_table"][b], c)))
        for t in range(c, c + 3):
            touched[int(inp["block_table"][b, t // 16]), t % 16] = True
    np.testing.assert_array_equal(_bits(out[~touched]), _bits(pool[~touched]))
