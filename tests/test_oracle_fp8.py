"""Pins of the E4M3 oracle (CPU): torch's float8_e4m3fn as an independent
library routine for every code and for in-range rounding, closed forms of the
format (largest value, one, smallest subnormal, ties to even, saturation),
round trips, and the quantisation error bound. Plus the quantised append
through the page table, bit for bit."""

import numpy as np
import pytest
import torch

import oracle


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256)
    ours = oracle.e4m3_decode(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_closed_forms():
    assert oracle.e4m3_decode([0x7E])[0] == 448.0          # S.1111.110
    assert np.isnan(oracle.e4m3_decode([0x7F])[0])         # S.1111.111
    assert oracle.e4m3_decode([0x38])[0] == 1.0            # exponent 7 = bias
    assert oracle.e4m3_decode([0x01])[0] == 2.0 ** -9      # smallest subnormal
    assert oracle.e4m3_decode([0x08])[0] == 2.0 ** -6      # smallest normal
    assert oracle.e4m3_decode([0x80])[0] == 0.0 and np.signbit(oracle.e4m3_decode([0x80])[0])
    enc = oracle.e4m3_encode
    assert enc([1.0])[0] == 0x38 and enc([-1.0])[0] == 0xB8
    assert enc([448.0])[0] == 0x7E
    # ties to even: 2^-10 is halfway between 0 and 2^-9; 3*2^-10 between codes 1 and 2
    assert enc([2.0 ** -10])[0] == 0x00
    assert enc([3 * 2.0 ** -10])[0] == 0x02
    # 1 + 1/16 is halfway between 1 (0x38, even) and 1.125 (0x39)
    assert enc([1.0625])[0] == 0x38
    assert enc([1.1875])[0] == 0x3A  # halfway 1.125 / 1.25 -> even 0x3A
    # saturation instead of NaN beyond 448
    for v in (449.0, 464.0, 465.0, 1000.0, 1e30, float("inf")):
        assert enc([v])[0] == 0x7E and enc([-v])[0] == 0xFE
    assert (enc([float("nan")])[0] & 0x7F) == 0x7F


def _all_finite_values():
    return oracle.e4m3_decode(np.arange(0x7F))


def test_encode_matches_torch_in_range():
    vals = _all_finite_values()
    mids = (vals[1:] + vals[:-1]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([vals, -vals, mids, -mids,
                        np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        rng.uniform(-448, 448, 2000), rng.normal(0, 1, 2000)]).astype(np.float32)
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = oracle.e4m3_decode(codes)
    back = oracle.e4m3_encode(vals.astype(np.float32))
    # +0 and -0 keep their sign bit
    assert np.array_equal(back, codes.astype(np.uint8))


def test_quantisation_error_bound():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 3, (64, 4, 32)).astype(np.float32)
    scale = np.array([0.01, 0.1, 1.0, 7.0], dtype=np.float32)
    deq = oracle.dequantize(oracle.quantize(x, scale), scale)
    y = x / scale.reshape(-1, 1)
    # half an ulp: 2^-4 relative for normal values, 2^-10 absolute below 2^-6
    bound = np.maximum(np.abs(np.clip(y, -448, 448)) * 2.0 ** -4, 2.0 ** -10) * scale.reshape(-1, 1)
    sat = np.abs(y) > 448
    err = np.abs(deq - x)
    assert (err[~sat] <= bound[~sat] + 1e-12).all()
    # saturated entries come back as +-448 * scale
    assert np.allclose(np.abs(deq[sat]), (448.0 * scale.reshape(-1, 1) * np.ones_like(y))[sat])


def test_quantised_append_through_the_page_table():
    rng = np.random.default_rng(2)
    B, Nnew, Hkv, d, P = 2, 3, 2, 8, 6
    table = np.array([[4, 1, -1], [0, 5, 2]])
    cache_lens = np.array([15, 30])
    pool = rng.integers(0, 256, (P, 16, Hkv, d)).astype(np.uint8)
    new = rng.normal(0, 2, (B, Nnew, Hkv, d)).astype(np.float32)
    scale = np.array([0.5, 0.02], dtype=np.float32)
    out = oracle.kv_append_ref(pool, oracle.quantize(new, scale), table, cache_lens)
    for b in range(B):
        for r in range(Nnew):
            t = cache_lens[b] + r
            blk, slot = table[b][t // 16], t % 16
            for h in range(Hkv):
                for j in range(d):
                    want = oracle.e4m3_encode([np.float32(new[b, r, h, j]) / scale[h]])[0]
                    assert out[blk, slot, h, j] == want
    # nothing else changed
    touched = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(B):
        for r in range(Nnew):
            t = cache_lens[b] + r
            touched[table[b][t // 16], t % 16] = True
    assert np.array_equal(out[~touched], pool[~touched])
