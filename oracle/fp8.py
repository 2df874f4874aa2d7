"""E4M3 8-bit floating point and the quantised K/V cache — TEST INFRASTRUCTURE.

Source: "Phase 07 · 12: KV cache, Flash Attention and inference
optimisation", section "Paged attention", names an fp8 K/V cache
(`--kv-cache-dtype fp8`) as the serving option that halves cache memory; the
page gives no encoding. Reading taken (and stated where the method is
documented): the OCP 8-bit format E4M3 in its "fn" variant — 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, no
infinities, the bit pattern S.1111.111 is NaN, the largest finite value is
448 — with one fp32 scale per K/V head:

    code   = E4M3 nearest-even( clamp(x / scale, -448, 448) )
    value  = decode(code) * scale

where x / scale is one IEEE fp32 division of the fp32 value of the stored
input (bf16 inputs are exact in fp32). Values beyond the largest finite
magnitude saturate to ±448 instead of becoming NaN.

Everything here is written from that definition with plain loops and
lookups: decoding reads the three fields of the byte; encoding takes the
nearest entry of the table of all finite values (ties to the even code).
The attention over a quantised cache is the plain definition
(``decode_attention``) over the dequantised fp64 cache.
"""

import numpy as np

E4M3_MAX = 448.0


def _decode_byte(code):
    """fp64 value of one E4M3 byte, from its three fields."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the value of every byte, once
_TABLE = np.array([_decode_byte(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """fp64 values of E4M3 bytes (any integer array shape)."""
    return _TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


# codes 0x00..0x7E (all non-negative finite values), ascending
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]


def _encode_magnitudes(a):
    """Nearest non-negative E4M3 codes of non-negative finite values <= 448:
    the entry of the value table at the smallest distance; when the next
    entry is exactly as close, the even code of the two."""
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    out = np.empty(a.shape, dtype=np.int64)
    for s0 in range(0, a.size, 1 << 16):  # bounded memory for the distance matrix
        chunk = a[s0:s0 + (1 << 16)]
        dist = np.abs(_POS_VALUES[None, :] - chunk[:, None])
        best = np.argmin(dist, axis=1)  # the lower index on a tie
        nxt = np.minimum(best + 1, len(_POS_VALUES) - 1)
        tie = (nxt != best) & (dist[np.arange(len(chunk)), nxt] == dist[np.arange(len(chunk)), best])
        pick = np.where(tie & (_POS_CODES[best] % 2 == 1), nxt, best)
        out[s0:s0 + len(chunk)] = _POS_CODES[pick]
    return out


def e4m3_encode(values):
    """E4M3 bytes (uint8) of fp32 values: saturate to ±448, then round to the
    nearest representable value, ties to even. NaN encodes as 0x7F (with its
    sign bit)."""
    x = np.asarray(values, dtype=np.float32)
    v = x.astype(np.float64).reshape(-1)
    neg = np.signbit(v)
    nan = np.isnan(v)
    mag = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    code = _encode_magnitudes(mag)
    code = np.where(nan, 0x7F, code) | np.where(neg, 0x80, 0)
    return code.astype(np.uint8).reshape(x.shape)


def quantize(x, scale):
    """Codes of x (any float array, last axes [..., Hkv, d]) with one scale per
    K/V head: one fp32 division per element, then E4M3 encoding."""
    xf = np.asarray(x, dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32).reshape(-1, 1)  # [Hkv, 1]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xf / s).astype(np.float32)
    return e4m3_encode(y)


def dequantize(codes, scale):
    """fp64 values of a quantised cache (last axes [..., Hkv, d])."""
    s = np.asarray(scale, dtype=np.float64).reshape(-1, 1)
    return e4m3_decode(codes) * s
