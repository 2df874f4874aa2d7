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


def e4m3_decode(codes):
    """fp64 values of E4M3 bytes (any integer array shape)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    out = np.empty(c.shape, dtype=np.float64)
    flat_c = c.reshape(-1)
    flat_o = out.reshape(-1)
    for i, code in enumerate(flat_c):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            flat_o[i] = np.nan
        elif e == 0:
            flat_o[i] = sign * (m / 8.0) * 2.0 ** -6
        else:
            flat_o[i] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


# codes 0x00..0x7E (all non-negative finite values), ascending
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES)


def _encode_one(v):
    """Nearest non-negative E4M3 code of a non-negative finite v <= 448."""
    # distance to every finite value; the nearest wins, ties go to the even code
    dist = np.abs(_POS_VALUES - v)
    best = int(np.argmin(dist))
    ties = np.nonzero(dist == dist[best])[0]
    if len(ties) > 1:
        even = [int(t) for t in ties if int(_POS_CODES[t]) % 2 == 0]
        best = even[0]
    return int(_POS_CODES[best])


def e4m3_encode(values):
    """E4M3 bytes (uint8) of fp32 values: saturate to ±448, then round to the
    nearest representable value, ties to even. NaN encodes as 0x7F (with its
    sign bit)."""
    x = np.asarray(values, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    for i, v in enumerate(flat_x):
        v = float(v)
        neg = np.signbit(v)
        if np.isnan(v):
            flat_o[i] = 0x7F | (0x80 if neg else 0)
            continue
        a = min(abs(v), E4M3_MAX)
        flat_o[i] = _encode_one(a) | (0x80 if neg else 0)
    return out


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
