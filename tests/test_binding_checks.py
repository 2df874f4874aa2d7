"""The Python binding rejects mis-shaped or mis-typed tensors before any call
into the library (CPU only: every call here fails a host-side check first).

Caller-supplied outputs (out, lse, dq, dk, dv) are written by the kernels with
the layout the shapes imply, and a contiguous cache's max_seq_len is its row
stride, so a mismatch would write or read past the tensors on the device:
each must raise ValueError or TypeError here, and a correctly shaped CPU call
must get as far as the device check.
"""

import os

import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta

pytestmark = pytest.mark.skipif(not os.path.exists(eta.LIB_PATH),
                                reason="libattn.so not built (run __graft_entry__.build())")

bf = torch.bfloat16
f32 = torch.float32
i32 = torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def _raises(fn, exc, match):
    with pytest.raises(exc, match=match):
        fn()


def test_well_formed_calls_reach_the_device_check():
    q, k = z(1, 4, 8, 64), z(1, 2, 8, 64)
    _raises(lambda: eta.attn_prefill(q, k, k, out=z(1, 4, 8, 64), lse=z(1, 4, 8, dtype=f32)),
            ValueError, "GPU device")
    qd, cache = z(2, 1, 4, 64), z(2, 32, 2, 64)
    _raises(lambda: eta.attn_decode_paged(qd, cache, cache, torch.ones(2, dtype=i32),
                                          max_seq_len=32), ValueError, "GPU device")


PREFILL_BAD = [
    ("out shape", dict(out=z(1, 4, 9, 64)), ValueError, "out must have shape"),
    ("out dtype", dict(out=z(1, 4, 8, 64, dtype=f32)), TypeError, "out must be"),
    ("lse shape", dict(lse=z(1, 4, 9, dtype=f32)), ValueError, "lse must have shape"),
    ("lse dtype", dict(lse=z(1, 4, 8)), TypeError, "lse must be"),
]


@pytest.mark.parametrize("what,kw,exc,match", PREFILL_BAD, ids=[c[0] for c in PREFILL_BAD])
def test_prefill_outputs_checked(what, kw, exc, match):
    q, k = z(1, 4, 8, 64), z(1, 2, 8, 64)
    _raises(lambda: eta.attn_prefill(q, k, k, **kw), exc, match)


def test_prefill_inputs_checked():
    _raises(lambda: eta.attn_prefill(z(4, 8, 64), z(1, 2, 8, 64), z(1, 2, 8, 64)), ValueError,
            "dimensions")
    _raises(lambda: eta.attn_prefill(z(1, 4, 8, 64), z(1, 2, 8, 32), z(1, 2, 8, 32)), ValueError,
            "matching q")
    _raises(lambda: eta.attn_prefill(z(1, 4, 8, 64), z(1, 2, 8, 64, dtype=f32),
                                     z(1, 2, 8, 64, dtype=f32)), TypeError, "one dtype")


BWD_BAD = [
    ("dq shape", dict(dq=z(1, 4, 8, 32)), ValueError, "dq must have shape"),
    ("dq dtype", dict(dq=z(1, 4, 8, 64, dtype=f32)), TypeError, "dq must be"),
    ("dk shape", dict(dk=z(1, 2, 7, 64)), ValueError, "dk must have shape"),
    ("dv dtype", dict(dv=z(1, 2, 8, 64, dtype=f32)), TypeError, "dv must be"),
]


@pytest.mark.parametrize("what,kw,exc,match", BWD_BAD, ids=[c[0] for c in BWD_BAD])
def test_backward_outputs_checked(what, kw, exc, match):
    q, k = z(1, 4, 8, 64), z(1, 2, 8, 64)
    lse = z(1, 4, 8, dtype=f32)
    _raises(lambda: eta.attn_prefill_backward(q, k, k, q, lse, q, **kw), exc, match)


def _decode_args(paged, dtype=bf):
    B, Nq, Hq, Hkv, d = 2, 1, 4, 2, 64
    q = z(B, Nq, Hq, d)
    if paged:
        cache = z(6, 16, Hkv, d, dtype=dtype)
        table = torch.zeros((B, 3), dtype=i32)
    else:
        cache = z(B, 48, Hkv, d, dtype=dtype)
        table = None
    return q, cache, table, torch.ones(B, dtype=i32)


DECODE_BAD = [
    ("out shape", True, dict(out=z(2, 1, 4, 32)), ValueError, "out must have shape"),
    ("out dtype", True, dict(out=z(2, 1, 4, 64, dtype=f32)), TypeError, "out must be"),
    ("lse shape", True, dict(lse=z(2, 4, 2, dtype=f32)), ValueError, "lse must have shape"),
    ("lse dtype", False, dict(lse=z(2, 4, 1)), TypeError, "lse must be"),
    ("contiguous max_seq_len past the cache", False, dict(max_seq_len=64), ValueError,
     "second dimension"),
    ("contiguous max_seq_len below the stride", False, dict(max_seq_len=32), ValueError,
     "second dimension"),
    ("paged max_seq_len past the table", True, dict(max_seq_len=49), ValueError, "max_seq_len"),
]


@pytest.mark.parametrize("what,paged,kw,exc,match", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_checked(what, paged, kw, exc, match):
    q, cache, table, lens = _decode_args(paged)
    _raises(lambda: eta.attn_decode_paged(q, cache, cache, lens, block_table=table, **kw), exc,
            match)
    if "max_seq_len" in kw or "out" in kw or "lse" in kw:
        _raises(lambda: eta.attn_prefill_paged(q, cache, cache, lens, block_table=table, **kw),
                exc, match)


def test_decode_cache_dtype_checked():
    q, cache, table, lens = _decode_args(True, dtype=f32)
    _raises(lambda: eta.attn_decode_paged(q, cache, cache, lens, block_table=table), TypeError,
            "one dtype")
    q, cache, table, lens = _decode_args(True, dtype=torch.uint8)
    _raises(lambda: eta.attn_decode_paged(q, cache, cache, lens, block_table=table), TypeError,
            "one dtype")


def test_fp8_decode_checked():
    q, cache, table, lens = _decode_args(True, dtype=torch.uint8)
    s = torch.ones(2, dtype=f32)
    _raises(lambda: eta.attn_decode_paged_fp8(q, cache, cache, s, s, lens, block_table=table,
                                              out=z(2, 1, 4, 32)), ValueError, "out must have")
    _raises(lambda: eta.attn_decode_paged_fp8(q, z(6, 16, 2, 64), z(6, 16, 2, 64), s, s, lens,
                                              block_table=table), TypeError, "fp8 cache")
    _raises(lambda: eta.attn_decode_paged_fp8(q, cache, cache, torch.ones(3, dtype=f32), s, lens,
                                              block_table=table), ValueError, "scales")


def test_append_checked():
    kn = z(2, 3, 2, 64)
    cache = z(2, 48, 2, 64)
    lens = torch.zeros(2, dtype=i32)
    _raises(lambda: eta.kv_append(kn, kn, cache, cache, lens, max_seq_len=96), ValueError,
            "second dimension")
    _raises(lambda: eta.kv_append(kn, kn, z(3, 48, 2, 64), z(3, 48, 2, 64), lens), ValueError,
            "contiguous cache")
    _raises(lambda: eta.kv_append(kn, kn, cache, cache, lens,
                                  block_table=torch.zeros((2, 3), dtype=i32)), ValueError,
            "paged cache")
    c8 = torch.zeros((2, 48, 2, 64), dtype=torch.uint8)
    s = torch.ones(2, dtype=f32)
    _raises(lambda: eta.kv_append_fp8(kn, kn, c8, c8, s, s, lens, max_seq_len=47), ValueError,
            "second dimension")


def test_gather_checked():
    cache = z(6, 16, 2, 64)
    lens = torch.ones(2, dtype=i32)
    table = torch.zeros((2, 3), dtype=i32)
    _raises(lambda: eta.attn_gather_paged(cache, lens, table, out=z(2, 40, 2, 64)), ValueError,
            "out must have shape")
    _raises(lambda: eta.attn_gather_paged(cache, lens, table, out=z(2, 48, 2, 64, dtype=f32)),
            TypeError, "out must be")
