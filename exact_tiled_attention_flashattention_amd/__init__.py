"""MI355X-native exact tiled attention: Python binding of libattn.so.

Thin ctypes marshalling over the C ABI in ``include/attn.h``: shape, dtype
and device checks, output allocation through torch, and the call. Every step
of the computation runs in the library's HIP kernels; there is no fallback.
If ``libattn.so`` has not been built (``__graft_entry__.build()`` or
``python -m exact_tiled_attention_flashattention_amd.build``), every call
raises.

Entry points (same names as the C ABI):
    attn_prefill(q, k, v, scale=None, causal=False, q_offset=0)      -> (o, lse)
    attn_prefill_backward(q, k, v, o, lse, dout, ...)                -> (dq, dk, dv)
    attn_decode_paged(q, k_cache, v_cache, seq_lens, block_table=None, ...) -> (o, lse)
    kv_append(k_new, v_new, k_cache, v_cache, cache_lens, block_table=None, ...)
    attn_gather_paged(cache, seq_lens, block_table, max_seq_len)     -> out
    BlockPool(num_blocks).grow(table_row, cur_len, new_len) / .release(table_row, len)
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EWORKSPACE = -3
ATTN_EHIP = -4
ATTN_ENOSPACE = -5
ATTN_F32 = 0
ATTN_BF16 = 1
BLOCK_TOKENS = 16
NOALLOC_SCRATCH_BYTES = 32 << 20  # ATTN_DECODE_NOALLOC_SCRATCH_BYTES

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _load().attn_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P]
    lib.attn_prefill.restype = I
    lib.attn_prefill_paged.argtypes = [P, P, P, P, I, I, P, P, P, I, I, I, I, I, I, F, I, I, P]
    lib.attn_prefill_paged.restype = I
    lib.attn_prefill_waves.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, I, P]
    lib.attn_prefill_waves.restype = I
    lib.attn_prefill_paged_waves.argtypes = [P, P, P, P, I, I, P, P, P, I, I, I, I, I, I, F, I,
                                             I, I, P]
    lib.attn_prefill_paged_waves.restype = I
    lib.attn_prefill_workgroup_waves.argtypes = [I, I, I, I, I, I]
    lib.attn_prefill_workgroup_waves.restype = I
    lib.attn_decode_paged_fp8.argtypes = [P, P, P, P, P, P, I, I, P, P, P, I, I, I, I, I, F, I, I,
                                          I, P, SZ, P]
    lib.attn_decode_paged_fp8.restype = I
    lib.kv_append_fp8.argtypes = [P, P, P, P, P, P, P, I, I, P, I, I, I, I, I, P]
    lib.kv_append_fp8.restype = I
    lib.attn_decode_paged.argtypes = [P, P, P, P, I, I, P, P, P, I, I, I, I, I, I, F, I, I, I,
                                      P, SZ, P]
    lib.attn_decode_paged.restype = I
    lib.attn_decode_paged_noalloc.argtypes = [P, P, P, P, I, I, P, P, P, I, I, I, I, I, I, F, I,
                                              I, I, P]
    lib.attn_decode_paged_noalloc.restype = I
    lib.attn_decode_num_splits.argtypes = [I, I, I, I, I, I, I]
    lib.attn_decode_num_splits.restype = I
    lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    lib.attn_decode_workspace_bytes.restype = SZ
    lib.kv_append.argtypes = [P, P, P, P, P, I, I, P, I, I, I, I, I, I, P]
    lib.kv_append.restype = I
    lib.attn_gather_paged.argtypes = [P, P, I, I, P, P, I, I, I, I, I, P]
    lib.attn_gather_paged.restype = I
    lib.attn_prefill_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I,
                                          I, P, SZ, P]
    lib.attn_prefill_backward.restype = I
    lib.attn_prefill_backward_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.attn_prefill_backward_workspace_bytes.restype = SZ
    lib.attn_block_pool_bytes.argtypes = [I]
    lib.attn_block_pool_bytes.restype = SZ
    lib.attn_block_pool_init.argtypes = [P, SZ, I]
    lib.attn_block_pool_init.restype = I
    lib.attn_block_pool_free_count.argtypes = [P]
    lib.attn_block_pool_free_count.restype = I
    lib.attn_block_pool_grow.argtypes = [P, P, I, I, I]
    lib.attn_block_pool_grow.restype = I
    lib.attn_block_pool_release.argtypes = [P, P, I, I]
    lib.attn_block_pool_release.restype = I
    lib.attn_strerror.argtypes = [I]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes handle (raises if libattn.so is missing)."""
    return _load()


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(status, where):
    if status != ATTN_OK:
        raise AttnError(status, where)


def _need_gpu(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors must share one device ({dev} and {t.device})")


def _dims(t, n, name):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {list(t.shape)}")
    return tuple(t.shape)


def _expect(t, shape, dtype, name):
    """A caller-supplied output (or input) must have exactly this shape and dtype:
    the kernels write and read it with that layout and nothing else bounds them."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def attn_prefill(q, k, v, scale=None, causal=False, q_offset=0, out=None, lse=None,
                 want_lse=True, waves=0):
    """Prefill. q [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d] -> o [B,Hq,Nq,d], lse [B,Hq,Nq] f32.
    ``waves`` (tests): force the bf16 kernel's workgroup width, 4 or 8 (0 = the
    library's choice, attn_prefill_workgroup_waves)."""
    lib = _load()
    B, Hq, Nq, d = _dims(q, 4, "q")
    _dims(k, 4, "k")
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _need_gpu(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _dtype_code(q), B, Hq, Hkv, Nq, Nk,
            d, float(scale), int(bool(causal)), int(q_offset))
    if waves:
        st = lib.attn_prefill_waves(*args, int(waves), _stream(q.device))
    else:
        st = lib.attn_prefill(*args, _stream(q.device))
    _check(st, "attn_prefill")
    return out, lse


def attn_prefill_backward(q, k, v, o, lse, dout, scale=None, causal=False, q_offset=0, dq=None,
                          dk=None, dv=None, workspace=None):
    """Backward of attn_prefill (bf16). q, o, dout [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d];
    lse [B,Hq,Nq] f32 from the forward -> dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d]."""
    lib = _load()
    B, Hq, Nq, d = _dims(q, 4, "q")
    _dims(k, 4, "k")
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, Nk, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    for t in (k, v, o, dout):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, o, dout must share one dtype")
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, Nq):
        raise ValueError("lse must be float32 [B, Hq, Nq]")
    _expect(dq, q.shape, q.dtype, "dq")
    _expect(dk, k.shape, q.dtype, "dk")
    _expect(dv, v.shape, q.dtype, "dv")
    _need_gpu(q, k, v, o, lse, dout, dq, dk, dv, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    need = int(lib.attn_prefill_backward_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                                                         int(q_offset)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib.attn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(q), B, Hq, Hkv, Nq,
                                   Nk, d, float(scale), int(bool(causal)), int(q_offset),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(q.device))
    _check(st, "attn_prefill_backward")
    return dq, dk, dv


def attn_prefill_backward_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal=False, q_offset=0):
    return int(_load().attn_prefill_backward_workspace_bytes(B, Hq, Hkv, Nq, Nk, d,
                                                             int(bool(causal)), int(q_offset)))


def _check_cache_args(q, k_cache, v_cache, seq_lens, block_table, fp8=False):
    B, Nq, Hq, d = _dims(q, 4, "q")
    _dims(k_cache, 4, "k_cache")
    if k_cache.shape[3] != d or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache/v_cache must share a shape with head dim d")
    if fp8:
        if q.dtype != torch.bfloat16:
            raise TypeError("q is bf16")
        _fp8_cache(k_cache)
        _fp8_cache(v_cache)
    elif k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B, max_blocks]")
        if k_cache.shape[1] != BLOCK_TOKENS:
            raise ValueError("a paged cache is [num_blocks, 16, Hkv, d]")
    elif k_cache.shape[0] != B:
        raise ValueError("a contiguous cache is [B, max_len, Hkv, d]")


def attn_prefill_paged(q, k_cache, v_cache, seq_lens, block_table=None, scale=None, causal=True,
                       max_seq_len=None, out=None, lse=None, want_lse=True, waves=0):
    """Chunked prefill against a cache. q [B,Nq,Hq,d]; caches [P,16,Hkv,d] (paged) or
    [B,L,Hkv,d] (contiguous); seq_lens [B] int32 (keys incl. the Nq new ones)
    -> o [B,Nq,Hq,d], lse [B,Hq,Nq]."""
    lib = _load()
    _check_cache_args(q, k_cache, v_cache, seq_lens, block_table)
    B, Nq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _need_gpu(q, k_cache, v_cache, seq_lens, block_table, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), mb, nblocks,
            _ptr(seq_lens), _ptr(out), _ptr(lse), _dtype_code(q), B, Hq, Hkv, Nq, d, float(scale),
            int(bool(causal)), L)
    if waves:
        st = lib.attn_prefill_paged_waves(*args, int(waves), _stream(q.device))
    else:
        st = lib.attn_prefill_paged(*args, _stream(q.device))
    _check(st, "attn_prefill_paged")
    return out, lse


def attn_prefill_workgroup_waves(B, Hq, Hkv, Nq, causal, dtype=ATTN_BF16):
    """Waves per workgroup (4 or 8) the bf16 prefill kernel picks for this shape."""
    st = _load().attn_prefill_workgroup_waves(dtype, B, Hq, Hkv, Nq, int(bool(causal)))
    _check(min(st, 0), "attn_prefill_workgroup_waves")
    return st


def attn_decode_num_splits(B, Hq, Hkv, Nq, d, max_seq_len, num_splits=0):
    st = _load().attn_decode_num_splits(B, Hq, Hkv, Nq, d, max_seq_len, num_splits)
    _check(min(st, 0), "attn_decode_num_splits")
    return st


def attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, max_seq_len, num_splits=0):
    return int(_load().attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, max_seq_len, num_splits))


def _check_table(block_table, cache, B):
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B, max_blocks]")
        if cache.shape[1] != BLOCK_TOKENS:
            raise ValueError("a paged cache is [num_blocks, 16, Hkv, d]")
    elif cache.shape[0] != B:
        raise ValueError("a contiguous cache is [B, max_len, Hkv, d]")


def _cache_geometry(k_cache, block_table, max_seq_len):
    """(max_len, max_blocks_per_seq, num_blocks) of a cache. A contiguous cache's
    max_len is its row stride ([B, max_len, Hkv, d]), so it must be the tensor's
    own second dimension; a paged cache's max_len only caps the positions."""
    if block_table is None:
        cap = k_cache.shape[1]
        if max_seq_len is not None and int(max_seq_len) != cap:
            raise ValueError(f"a contiguous cache's max_seq_len is its second dimension ({cap}), "
                             f"got {max_seq_len}")
        return cap, 0, 0
    mb = block_table.shape[1]
    cap = mb * BLOCK_TOKENS
    if max_seq_len is not None and not 0 <= int(max_seq_len) <= cap:
        raise ValueError(f"max_seq_len must be in [0, {cap}] (16 x the table's columns), "
                         f"got {max_seq_len}")
    return (cap if max_seq_len is None else int(max_seq_len)), mb, k_cache.shape[0]


def attn_decode_paged(q, k_cache, v_cache, seq_lens, block_table=None, scale=None, causal=True,
                      max_seq_len=None, num_splits=0, workspace=None, out=None, lse=None,
                      want_lse=True):
    """Decode. q [B,Nq,Hq,d]; caches [P,16,Hkv,d] (paged) or [B,L,Hkv,d] (contiguous);
    seq_lens [B] int32 (keys incl. the Nq new ones) -> o [B,Nq,Hq,d], lse [B,Hq,Nq]."""
    lib = _load()
    _check_cache_args(q, k_cache, v_cache, seq_lens, block_table)
    B, Nq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _need_gpu(q, k_cache, v_cache, seq_lens, block_table, workspace, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, L, num_splits)
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), mb,
                               nblocks, _ptr(seq_lens), _ptr(out), _ptr(lse), _dtype_code(q), B, Hq,
                               Hkv, Nq, d, float(scale), int(bool(causal)), L, int(num_splits),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(q.device))
    _check(st, "attn_decode_paged")
    return out, lse


def attn_decode_paged_noalloc(q, k_cache, v_cache, seq_lens, block_table=None, scale=None,
                              causal=True, max_seq_len=None, num_splits=0, out=None, lse=None,
                              want_lse=True):
    """attn_decode_paged whose partial results live in the library's own device
    array (the C call allocates nothing; pass out/lse to allocate nothing here
    either). Same arguments and results, no workspace; raises AttnError
    (ATTN_EWORKSPACE) when the call needs more than NOALLOC_SCRATCH_BYTES."""
    lib = _load()
    _check_cache_args(q, k_cache, v_cache, seq_lens, block_table)
    B, Nq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _need_gpu(q, k_cache, v_cache, seq_lens, block_table, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       mb, nblocks, _ptr(seq_lens), _ptr(out), _ptr(lse),
                                       _dtype_code(q), B, Hq, Hkv, Nq, d, float(scale),
                                       int(bool(causal)), L, int(num_splits), _stream(q.device))
    _check(st, "attn_decode_paged_noalloc")
    return out, lse


def kv_append(k_new, v_new, k_cache, v_cache, cache_lens, block_table=None, max_seq_len=None):
    """Write k_new/v_new [B,Nnew,Hkv,d] at positions cache_lens[b] + r (in place)."""
    lib = _load()
    B, Nnew, Hkv, d = _dims(k_new, 4, "k_new")
    _dims(k_cache, 4, "k_cache")
    if v_new.shape != k_new.shape or k_cache.shape[2:] != (Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between new rows and cache")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("new rows and cache must share one dtype")
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    _check_table(block_table, k_cache, B)
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _need_gpu(k_new, v_new, k_cache, v_cache, cache_lens, block_table)
    st = lib.kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                       mb, nblocks, _ptr(cache_lens), _dtype_code(k_new), B, Hkv, Nnew, d, L,
                       _stream(k_new.device))
    _check(st, "kv_append")


def _fp8_cache(t):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("an fp8 cache is uint8 (E4M3 codes) or float8_e4m3fn")


def _scales(s, Hkv, device):
    if s.dtype != torch.float32 or s.shape != (Hkv,) or s.device != device:
        raise ValueError("scales must be float32 [Hkv] on the cache's device")


def kv_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, cache_lens, block_table=None,
                  max_seq_len=None):
    """Quantise k_new/v_new [B,Nnew,Hkv,d] (bf16) into an E4M3 cache at positions
    cache_lens[b] + r (in place); code = nearest(x / scale[h]), saturating at 448."""
    lib = _load()
    B, Nnew, Hkv, d = _dims(k_new, 4, "k_new")
    _dims(k_cache, 4, "k_cache")
    if v_new.shape != k_new.shape or k_cache.shape[2:] != (Hkv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between new rows and cache")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise TypeError("new rows are bf16")
    _fp8_cache(k_cache)
    _fp8_cache(v_cache)
    _scales(k_scale, Hkv, k_cache.device)
    _scales(v_scale, Hkv, k_cache.device)
    if cache_lens.dtype != torch.int32 or cache_lens.shape != (B,):
        raise ValueError("cache_lens must be int32 [B]")
    _check_table(block_table, k_cache, B)
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _need_gpu(k_new, v_new, k_cache, v_cache, k_scale, v_scale, cache_lens, block_table)
    st = lib.kv_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                           _ptr(v_scale), _ptr(block_table), mb, nblocks, _ptr(cache_lens), B, Hkv,
                           Nnew, d, L, _stream(k_new.device))
    _check(st, "kv_append_fp8")


def attn_decode_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table=None,
                          scale=None, causal=True, max_seq_len=None, num_splits=0, workspace=None,
                          out=None, lse=None, want_lse=True):
    """Decode against an E4M3 cache with per-head scales. q [B,Nq,Hq,d] bf16; caches
    uint8 [P,16,Hkv,d] (paged) or [B,L,Hkv,d]; -> o [B,Nq,Hq,d], lse [B,Hq,Nq]."""
    lib = _load()
    _check_cache_args(q, k_cache, v_cache, seq_lens, block_table, fp8=True)
    B, Nq, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    _scales(k_scale, Hkv, k_cache.device)
    _scales(v_scale, Hkv, k_cache.device)
    L, mb, nblocks = _cache_geometry(k_cache, block_table, max_seq_len)
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _need_gpu(q, k_cache, v_cache, k_scale, v_scale, seq_lens, block_table, workspace, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, Nq, d, L, num_splits)
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(block_table), mb, nblocks, _ptr(seq_lens),
                                   _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, d, float(scale),
                                   int(bool(causal)), L, int(num_splits), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(q.device))
    _check(st, "attn_decode_paged_fp8")
    return out, lse


def attn_gather_paged(cache, seq_lens, block_table=None, max_seq_len=None, out=None):
    """Gather each sequence's first seq_lens[b] rows into out [B, max_seq_len, Hkv, d]."""
    lib = _load()
    _dims(cache, 4, "cache")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be int32 [B]")
    B = seq_lens.shape[0]
    Hkv, d = cache.shape[2], cache.shape[3]
    _check_table(block_table, cache, B)
    L, mb, nblocks = _cache_geometry(cache, block_table, max_seq_len)
    _expect(out, (B, L, Hkv, d), cache.dtype, "out")
    _need_gpu(cache, seq_lens, block_table, out)
    if out is None:
        out = torch.zeros((B, L, Hkv, d), dtype=cache.dtype, device=cache.device)
    st = lib.attn_gather_paged(_ptr(cache), _ptr(block_table), mb, nblocks, _ptr(seq_lens),
                               _ptr(out), _dtype_code(cache), B, Hkv, d, L, _stream(cache.device))
    _check(st, "attn_gather_paged")
    return out


class BlockPool:
    """Host-side pool of a paged cache's physical 16-token blocks (the C ABI's
    attn_block_pool_*; the state sits in a buffer this object owns). Table rows
    are host int32 numpy arrays (-1 = no block); copy the table to the device
    before a kernel reads it."""

    def __init__(self, num_blocks):
        lib = _load()
        n = int(lib.attn_block_pool_bytes(int(num_blocks)))
        if n == 0:
            raise ValueError("num_blocks must be >= 0")
        self._buf = (ctypes.c_int32 * ((n + 3) // 4))()
        self.num_blocks = int(num_blocks)
        _check(lib.attn_block_pool_init(ctypes.addressof(self._buf), n, self.num_blocks),
               "attn_block_pool_init")

    def _addr(self):
        return ctypes.addressof(self._buf)

    @staticmethod
    def _row(table_row):
        import numpy as np

        if not isinstance(table_row, np.ndarray) or table_row.dtype != np.int32 or \
                table_row.ndim != 1 or not table_row.flags["C_CONTIGUOUS"] or \
                not table_row.flags["WRITEABLE"]:
            raise TypeError("a table row is a writeable contiguous 1-D int32 numpy array")
        return table_row.ctypes.data, table_row.shape[0]

    def free_count(self):
        st = _load().attn_block_pool_free_count(self._addr())
        _check(min(st, 0), "attn_block_pool_free_count")
        return st

    def grow(self, table_row, cur_len, new_len):
        """Blocks for positions [cur_len, new_len); False (nothing changed) when the
        pool has too few free blocks."""
        ptr, mb = self._row(table_row)
        st = _load().attn_block_pool_grow(self._addr(), ptr, mb, int(cur_len), int(new_len))
        if st == ATTN_ENOSPACE:
            return False
        _check(st, "attn_block_pool_grow")
        return True

    def release(self, table_row, length):
        """Free-on-finish: the sequence's ceil(length/16) blocks go back to the pool."""
        ptr, mb = self._row(table_row)
        _check(_load().attn_block_pool_release(self._addr(), ptr, mb, int(length)),
               "attn_block_pool_release")


__all__ = [
    "BlockPool",
    "attn_prefill_backward",
    "attn_prefill_backward_workspace_bytes",
    "attn_prefill",
    "attn_prefill_paged",
    "attn_prefill_workgroup_waves",
    "attn_decode_paged_fp8",
    "kv_append_fp8",
    "attn_decode_paged",
    "attn_decode_paged_noalloc",
    "attn_decode_num_splits",
    "attn_decode_workspace_bytes",
    "kv_append",
    "attn_gather_paged",
    "library",
    "AttnError",
    "LIB_PATH",
]
