"""The oracle's own page-table gather and cache append (test infrastructure).

Layout ("Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
section "Paged attention: the KV cache as virtual memory"): the cache is cut
into 16-token blocks and a page table maps a logical token position to a
physical block. Read plainly, logical token t of sequence b lives in physical
block ``table[b][t // 16]`` at slot ``t % 16``; a pool is
[num_blocks, 16, Hkv, d] (the per-token (Hkv, d) rows of the cache layout that
"[BEE-30062]", section "為長上下文推論啟用 FlashDecoding", gives, cut into
blocks).

These helpers move stored values only (no arithmetic), so they work on numpy
arrays and on torch tensors alike and keep bf16 bit patterns intact.
"""

import numpy as np


def _rows(x):
    return int(x.shape[0])


def _table_entry(table_row, i):
    return int(table_row[i])


def gather_paged(pool, table_row, n, block_size=16):
    """Logical rows 0..n-1 of one sequence, gathered through its table row.

    Returns an array of shape [n, *pool.shape[2:]] of the pool's own type.
    """
    nblk = -(-n // block_size)
    parts = []
    for i in range(nblk):
        blk = _table_entry(table_row, i)
        if blk < 0 or blk >= _rows(pool):
            raise IndexError(f"table entry {i} = {blk} outside the pool")
        take = min(block_size, n - i * block_size)
        parts.append(pool[blk, :take])
    if hasattr(pool, "detach"):
        import torch

        if not parts:
            return pool.new_empty((0,) + tuple(pool.shape[2:]))
        return torch.cat(parts, dim=0)
    if not parts:
        return np.empty((0,) + tuple(pool.shape[2:]), dtype=pool.dtype)
    return np.concatenate(parts, axis=0)


def gather_contiguous(cache, b, n):
    """Rows 0..n-1 of sequence b of a contiguous cache [B, max_len, Hkv, d]."""
    if n > cache.shape[1]:
        raise IndexError("sequence longer than the contiguous cache")
    return cache[b, :n]


def kv_append_ref(pool, new_rows, table, cache_lens, block_size=16):
    """Return a copy of ``pool`` with ``new_rows`` written after each sequence.

    The decode step grows the cache by concatenating the new token's K (and V)
    ("大模型面试笔记——Attention篇" §4; "Phase 07 · 12", "Build it, step 1":
    append per layer and head). With the paged layout, row r of sequence b
    lands at logical position t = cache_lens[b] + r, i.e. in block
    table[b][t // 16], slot t % 16. ``new_rows`` is [B, Nnew, Hkv, d].
    Nothing else in the pool changes.
    """
    out = pool.clone() if hasattr(pool, "detach") else np.array(pool, copy=True)
    B, Nnew = int(new_rows.shape[0]), int(new_rows.shape[1])
    for b in range(B):
        c = int(cache_lens[b])
        for r in range(Nnew):
            t = c + r
            blk = _table_entry(table[b], t // block_size)
            if blk < 0 or blk >= _rows(pool):
                raise IndexError(f"no block for position {t} of sequence {b}")
            out[blk, t % block_size] = new_rows[b, r]
    return out
