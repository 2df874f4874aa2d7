"""A second, tiled path through the same attention, used only to pin the oracle.

"Phase 07 · 12: KV cache, Flash Attention and inference optimisation", section
"Build it, step 2", and "大模型面试笔记——Attention篇" §2 describe streaming the
keys in tiles while keeping, per query row, a running maximum m, a running
denominator l and an unnormalised output. When a tile raises the maximum, the
old l and the old output are multiplied by exp(m_old - m_new) (taken as 0 while
m_old is still -inf); the tile's own terms are exp(s - m_new); the division by
l happens once, after the last tile. The pages state that this reproduces the
full softmax result exactly (up to floating-point reassociation); the oracle's
self-tests check exactly that for every tile size.

Written here from that description, in fp64, one query row at a time.
"""

import math

import numpy as np

from .attention import NEG_INF, _f64


def online_attention_rows(q, pos, k, v, scale, causal, tile):
    """Tiled running-(max, sum) attention; same contract as attention_rows."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    pos = np.asarray(pos, dtype=np.int64)
    R = q.shape[0]
    n = k.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full((R,), NEG_INF, dtype=np.float64)
    for r in range(R):
        run_max = NEG_INF
        run_sum = 0.0
        acc = np.zeros(v.shape[1], dtype=np.float64)
        limit = min(n, int(pos[r]) + 1) if causal else n
        for start in range(0, limit, tile):
            stop = min(limit, start + tile)
            s = scale * (k[start:stop] @ q[r])
            tile_max = float(s.max())
            new_max = max(run_max, tile_max)
            carry = 0.0 if run_max == NEG_INF else math.exp(run_max - new_max)
            e = np.exp(s - new_max)
            run_sum = run_sum * carry + float(e.sum())
            acc = acc * carry + e @ v[start:stop]
            run_max = new_max
        if run_sum > 0.0:
            out[r] = acc / run_sum
            lse[r] = run_max + math.log(run_sum)
    return out, lse
