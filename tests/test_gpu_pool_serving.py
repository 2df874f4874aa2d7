"""Serving on the GPU with the native block pool: sequences finish, their
blocks return to the pool ("Phase 07 · 12", sections "Paged attention" and
"Exercises", item 3) and new sequences reuse them while stale rows from the
old owners still sit in the reused blocks. The pool fills host table rows;
kv_append writes through them and the paged decode reads through them, and
every decode is checked against the oracle's own append and gather of the
same tables (the stale rows past a sequence's length must stay invisible).
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta
import oracle
from tests.gpu_helpers import announce, check, need_gpu

pytestmark = pytest.mark.gpu

Hq, Hkv, d = 8, 2, 128
MB = 16          # table entries per sequence (256 positions)
POOL = 20        # physical blocks: far fewer than 4 sequences x 16


def _draw(g, n):
    return torch.randn((1, n, Hkv, d), generator=g).to(torch.bfloat16)


class Server:
    """Host state of a few sequences on one paged pool, mirrored on the CPU
    for the oracle."""

    def __init__(self, dev, seed):
        self.dev = dev
        self.g = torch.Generator().manual_seed(seed)
        self.pool = eta.BlockPool(POOL)
        # device pools start as NaN-free noise so stale rows are real values
        self.kp_cpu = torch.randn((POOL, 16, Hkv, d), generator=self.g).to(torch.bfloat16)
        self.vp_cpu = torch.randn((POOL, 16, Hkv, d), generator=self.g).to(torch.bfloat16)
        self.kp = self.kp_cpu.to(dev)
        self.vp = self.vp_cpu.to(dev)
        self.rows = {}
        self.lens = {}

    def start(self, s):
        self.rows[s] = np.full(MB, -1, np.int32)
        self.lens[s] = 0

    def append(self, s, n):
        """n new K/V rows for sequence s: blocks from the pool, kv_append on the
        GPU, the oracle's own append on the CPU mirror."""
        assert self.pool.grow(self.rows[s], self.lens[s], self.lens[s] + n)
        k, v = _draw(self.g, n), _draw(self.g, n)
        table = torch.from_numpy(self.rows[s].copy()).view(1, MB)
        cl = torch.tensor([self.lens[s]], dtype=torch.int32)
        eta.kv_append(k.to(self.dev), v.to(self.dev), self.kp, self.vp, cl.to(self.dev),
                      block_table=table.to(self.dev))
        self.kp_cpu = oracle.kv_append_ref(self.kp_cpu, k, table, cl)
        self.vp_cpu = oracle.kv_append_ref(self.vp_cpu, v, table, cl)
        self.lens[s] += n

    def finish(self, s):
        self.pool.release(self.rows[s], self.lens[s])
        del self.rows[s], self.lens[s]

    def decode(self, seqs, Nq, what):
        """Append Nq new tokens to each of `seqs`, then one paged decode over
        them, checked against the oracle."""
        for s in seqs:
            self.append(s, Nq)
        table = torch.from_numpy(np.stack([self.rows[s] for s in seqs]))
        sl = torch.tensor([self.lens[s] for s in seqs], dtype=torch.int32)
        q = torch.randn((len(seqs), Nq, Hq, d), generator=self.g).to(torch.bfloat16)
        o, lse = eta.attn_decode_paged(q.to(self.dev), self.kp, self.vp, sl.to(self.dev),
                                       block_table=table.to(self.dev), causal=True)
        torch.cuda.synchronize()
        O, L = oracle.decode_attention(q, self.kp_cpu, self.vp_cpu, sl, 1 / math.sqrt(d), True,
                                       block_table=table)
        check(o, O, lse, L, "bf16", what)


def test_blocks_reused_after_finish():
    dev = need_gpu()
    announce(f"pool-driven serving Hq={Hq} Hkv={Hkv} d={d} pool={POOL} blocks, block reuse")
    srv = Server(dev, 77)
    for s, n in ((0, 70), (1, 100), (2, 37)):
        srv.start(s)
        srv.append(s, n)
    srv.decode([0, 1, 2], 4, "3 sequences, 4-token decode")
    used = POOL - srv.pool.free_count()
    srv.finish(0)                               # its 5 blocks (74 tokens) go back
    assert srv.pool.free_count() == POOL - used + 5
    srv.start(3)
    srv.append(3, 50)                           # takes 4 of those blocks; the tail
    assert POOL - srv.pool.free_count() == used - 1   # of its last one holds stale rows
    srv.decode([1, 3, 2], 1, "after reuse, 1-token decode")
    srv.finish(2)
    srv.start(4)
    srv.append(4, 3)
    srv.decode([4, 3, 1], 4, "second reuse, 4-token decode")
    for s in list(srv.rows):
        srv.finish(s)
    assert srv.pool.free_count() == POOL
