"""Chat-serving simulation of a KV cache: paged blocks against contiguous slabs.

"Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
section "Exercises", item 3: keep the cache in fixed 16-token blocks, return a
sequence's blocks to the pool when it finishes, simulate 1000 chat
completions of differing lengths and compare the memory fragmentation with
contiguous allocation. The paged side runs on the library's native block pool
(``BlockPool``, the C ABI's attn_block_pool_*), with a real block-table row
per chat; the contiguous side is a first-fit allocator over one linear range
of cache positions, written here only as the comparison.

Schedule (shared by every scheme): all chats wait in a first-come queue at
step 0; each step every running chat writes one token, then queued chats are
admitted in order while the cache can take them (the first that does not fit
stops admission), then the step is recorded, then finished chats free their
memory.
  * paged: a chat holds ceil(len / 16) blocks and grows one block at a time;
    admission needs the blocks of its context plus this step's token; when a
    running chat finds no free block, the most recently admitted running chat
    is preempted (blocks freed, back to the head of the queue, its generated
    tokens recomputed as prompt on re-admission).
  * contiguous, reserve-max: a chat reserves prompt + max_new_tokens
    positions at admission (its output length is unknown in advance).
  * contiguous, reserve-exact: a chat reserves exactly prompt + output
    positions (an oracle that knows every output length; the best contiguous
    can do).
"""

import numpy as np

from . import BLOCK_TOKENS, BlockPool


def _blocks(n):
    return (int(n) + BLOCK_TOKENS - 1) // BLOCK_TOKENS


def run_paged(prompts, outputs, num_blocks, check_tables=True):
    """Paged scheme on the native pool. Returns a dict with ``records``: one
    (running, live_tokens, blocks_in_use, admitted, finished, preempted) per
    step, and summary figures."""
    n = len(prompts)
    pool = BlockPool(num_blocks)
    max_ctx = max(int(p) + int(r) for p, r in zip(prompts, outputs))
    tables = np.full((n, _blocks(max_ctx) + 1), -1, dtype=np.int32)
    gen = np.zeros(n, dtype=np.int64)
    length = np.zeros(n, dtype=np.int64)
    queue = list(range(n))
    running = []
    records = []
    while queue or running:
        preempted = 0
        i = 0
        while i < len(running):
            c = running[i]
            if pool.grow(tables[c], length[c], length[c] + 1):
                length[c] += 1
                gen[c] += 1
                i += 1
                continue
            victim = running.pop()
            pool.release(tables[victim], length[victim])
            length[victim] = 0
            queue.insert(0, victim)
            preempted += 1
            # the growing chat itself was the newest: it waits in the queue now
            # (otherwise retry its grow with the freed blocks)
        admitted = 0
        while queue:
            c = queue[0]
            ctx = int(prompts[c]) + int(gen[c]) + 1
            if not pool.grow(tables[c], 0, ctx):
                break
            queue.pop(0)
            length[c] = ctx
            gen[c] += 1
            running.append(c)
            admitted += 1
        if not running and queue:
            raise ValueError("a chat does not fit in the pool on its own")
        in_use = num_blocks - pool.free_count()
        if check_tables:
            ids = np.concatenate([tables[c][:_blocks(length[c])] for c in running]) \
                if running else np.empty(0, np.int32)
            if len(ids) != in_use or len(np.unique(ids)) != len(ids) or \
                    (len(ids) and (ids.min() < 0 or ids.max() >= num_blocks)):
                raise AssertionError("block tables are inconsistent with the pool")
        records.append((len(running), int(sum(length[c] for c in running)), in_use, admitted,
                        0, preempted))
        finished = 0
        still = []
        for c in running:
            if gen[c] >= outputs[c]:
                pool.release(tables[c], length[c])
                length[c] = 0
                finished += 1
            else:
                still.append(c)
        running = still
        r = records[-1]
        records[-1] = (r[0], r[1], r[2], r[3], finished, r[5])
    if pool.free_count() != num_blocks:
        raise AssertionError("blocks leaked")
    return _summary("paged", records, num_blocks * BLOCK_TOKENS,
                    reserved=lambda rec: rec[2] * BLOCK_TOKENS)


def run_contiguous(prompts, outputs, capacity, max_new_tokens=None):
    """Contiguous first-fit scheme over ``capacity`` positions. With
    ``max_new_tokens`` each chat reserves prompt + max_new_tokens (reserve-max),
    else prompt + its own output length (reserve-exact)."""
    n = len(prompts)
    holes = [(0, int(capacity))]  # (start, size), sorted by start, never adjacent
    where = {}
    gen = np.zeros(n, dtype=np.int64)
    queue = list(range(n))
    running = []
    records = []
    blocked_by_holes = 0

    def need(c):
        return int(prompts[c]) + int(max_new_tokens if max_new_tokens is not None else outputs[c])

    def take(size):
        for i, (s, z) in enumerate(holes):
            if z >= size:
                if z == size:
                    holes.pop(i)
                else:
                    holes[i] = (s + size, z - size)
                return s
        return None

    def give(s, size):
        holes.append((s, size))
        holes.sort()
        merged = []
        for a, z in holes:
            if merged and merged[-1][0] + merged[-1][1] == a:
                merged[-1] = (merged[-1][0], merged[-1][1] + z)
            else:
                merged.append((a, z))
        holes[:] = merged

    while queue or running:
        for c in running:
            gen[c] += 1
        admitted = 0
        while queue:
            c = queue[0]
            size = need(c)
            if size > capacity:
                raise ValueError("a chat does not fit in the cache on its own")
            s = take(size)
            if s is None:
                if sum(z for _, z in holes) >= size:
                    blocked_by_holes += 1
                break
            queue.pop(0)
            where[c] = (s, size)
            gen[c] += 1
            running.append(c)
            admitted += 1
        live = int(sum(int(prompts[c]) + int(gen[c]) for c in running))
        reserved = int(sum(where[c][1] for c in running))
        finished = 0
        still = []
        for c in running:
            if gen[c] >= outputs[c]:
                give(*where.pop(c))
                finished += 1
            else:
                still.append(c)
        records.append((len(still) + finished, live, reserved, admitted, finished, 0))
        running = still
    name = "contiguous_reserve_max" if max_new_tokens is not None else "contiguous_reserve_exact"
    out = _summary(name, records, capacity, reserved=lambda rec: rec[2])
    out["admissions_blocked_by_holes"] = blocked_by_holes
    return out


def _summary(name, records, capacity, reserved):
    steps = len(records)
    live = np.array([r[1] for r in records], dtype=np.float64)
    res = np.array([reserved(r) for r in records], dtype=np.float64)
    run = np.array([r[0] for r in records], dtype=np.float64)
    return {
        "scheme": name,
        "steps": steps,
        "mean_running": float(run.mean()) if steps else 0.0,
        "peak_running": int(run.max()) if steps else 0,
        "mean_live_over_capacity": float((live / capacity).mean()) if steps else 0.0,
        "mean_live_over_reserved": float((live / np.maximum(res, 1)).mean()) if steps else 0.0,
        "preemptions": int(sum(r[5] for r in records)),
        "records": records,
    }


def compare(prompts, outputs, capacity_tokens, max_new_tokens):
    """The three schemes on one draw of chats; records dropped."""
    out = []
    for r in (run_paged(prompts, outputs, capacity_tokens // BLOCK_TOKENS, check_tables=False),
              run_contiguous(prompts, outputs, capacity_tokens, max_new_tokens),
              run_contiguous(prompts, outputs, capacity_tokens)):
        r = dict(r)
        r.pop("records")
        out.append(r)
    return out
