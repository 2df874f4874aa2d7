"""Block pool of a paged cache and the chat-serving simulation over it — TEST
INFRASTRUCTURE (the checker of the native pool and of the simulation driver).

Source: "Phase 07 · 12: KV cache, Flash Attention and inference optimisation",
section "Paged attention" (the cache is cut into 16-token blocks; a page table
maps logical positions to physical blocks) and section "Exercises", item 3
(a toy paged cache of fixed 16-token blocks whose blocks go back to the pool
when a sequence finishes; simulate 1000 chat completions of differing lengths
and compare the fragmentation with contiguous allocation).

The page fixes what the pool must guarantee, not which block it hands out, so
this model keeps the free blocks as a plain set and decides everything from
counts: a sequence of n tokens holds exactly ceil(n / 16) distinct blocks, a
request succeeds iff that many are free, and release returns them all. Any
pool that follows those rules makes the same admission, growth and preemption
decisions as this one, step for step.

Simulation (the reading taken of the exercise; the page gives no schedule):
all chats wait in a first-come queue at step 0. Each step
  1. every running chat writes one more token (its cache grows by one
     position); when the pool has no block for it, the most recently admitted
     running chat is preempted (its blocks freed, and it goes back to the head
     of the queue keeping the tokens it generated, which are recomputed as
     prompt when it is admitted again) until the grow succeeds or the growing
     chat is itself the one preempted;
  2. queued chats are admitted in order while the pool can hold their context
     (prompt + tokens generated before a preemption) plus the token this step
     writes; the first that does not fit stops admission;
  3. the step is recorded (running chats, live tokens, blocks in use);
  4. chats that have generated all their output tokens finish and release
     their blocks.
"""

BLOCK = 16


def blocks_for(n):
    """Blocks that hold positions 0..n-1: ceil(n / 16)."""
    return -(-int(n) // BLOCK)


class SetPool:
    """The plain pool: a set of free block ids and each sequence's list."""

    def __init__(self, num_blocks):
        self.num_blocks = int(num_blocks)
        self.free = set(range(self.num_blocks))
        self.held = {}  # sequence id -> list of block ids, logical order

    def grow(self, seq, cur_len, new_len):
        need = blocks_for(new_len) - blocks_for(cur_len)
        if need > len(self.free):
            return False
        mine = self.held.setdefault(seq, [])
        if len(mine) != blocks_for(cur_len):
            raise ValueError("sequence holds the wrong number of blocks")
        for _ in range(need):
            mine.append(self.free.pop())
        return True

    def release(self, seq):
        for e in self.held.pop(seq, []):
            if e in self.free:
                raise ValueError("block freed twice")
            self.free.add(e)

    def in_use(self):
        return self.num_blocks - len(self.free)


def simulate_paged(prompts, outputs, num_blocks):
    """Run the schedule above over a pool of ``num_blocks`` blocks.

    Returns (steps, records) with one record per step:
    (running, live_tokens, blocks_in_use, admitted, finished, preempted)."""
    n = len(prompts)
    pool = SetPool(num_blocks)
    gen = [0] * n          # tokens generated so far
    length = [0] * n       # tokens in the cache while running
    queue = list(range(n))
    running = []           # in admission order
    records = []
    while queue or running:
        preempted = 0
        # 1. grow every running chat by the token it writes this step
        i = 0
        while i < len(running):
            c = running[i]
            while not pool.grow(c, length[c], length[c] + 1):
                victim = running.pop()
                pool.release(victim)
                length[victim] = 0
                queue.insert(0, victim)
                preempted += 1
                if victim == c:
                    break
            else:
                length[c] += 1
                gen[c] += 1
                i += 1
        # 2. admit in order
        admitted = 0
        while queue:
            c = queue[0]
            ctx = prompts[c] + gen[c] + 1
            if not pool.grow(c, 0, ctx):
                pool.held.pop(c, None)
                break
            queue.pop(0)
            length[c] = ctx
            gen[c] += 1
            running.append(c)
            admitted += 1
        if not running and queue:
            raise ValueError("a chat does not fit in the pool on its own")
        # 3. record
        live = sum(length[c] for c in running)
        rec_running = len(running)
        rec_blocks = pool.in_use()
        # 4. finish and free
        finished = 0
        still = []
        for c in running:
            if gen[c] >= outputs[c]:
                pool.release(c)
                length[c] = 0
                finished += 1
            else:
                still.append(c)
        running = still
        records.append((rec_running, live, rec_blocks, admitted, finished, preempted))
    return len(records), records
