"""Pins of the oracle's block pool and chat-serving simulation (CPU only).

"Phase 07 · 12", sections "Paged attention" and "Exercises" (item 3): a
sequence of n tokens lives in ceil(n / 16) fixed 16-token blocks, and a
finished sequence's blocks return to the pool. The pins are closed forms of
that rule and conservation laws any correct schedule obeys; none of them
re-runs the oracle's own code path to produce its expected value.
"""

import random

import pytest

from oracle import pool as op


@pytest.mark.parametrize("n,blocks", [(0, 0), (1, 1), (15, 1), (16, 1), (17, 2), (32, 2),
                                      (33, 3), (16384, 1024), (16385, 1025)])
def test_blocks_for_closed_form(n, blocks):
    assert op.blocks_for(n) == blocks


def test_set_pool_counts_and_ownership():
    rng = random.Random(3)
    pool = op.SetPool(50)
    lens = {}
    for _ in range(2000):
        s = rng.randrange(8)
        if s in lens and rng.random() < 0.3:
            pool.release(s)
            del lens[s]
            continue
        cur = lens.get(s, 0)
        new = cur + rng.randrange(0, 40)
        free_before = len(pool.free)
        ok = pool.grow(s, cur, new)
        need = -(-new // 16) - -(-cur // 16)
        assert ok == (need <= free_before)
        if ok:
            lens[s] = new
        else:
            assert len(pool.free) == free_before
        held = [e for v in pool.held.values() for e in v]
        assert len(held) == len(set(held)) == 50 - len(pool.free)
        assert not set(held) & pool.free
        for t, n in lens.items():
            assert len(pool.held.get(t, [])) == -(-n // 16)


def _check_laws(prompts, outputs, num_blocks, steps, recs):
    n = len(prompts)
    # every chat is admitted once more than it is preempted, and finishes once
    assert sum(r[3] for r in recs) - sum(r[5] for r in recs) == n
    assert sum(r[4] for r in recs) == n
    # one token per running chat per step: the step-chat count is the output total
    assert sum(r[0] for r in recs) == sum(outputs)
    for running, live, blocks, _, _, _ in recs:
        assert blocks <= num_blocks
        # only running chats hold blocks, each fewer than 16 positions unused
        assert live <= 16 * blocks < live + 16 * max(running, 1)
    assert steps == len(recs)


def test_single_chat():
    steps, recs = op.simulate_paged([100], [37], 64)
    assert steps == 37
    for k, (running, live, blocks, adm, fin, pre) in enumerate(recs, start=1):
        assert running == 1 and pre == 0
        assert live == 100 + k
        assert blocks == -(-(100 + k) // 16)
        assert adm == (1 if k == 1 else 0) and fin == (1 if k == 37 else 0)


def test_roomy_pool_runs_everything_at_once():
    prompts = [20, 300, 64, 1000, 5]
    outputs = [7, 50, 1, 33, 90]
    steps, recs = op.simulate_paged(prompts, outputs, 10_000)
    assert steps == max(outputs)
    assert recs[0][0] == len(prompts) and recs[0][3] == len(prompts)
    assert sum(r[5] for r in recs) == 0
    _check_laws(prompts, outputs, 10_000, steps, recs)


def test_one_chat_at_a_time_when_only_one_fits():
    # a pool of 4 blocks holds one chat of <= 64 tokens at a time: the chats
    # run back to back, so the makespan is the sum of the outputs
    prompts = [10, 30, 20]
    outputs = [20, 10, 40]
    steps, recs = op.simulate_paged(prompts, outputs, 4)
    _check_laws(prompts, outputs, 4, steps, recs)
    assert max(r[0] for r in recs) <= 2
    assert steps >= max(outputs)


def test_tight_pool_preempts_and_conserves():
    rng = random.Random(11)
    prompts = [rng.randint(16, 200) for _ in range(60)]
    outputs = [rng.randint(1, 150) for _ in range(60)]
    steps, recs = op.simulate_paged(prompts, outputs, 40)
    assert sum(r[5] for r in recs) > 0
    _check_laws(prompts, outputs, 40, steps, recs)


def test_chat_that_cannot_fit_is_an_error():
    with pytest.raises(ValueError):
        op.simulate_paged([100], [10], 4)  # 110 tokens need 7 blocks


def test_planted_mistake_fails_a_pin(monkeypatch):
    # blocks counted with floor instead of ceil: the single-chat pin must fail
    monkeypatch.setattr(op, "blocks_for", lambda n: int(n) // 16)
    steps, recs = op.simulate_paged([100], [37], 64)
    assert any(blocks != -(-(100 + k) // 16) for k, (_, _, blocks, _, _, _) in
               enumerate(recs, start=1))
