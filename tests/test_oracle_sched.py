"""Pins of the admission/allocation model (oracle/sched.py) against the pages' own
numbers and against invariants that do not come from the model.

Numbers the pages fix: the budget formula with the clamp to the context, the
128 MiB default pool, that full-context requests used to be limited to two at
a time in it, that a smaller pool queues requests whose budgets cannot fit
together, rejection of a budget above the whole pool, and release on early
completion.  Invariants checked on random traces: conservation of credits and
pages, no page owned twice, and that every active request can always grow to
its full budget (no deadlock).
"""
import numpy as np
import pytest

from oracle.sched import PAGE_TOKENS, SchedModel, budget_pages

PAGE_BYTES = PAGE_TOKENS * 8 * 64 * 2 * 2  # 16 tokens x 8 kv heads x 64 dims x bf16 x (K, V)


@pytest.mark.parametrize("prompt,max_new,pages", [
    (10, 64, 5 * 16),      # 73 processed tokens -> 5 pages per layer
    (1, 1, 1 * 16),        # only the prompt token is processed
    (16, 1, 1 * 16),
    (16, 2, 2 * 16),       # 17 tokens spill into a second page
    (2000, 128, 128 * 16),  # output clamped to 48: 2047 processed tokens
    (2047, 5, 128 * 16),
    (100, 29, 8 * 16),     # 128 processed tokens: exactly 8 pages
    (100, 30, 9 * 16),
])
def test_budget_formula(prompt, max_new, pages):
    assert budget_pages(prompt, max_new, 2048, 16) == pages


def test_default_pool_holds_two_full_context_requests():
    pool = (128 << 20) // PAGE_BYTES
    assert pool == 4096
    s = SchedModel(pool)
    ids = [s.submit(1024, 4096) for _ in range(3)]  # clamped to 1024 new -> 2047 processed
    assert s.admit() == ids[:2] and len(s.waiting) == 1
    s.finish(ids[0])
    assert s.admit() == [ids[2]]


def test_small_pool_queues_and_rejects():
    pool = (8 << 20) // PAGE_BYTES  # --kv-cache-mib 8
    assert pool == 256
    s = SchedModel(pool)
    a = s.submit(40, 64)   # 103 tokens -> 7 pages x 16 = 112
    b = s.submit(40, 64)
    c = s.submit(40, 64)
    assert s.submit(100, 2000) is None and s.stats["rejected"] == 1  # 2048 pages > 256
    assert s.admit() == [a, b] and [r.rid for r in s.waiting] == [c]
    assert s.stats["admission_waits"] == 1


def test_fifo_is_strict():
    s = SchedModel(64 * 16)
    big = s.submit(1000, 24)        # 1023 tokens -> 64 pages per layer: the whole pool
    small = s.submit(5, 5)
    first = s.submit(5, 5)
    assert s.admit() == [big]
    s2 = SchedModel(64 * 16)
    x = s2.submit(5, 5)
    big2 = s2.submit(1000, 24)
    y = s2.submit(5, 5)
    assert s2.admit() == [x]        # big2 does not fit beside x, and y may not pass it
    assert [r.rid for r in s2.waiting] == [big2, y]
    del small, first


def test_lazy_pages_and_release_on_early_finish():
    s = SchedModel(4096)
    r = s.submit(20, 100)           # 119 tokens -> 8 pages per layer of credit
    assert s.admit() == [r]
    assert s.credits_free == 4096 - 128 and s.assigned_pages() == 0  # credits, no pages yet
    assert s.grow(r, 20)             # prefill: 2 pages per layer
    assert s.assigned_pages() == 32
    assert s.grow(r, 33)             # third page in every layer
    assert s.assigned_pages() == 48
    assert not s.grow(r, 120)        # beyond the reserved prefix
    s.finish(r)                      # stops early
    assert s.assigned_pages() == 0 and s.credits_free == 4096


def test_static_mode_waits_for_the_whole_group():
    s = SchedModel(4096, static=True)
    a, b = s.submit(10, 10), s.submit(10, 10)
    assert s.admit() == [a, b]
    c = s.submit(10, 10)
    s.finish(a)
    assert s.admit() == []          # b still running
    s.finish(b)
    assert s.admit() == [c]


def test_stats_on_a_worked_trace():
    s = SchedModel(256)
    a = s.submit(40, 64)            # 112 pages of credit
    b = s.submit(40, 64)
    c = s.submit(40, 64)
    s.admit()                       # a, b; c waits
    for r in (a, b):
        s.grow(r, 40)               # 3 pages per layer each
    s.decode_batch(2)
    s.grow(a, 49)                   # a's 4th page
    s.finish(a)
    s.admit()                       # c
    s.grow(c, 40)
    s.decode_batch(2)
    snap = s.snapshot()
    assert snap["pool_pages"] == 256 and snap["peak_active"] == 2 and snap["largest_decode_batch"] == 2
    assert snap["peak_assigned_pages"] == (4 + 3) * 16 and snap["admission_waits"] == 1
    assert snap["free_pages"] == 256 - 6 * 16 and snap["completed"] == 1


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_the_invariants(seed):
    rng = np.random.default_rng(seed)
    s = SchedModel(int(rng.choice([256, 1024, 4096])), static=bool(seed % 2))
    progress = {}
    for step in range(400):
        if rng.random() < 0.3:
            rid = s.submit(int(rng.integers(1, 600)), int(rng.integers(1, 400)))
            if rid is not None:
                progress[rid] = 0
        for rid in s.admit():
            assert s.grow(rid, s.active[rid].prompt)  # prefill never fails once admitted
            progress[rid] = s.active[rid].prompt
        live = list(s.active)
        s.decode_batch(len(live))
        for rid in live:
            r = s.active[rid]
            if progress[rid] >= r.limit or rng.random() < 0.02:  # budget used up, or stops early
                s.finish(rid)
                continue
            progress[rid] += 1
            assert s.grow(rid, progress[rid]), "an admitted request could not grow within its budget"
        # conservation and ownership
        held = sum(r.credits for r in s.active.values())
        assert s.credits_free + held == s.pool
        owned = [p for r in s.active.values() for t in r.tables for p in t]
        assert len(owned) == len(set(owned)) == s.assigned_pages()
        assert all(0 <= p < s.pool for p in owned)
        for r in s.active.values():
            assert all(len(t) == -(-r.length // PAGE_TOKENS) for t in r.tables)
            assert len(r.tables[0]) * s.layers <= r.credits
