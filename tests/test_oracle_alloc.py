"""Pins for RefAllocator: the rules the pages state, checked on seeded random traces.

Pages: [SLAVA] lead paragraph (table from logical positions to physical blocks),
section "Ungenutzten Platz in Blöcken berechnen" (grow on demand, free at the
end), section "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung" and
[AIU] FAQ (several requests share a block; copy only on divergence, the shared
original stays intact); [ART] paged-attention paragraph (running out of
blocks is what triggers preemption).
"""

import numpy as np
import pytest

import oracle


def _invariants(a):
    # refcount conservation: each table entry holds one reference
    total_refs = sum(a.refcount)
    assert total_refs == sum(len(t) for t in a.tables.values())
    used = sum(1 for r in a.refcount if r > 0)
    assert used + len(a.free) == a.num_blocks
    assert all(a.refcount[b] == 0 for b in a.free)
    assert len(set(a.free)) == len(a.free)
    for sid, t in a.tables.items():
        assert len(t) == oracle.blocks_needed(a.lengths[sid], a.block_size)


def _slot_of(table, p, B):
    return table[p // B] * B + p % B


def test_slots_follow_table_bruteforce():
    rng = np.random.default_rng(0)
    a = oracle.RefAllocator(200, 16, rng.permutation(200))
    seqs = [a.create() for _ in range(5)]
    owner = {}
    for _ in range(60):
        s = int(rng.choice(seqs))
        n = int(rng.integers(0, 40))
        start = a.length(s)
        slots, pairs = a.append(s, n)
        assert pairs == []
        table = a.block_table(s)
        for k, p in enumerate(range(start, start + n)):
            assert slots[k] == _slot_of(table, p, 16)
            assert slots[k] not in owner      # private sequences never reuse a live slot
            owner[slots[k]] = (s, p)
        _invariants(a)


def test_free_returns_blocks_and_reuse_is_fifo():
    a = oracle.RefAllocator(8, 4, [7, 6, 5, 4, 3, 2, 1, 0])
    s0, s1 = a.create(), a.create()
    a.append(s0, 9)                    # 3 blocks: 7,6,5
    a.append(s1, 4)                    # 1 block: 4
    assert a.block_table(s0) == [7, 6, 5] and a.block_table(s1) == [4]
    a.free_seq(s0)
    assert list(a.free) == [3, 2, 1, 0, 7, 6, 5]
    s2 = a.create()
    a.append(s2, 5)
    assert a.block_table(s2) == [3, 2]
    _invariants(a)


def test_fork_shares_and_cow_on_divergence():
    B = 16
    a = oracle.RefAllocator(32, B)
    p = a.create()
    a.append(p, 40)                    # blocks 0,1,2 (2 is partly filled)
    c = a.fork(p, 40)
    assert a.block_table(c) == a.block_table(p) == [0, 1, 2]
    assert [a.refcount[b] for b in (0, 1, 2)] == [2, 2, 2]
    # the child writes position 40 inside shared block 2 -> one copy
    slots, pairs = a.append(c, 1)
    assert pairs == [(2, 3)]
    assert a.block_table(c) == [0, 1, 3] and a.block_table(p) == [0, 1, 2]
    assert slots == [3 * B + 40 % B]
    assert [a.refcount[b] for b in (0, 1, 2, 3)] == [2, 2, 1, 1]
    # the parent now owns block 2 alone: writing into it copies nothing
    slots, pairs = a.append(p, 3)
    assert pairs == [] and slots == [2 * B + 8, 2 * B + 9, 2 * B + 10]
    _invariants(a)


def test_fork_at_block_edge_never_copies():
    a = oracle.RefAllocator(16, 16)
    p = a.create()
    a.append(p, 32)
    c = a.fork(p, 32)
    slots, pairs = a.append(c, 20)
    assert pairs == [] and a.block_table(c)[:2] == [0, 1]
    assert a.refcount[0] == 2 and a.refcount[1] == 2


def test_fork_inside_block_copies_once_per_block():
    a = oracle.RefAllocator(16, 16)
    p = a.create()
    a.append(p, 30)
    c = a.fork(p, 21)                  # shares blocks 0,1; child stops inside block 1
    slots, pairs = a.append(c, 12)     # positions 21..32: copy block 1 once, then a fresh block
    assert pairs == [(1, 2)]
    assert a.block_table(c) == [0, 2, 3]
    assert slots[:11] == [2 * 16 + p for p in range(5, 16)] and slots[11] == 3 * 16
    _invariants(a)


def test_out_of_blocks_is_atomic_then_preemption_frees():
    a = oracle.RefAllocator(32, 16)
    s = [a.create() for _ in range(4)]
    for x in s:
        a.append(x, 16 * 8)            # 8 blocks each: pool exhausted
    before = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
    with pytest.raises(oracle.OutOfBlocks):
        a.append(s[0], 1)
    after = (list(a.free), list(a.refcount), {k: list(v) for k, v in a.tables.items()}, dict(a.lengths))
    assert before == after
    a.free_seq(s[3])                   # preempt one request
    slots, _ = a.append(s[0], 1)
    assert len(slots) == 1
    _invariants(a)


def test_random_traces_with_sharing():
    rng = np.random.default_rng(7)
    for trial in range(20):
        nb = int(rng.integers(20, 80))
        B = int(rng.choice([1, 2, 4, 16]))
        a = oracle.RefAllocator(nb, B, rng.permutation(nb))
        live = []
        for step in range(80):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    live.append(a.create())
                elif op == 1:
                    par = int(rng.choice(live))
                    live.append(a.fork(par, int(rng.integers(0, a.length(par) + 1))))
                elif op == 2:
                    s = int(rng.choice(live))
                    start = a.length(s)
                    old_tables = {k: list(v) for k, v in a.tables.items()}
                    shared_before = {b for b in range(nb) if a.refcount[b] > 1}
                    slots, pairs = a.append(s, int(rng.integers(0, 3 * B)))
                    table = a.block_table(s)
                    for k, slot in enumerate(slots):
                        assert slot == _slot_of(table, start + k, B)
                    for old, new in pairs:
                        assert old in shared_before       # only shared blocks are copied
                        assert a.refcount[new] == 1
                    # other sequences' tables are untouched by this append
                    for k, v in a.tables.items():
                        if k != s:
                            assert v == old_tables[k]
                else:
                    s = live.pop(int(rng.integers(0, len(live))))
                    a.free_seq(s)
            except oracle.OutOfBlocks:
                pass
            _invariants(a)
