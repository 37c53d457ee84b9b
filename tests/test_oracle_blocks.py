"""Pins for the block accounting and the allocator's block counts.

[SLAVA] section "Ungenutzten Platz in Blöcken berechnen" prints a worked case
(35 tokens, 16-slot blocks: 3 blocks, 48 slots, 13 empty, about 27%) and states
that only the last block can be partly filled.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_worked_example_closed_form():
    ex = json.load(open(GOLDEN))
    B, n = ex["block_size"], ex["tokens"]
    assert oracle.blocks_needed(n, B) == ex["blocks"]
    assert oracle.blocks_needed(n, B) * B == ex["slots"]
    assert oracle.unused_slots(n, B) == ex["unused"]
    assert round(100 * oracle.unused_fraction(n, B)) == ex["unused_percent_about"]


def test_worked_example_through_allocator():
    ex = json.load(open(GOLDEN))
    a = oracle.RefAllocator(64, ex["block_size"])
    s = a.create()
    slots, pairs = a.append(s, ex["tokens"])
    st = a.stats()
    assert pairs == []
    assert len(a.block_table(s)) == ex["blocks"]
    assert st["slots_logical"] == ex["slots"]
    assert st["slots_logical"] - st["tokens_logical"] == ex["unused"]
    assert len(slots) == ex["tokens"]


@pytest.mark.parametrize("B", [1, 2, 4, 16, 32, 64])
def test_only_last_block_partial(B):
    for n in range(0, 5 * B + 3):
        nb = oracle.blocks_needed(n, B)
        # nb blocks hold n tokens; nb-1 would not (fewest blocks)
        assert nb * B >= n and (nb - 1) * B < max(n, 1) or n == 0
        assert 0 <= oracle.unused_slots(n, B) <= B - 1
        a = oracle.RefAllocator(nb + 1, B)
        s = a.create()
        slots, _ = a.append(s, n)
        table = a.block_table(s)
        assert len(table) == nb
        # every block but the last is full: positions 0..B*(nb-1)-1 fill the first nb-1 blocks
        per_block = np.bincount(np.asarray(slots, dtype=np.int64) // B, minlength=nb + 1)
        full = [per_block[b] for b in table[:-1]]
        assert all(f == B for f in full)


def test_waste_shrinks_with_length():
    fr = [oracle.unused_fraction(16 * k + 3, 16) for k in range(1, 50)]
    assert all(a > b for a, b in zip(fr, fr[1:]))


def test_tiny_decode_counts():
    # contexts {35,16,1,50} at 16 slots/block: 3,1,1,4 blocks; 13,0,15,14 slots empty
    L = [35, 16, 1, 50]
    assert [oracle.blocks_needed(n, 16) for n in L] == [3, 1, 1, 4]
    assert [oracle.unused_slots(n, 16) for n in L] == [13, 0, 15, 14]
    a = oracle.RefAllocator(32, 16)
    for n in L:
        s = a.create()
        a.append(s, n)
    st = a.stats()
    assert st["blocks_used"] == 9 and st["slots_logical"] == 144
    assert st["slots_logical"] - st["tokens_logical"] == 42
