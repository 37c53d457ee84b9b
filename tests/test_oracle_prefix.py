"""Pins for the prefix cache of RefAllocator and its chained block hash.

Page: [ART] paragraph on prefix caching -- token blocks are hashed and kept, a
request that starts with the same tokens reuses the matching blocks instead of
recomputing them; [HADA] bullet "Prefix Caching".  The hash function is not
named there: FNV-1a 64 is a reading, pinned here against the published FNV
test vectors; the rest is pinned by closed-form hit counts, a hand-worked
eviction trace and invariants on random traces.
"""

import numpy as np
import pytest

import oracle
from oracle.prefix import FNV_OFFSET

B = 16


def test_fnv1a64_published_vectors():
    # FNV-1a 64 test vectors from the FNV authors' published test suite.
    assert oracle.fnv1a64(b"") == 0xCBF29CE484222325
    assert oracle.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert oracle.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_fnv1a64_continues_from_a_state():
    # Hashing in two pieces equals hashing the concatenation (byte-serial definition).
    assert oracle.fnv1a64(b"bar", oracle.fnv1a64(b"foo")) == oracle.fnv1a64(b"foobar")


def test_chain_names_the_whole_prefix():
    rng = np.random.default_rng(1)
    toks = rng.integers(0, 50000, size=5 * B + 7).tolist()
    h = oracle.chain(toks, B)
    assert len(h) == 5                      # full blocks only
    assert len(set(h)) == 5
    # a change in block 2 changes blocks 2.. and leaves 0, 1 alone
    t2 = list(toks)
    t2[2 * B + 3] += 1
    h2 = oracle.chain(t2, B)
    assert h2[:2] == h[:2] and all(a != b for a, b in zip(h2[2:], h[2:]))
    # the same block after a different prefix hashes differently
    t3 = list(toks)
    t3[0] += 1
    assert all(a != b for a, b in zip(oracle.chain(t3, B), h))
    # tokens are hashed as 4-byte ids: 256 and 1 differ even though 256 % 256 == 0
    assert oracle.block_hash(FNV_OFFSET, [256] * B) != oracle.block_hash(FNV_OFFSET, [0] * B)
    # negative ids hash as their 32-bit two's complement
    assert oracle.block_hash(FNV_OFFSET, [-1] * B) == oracle.block_hash(FNV_OFFSET, [0xFFFFFFFF] * B)


def _invariants(a):
    assert sum(a.refcount) == sum(len(t) for t in a.tables.values())
    assert sum(1 for r in a.refcount if r > 0) + len(a.free) == a.num_blocks
    assert all(a.refcount[b] == 0 for b in a.free)
    assert len(set(a.free)) == len(a.free)
    # the cache and the registry agree, one block per hash
    assert {blk: v[0] for blk, v in a.reg.items()} == {blk: h for h, blk in a.cache.items()}


@pytest.mark.parametrize("prompt_len, suffix_len, requests", [(64, 5, 8), (70, 1, 5), (16, 40, 4), (200, 16, 6)])
def test_shared_system_prompt_hits(prompt_len, suffix_len, requests):
    """R requests share a P-token prompt; each adds its own suffix.  The first
    registers its blocks; each later one reuses exactly the prompt's P // B full
    blocks (the block holding the prompt's tail and the suffix differs)."""
    rng = np.random.default_rng(prompt_len)
    prompt = rng.integers(0, 1000, size=prompt_len).tolist()
    a = oracle.RefAllocator(256, B)
    for r in range(requests):
        suffix = (100000 + r * 1000 + np.arange(suffix_len)).tolist()
        toks = prompt + suffix
        sid, cached = a.prefix_lookup(toks)
        want = 0 if r == 0 else min(prompt_len // B, (len(toks) - 1) // B) * B
        assert cached == want
        a.append(sid, len(toks) - cached)
        a.prefix_register(sid, toks)
        _invariants(a)
    st = a.prefix_stats()
    assert st["lookups"] == requests
    assert st["hit_blocks"] == (requests - 1) * (prompt_len // B)
    # registered: the prompt's full blocks once, plus each request's own full blocks past them
    own = (prompt_len + suffix_len) // B - prompt_len // B
    assert st["blocks_registered"] == prompt_len // B + requests * own
    assert st["evictions"] == 0


def test_lookup_leaves_one_token():
    a = oracle.RefAllocator(8, B)
    toks = list(range(2 * B))
    s = a.create()
    a.append(s, 2 * B)
    a.prefix_register(s, toks)
    assert a.prefix_lookup(toks)[1] == B            # 2B tokens: block 1 would leave none
    assert a.prefix_lookup(toks + [7])[1] == 2 * B
    assert a.prefix_lookup(toks[:B])[1] == 0
    assert a.prefix_lookup([])[1] == 0


def test_hand_worked_eviction():
    """Three blocks of 16.  Worked by hand:
    A = 33 tokens t -> blocks [0, 1, 2]; register -> 0, 1 cached (2 is partial).
    free A -> free list [0, 1, 2], both cached blocks on it.
    lookup(t) -> n_cached 32, blocks [0, 1] leave the free list -> free [2].
    append 1 -> block 2; free -> free list [0, 1, 2] (table order).
    C appends 1 token -> block 0, which is evicted when handed out.
    lookup(t) now misses at block 0; block 1 stays registered but unreachable.
    """
    t = list(range(1, 34))
    a = oracle.RefAllocator(3, B)
    s = a.create()
    a.append(s, 33)
    a.prefix_register(s, t)
    assert a.prefix_stats()["blocks_registered"] == 2
    a.free_seq(s)
    assert list(a.free) == [0, 1, 2] and a.prefix_stats()["registered_free"] == 2
    s2, cached = a.prefix_lookup(t)
    assert cached == 32 and a.block_table(s2) == [0, 1] and list(a.free) == [2]
    assert a.refcount[0] == 1 and a.refcount[1] == 1
    slots, pairs = a.append(s2, 1)
    assert slots == [2 * B] and pairs == []
    a.free_seq(s2)
    assert list(a.free) == [0, 1, 2]
    c = a.create()
    a.append(c, 1)
    assert a.block_table(c) == [0] and list(a.free) == [1, 2]
    st = a.prefix_stats()
    assert st["evictions"] == 1 and st["blocks_registered"] == 1 and 1 in a.reg
    s3, cached = a.prefix_lookup(t)
    assert cached == 0 and a.block_table(s3) == []
    _invariants(a)


def test_in_place_write_evicts():
    """A fork that shares a registered full block part-way, once the parent is
    gone, writes into that block in place: the block must leave the cache."""
    t = list(range(100, 100 + 2 * B))
    a = oracle.RefAllocator(6, B)
    p = a.create()
    a.append(p, 2 * B)
    a.prefix_register(p, t)
    child = a.fork(p, B + 4)                 # shares blocks 0 and 1 (1 part-way)
    slots, pairs = a.append(child, 1)        # refcount 2: copy-on-write, block 1 stays cached
    assert len(pairs) == 1 and a.prefix_stats()["evictions"] == 0
    child2 = a.fork(p, B + 4)
    a.free_seq(p)
    assert a.refcount[1] == 1
    slots, pairs = a.append(child2, 1)       # refcount 1: written in place
    assert pairs == [] and slots == [1 * B + B + 4 - B]
    st = a.prefix_stats()
    assert st["evictions"] == 1 and 1 not in a.reg and 0 in a.reg
    assert a.prefix_lookup(t + [0])[1] == B  # block 0 still hits, block 1 no longer
    _invariants(a)


def test_hit_requires_parent_and_tokens():
    """A lookup hits only along the chain: block 1 of another prompt is not
    reused even when its own 16 tokens match."""
    a = oracle.RefAllocator(8, B)
    x = list(range(B)) + list(range(500, 500 + B))
    s = a.create()
    a.append(s, 2 * B)
    a.prefix_register(s, x)
    y = list(range(1, B + 1)) + list(range(500, 500 + B)) + [9]
    assert a.prefix_lookup(y)[1] == 0
    assert a.prefix_lookup(x + [9])[1] == 2 * B


def test_register_keeps_first_block_for_a_hash():
    a = oracle.RefAllocator(8, B)
    t = list(range(B))
    s1, s2 = a.create(), a.create()
    a.append(s1, B)
    a.append(s2, B)
    a.prefix_register(s1, t)
    a.prefix_register(s2, t)                  # same hash: s2's block stays unregistered
    assert list(a.reg) == [a.block_table(s1)[0]]
    a.prefix_register(s1, t)                  # already registered: no change
    assert len(a.reg) == 1


@pytest.mark.parametrize("seed", range(6))
def test_random_traces_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(10, 60))
    a = oracle.RefAllocator(nb, B, rng.permutation(nb))
    prompts = [rng.integers(0, 30, size=int(rng.integers(1, 80))).tolist() for _ in range(3)]
    live = {}
    for _ in range(200):
        op = int(rng.integers(0, 4))
        if op == 0 or not live:
            toks = prompts[int(rng.integers(0, 3))] + rng.integers(0, 30, size=int(rng.integers(1, 20))).tolist()
            sid, cached = a.prefix_lookup(toks)
            assert cached % B == 0 and cached <= len(toks) - 1
            try:
                a.append(sid, len(toks) - cached)
            except oracle.OutOfBlocks:
                a.free_seq(sid)
            else:
                live[sid] = toks
        elif op == 1:
            sid = list(live)[int(rng.integers(0, len(live)))]
            a.prefix_register(sid, live[sid], int(rng.integers(0, len(live[sid]) + 1)))
        else:
            sid = list(live)[int(rng.integers(0, len(live)))]
            a.free_seq(sid)
            del live[sid]
        _invariants(a)
        # a cached block's recorded tokens are those of every live holder at that position
        for sid, toks in live.items():
            for j, blk in enumerate(a.block_table(sid)):
                if blk in a.reg and (j + 1) * B <= len(toks):
                    assert list(a.reg[blk][2]) == toks[j * B:(j + 1) * B]
