"""The library's host allocator against RefAllocator: identical op traces give
identical tables, slots, copy pairs, refcounts, free lists and statistics.

No GPU is involved: the allocator is host code in the same shared library.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import ensure_library


def same_state(lib_a, ref, live):
    assert lib_a.free_list() == list(ref.free)
    for b in range(ref.num_blocks):
        assert lib_a.refcount(b) == ref.refcount[b]
    for s_lib, s_ref in live:
        assert lib_a.block_table(s_lib) == ref.block_table(s_ref)
        assert lib_a.length(s_lib) == ref.length(s_ref)
    st = lib_a.stats()
    rs = ref.stats()
    for k in rs:
        assert st[k] == rs[k], k


@pytest.mark.parametrize("seed", range(12))
def test_random_traces_bit_exact(seed):
    pa = ensure_library()
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(8, 120))
    B = 16
    order = rng.permutation(nb)
    a = pa.BlockAllocator(nb, B, order)
    r = oracle.RefAllocator(nb, B, order)
    live = []
    for step in range(150):
        op = int(rng.integers(0, 5))
        if op == 0 or not live:
            live.append((a.create(), r.create()))
        elif op == 1:
            pl, pr = live[int(rng.integers(0, len(live)))]
            k = int(rng.integers(0, r.length(pr) + 1))
            live.append((a.fork(pl, k), r.fork(pr, k)))
        elif op in (2, 3):
            sl, sr = live[int(rng.integers(0, len(live)))]
            n = int(rng.integers(0, 40))
            try:
                want = r.append(sr, n)
            except oracle.OutOfBlocks:
                with pytest.raises(pa.OutOfBlocks):
                    a.append(sl, n)
            else:
                slots, pairs = a.append(sl, n)
                assert slots.tolist() == want[0]
                assert pairs == want[1]
        else:
            k = int(rng.integers(0, len(live)))
            sl, sr = live.pop(k)
            a.free_seq(sl)
            r.free_seq(sr)
        same_state(a, r, live)


@pytest.mark.parametrize("name", ["tiny_decode", "mixed_superbatch", "shared_prefix_cow"])
def test_named_workload_traces(name):
    pa = ensure_library()
    wl = workloads.named(name)
    a = pa.BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    r = oracle.RefAllocator(wl.num_blocks, wl.block_size, wl.free_order)
    ids_a, ctx_a, new_a, cow_a = workloads.drive(wl, a)
    ids_r, ctx_r, new_r, cow_r = workloads.drive(wl, r)
    assert np.array_equal(ctx_a, ctx_r) and np.array_equal(new_a, new_r)
    assert cow_a == cow_r
    same_state(a, r, [(ids_a[h], ids_r[h]) for h in wl.batch])
    if name == "shared_prefix_cow":
        assert len(cow_r) == 1                 # exactly the diverging sequence copies
        prefix = r.block_table(ids_r[0])[:128]
        # 255 sequences still hold all 128 prefix blocks; the diverging one swapped its last
        assert all(r.refcount[b] == 256 for b in prefix[:127])
        assert r.refcount[prefix[127]] == 255


def test_out_of_blocks_atomic_and_errors():
    pa = ensure_library()
    a = pa.BlockAllocator(4, 16)
    s = a.create()
    a.append(s, 60)
    before = (a.free_list(), a.block_table(s), a.length(s))
    with pytest.raises(pa.OutOfBlocks):
        a.append(s, 10)
    assert (a.free_list(), a.block_table(s), a.length(s)) == before
    with pytest.raises(pa.PagedAttnError):
        a.fork(s, 61)
    with pytest.raises(pa.PagedAttnError):
        a.append(99, 1)
    with pytest.raises(pa.PagedAttnError):
        pa.BlockAllocator(3, 16, [0, 0, 1])
    # a copy-on-write with no room for the pair is refused without changes
    c = a.fork(s, 60)
    a.free_seq(s)
    s2 = a.create()
    a.append(s2, 0)
    a2 = pa.BlockAllocator(8, 16)
    p = a2.create()
    a2.append(p, 20)
    ch = a2.fork(p, 20)
    before = (a2.free_list(), a2.block_table(ch), a2.refcount(1))
    with pytest.raises(pa.PagedAttnError):
        a2.append(ch, 1, cow_cap=0)
    assert (a2.free_list(), a2.block_table(ch), a2.refcount(1)) == before
    slots, pairs = a2.append(ch, 1)
    assert pairs == [(1, 2)]


def same_prefix_state(lib_a, ref):
    assert lib_a.prefix_stats() == ref.prefix_stats()


@pytest.mark.parametrize("seed", range(10))
def test_random_prefix_traces_bit_exact(seed):
    """Lookups, registrations, appends, forks and frees over a few shared prompts
    drawn from a small vocabulary, so that hits, misses, evictions and in-place
    writes into registered blocks all occur."""
    pa = ensure_library()
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(12, 40))
    B = 16
    order = rng.permutation(nb)
    a = pa.BlockAllocator(nb, B, order)
    r = oracle.RefAllocator(nb, B, order)
    prompts = [rng.integers(0, 20, size=int(rng.integers(1, 90))).tolist() for _ in range(4)]
    live = []          # (lib id, ref id, planned tokens; the first r.length(ref id) are stored)
    for step in range(400):
        op = int(rng.integers(0, 8))
        if op == 0 or not live:
            toks = prompts[int(rng.integers(0, 4))] + rng.integers(0, 20, size=int(rng.integers(0, 30))).tolist()
            sl, cl = a.prefix_lookup(toks)
            sr, cr = r.prefix_lookup(toks)
            assert cl == cr
            live.append((sl, sr, toks))
        elif op == 1:
            sl, sr, toks = live[int(rng.integers(0, len(live)))]
            k = int(rng.integers(0, r.length(sr) + 1))
            live.append((a.fork(sl, k), r.fork(sr, k), list(toks[:k])))
        elif op in (2, 3):
            i = int(rng.integers(0, len(live)))
            sl, sr, toks = live[i]
            n = int(rng.integers(0, 40))
            try:
                want = r.append(sr, n)
            except oracle.OutOfBlocks:
                with pytest.raises(pa.OutOfBlocks):
                    a.append(sl, n)
            else:
                slots, pairs = a.append(sl, n)
                assert slots.tolist() == want[0] and pairs == want[1]
                short = r.length(sr) - len(toks)
                if short > 0:
                    toks.extend(rng.integers(0, 20, size=short).tolist())
        elif op in (4, 5):
            sl, sr, toks = live[int(rng.integers(0, len(live)))]
            k = int(rng.integers(0, r.length(sr) + 1))
            a.prefix_register(sl, toks, k)
            r.prefix_register(sr, toks, k)
        else:
            sl, sr, _ = live.pop(int(rng.integers(0, len(live))))
            a.free_seq(sl)
            r.free_seq(sr)
        same_state(a, r, [(x[0], x[1]) for x in live])
        same_prefix_state(a, r)
    st = r.prefix_stats()
    assert st["lookups"] > 0 and st["hit_blocks"] > 0 and st["evictions"] > 0


def test_prefix_errors():
    pa = ensure_library()
    a = pa.BlockAllocator(4, 16)
    s = a.create()
    a.append(s, 20)
    with pytest.raises(pa.PagedAttnError):
        a.prefix_register(s, list(range(21)))         # more tokens than the sequence holds
    with pytest.raises(pa.PagedAttnError):
        a.prefix_register(7, list(range(4)))          # unknown sequence
    with pytest.raises(pa.PagedAttnError):
        a.prefix_lookup([1, 2, 3], -1)
    assert a.prefix_lookup([]) == (1, 0)


def _lcp(a, b):
    k = 0
    while k < min(len(a), len(b)) and a[k] == b[k]:
        k += 1
    return k


@pytest.mark.parametrize("seed", range(6))
def test_shared_blocks_is_the_common_table_prefix(seed):
    """pa_alloc_shared_blocks = the length of the common prefix of consecutive block tables (computed
    here from the tables alone), on random fork/append/free traces."""
    pa = ensure_library()
    rng = np.random.default_rng(300 + seed)
    nb = 200
    a = pa.BlockAllocator(nb, 16, rng.permutation(nb))
    live = [a.create()]
    a.append(live[0], int(rng.integers(1, 200)))
    for _ in range(120):
        op = int(rng.integers(0, 4))
        try:
            if op == 0:
                p = live[int(rng.integers(0, len(live)))]
                live.append(a.fork(p, int(rng.integers(0, a.length(p) + 1))))
            elif op in (1, 2):
                a.append(live[int(rng.integers(0, len(live)))], int(rng.integers(0, 30)))
            elif len(live) > 1:
                a.free_seq(live.pop(int(rng.integers(0, len(live)))))
        except pa.OutOfBlocks:
            pass
        order = [live[k] for k in rng.permutation(len(live))]
        got = a.shared_blocks(order)
        tabs = [a.block_table(s) for s in order]
        assert list(got) == [0] + [_lcp(x, y) for x, y in zip(tabs, tabs[1:])]
    with pytest.raises(pa.PagedAttnError):
        a.shared_blocks([10 ** 6])
