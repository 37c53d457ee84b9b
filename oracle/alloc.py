"""RefAllocator: block allocator with block tables, refcounts and copy-on-write.

What the pages fix:
  * [SLAVA] lead paragraph: a request's cache lives in separate fixed-size
    blocks; a block table maps the request's logical token positions to
    physical blocks.
  * [SLAVA] section "Ungenutzten Platz in Blöcken berechnen": blocks are added
    as a sequence grows and given back when the request ends; nothing is
    reserved up front; only the last block is partly filled.
  * [SLAVA] section "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung"
    and [AIU] "Questions fréquemment posées" (sharing question): several
    requests may point at the same physical block; a copy is made only when a
    branch diverges, so the shared state is never corrupted.
  * [ART] paragraph on paged attention: blocks of 16 tokens; running out of
    blocks is a signal for preemption.

Readings taken where the pages are silent:
  * The free list starts in a caller-given order (default 0..N-1).  Blocks are
    taken from its head; a block whose refcount drops to zero goes to its tail.
  * Sequence ids are 0, 1, 2, ... in creation order and are never reused.
  * ``fork(parent, k)`` gives the child the parent's first ceil(k/B) blocks
    (refcount + 1 each) and length k; k must not exceed the parent's length.
  * ``append(seq, n)`` handles positions p = len .. len+n-1 in order: at a block
    edge (p % B == 0) it takes a fresh block; otherwise, the first time it
    writes into a block whose refcount is above one, it copies that block
    (copy-on-write): takes a fresh block, records the pair (old, new), drops the
    old block's refcount by one and points the table entry at the new block.
    The slot of position p is ``table[p // B] * B + p % B``.
  * ``append`` is all-or-nothing: if the free list cannot cover every block it
    needs, it raises OutOfBlocks and changes nothing.
  * ``free(seq)`` drops the refcount of each of the sequence's blocks in table
    order, returning those that reach zero to the tail of the free list.

Prefix caching ([ART] paragraph on prefix caching: blocks of tokens are hashed
and kept; a request starting with the same tokens reuses them), readings:
  * Block hashes chain as in ``oracle.prefix``.  A registered block carries its
    hash, its parent's hash and its tokens; the cache maps a hash to at most
    one block; a lookup hits only if hash, parent hash and tokens all match.
  * ``prefix_register(seq, tokens, n)`` registers, in order, each full block
    of the first n tokens that is not registered yet, unless another block is
    already registered under its hash.
  * ``prefix_lookup(tokens, n)`` creates a sequence holding the longest run of
    hitting full blocks from the start, leaving at least one token uncached
    (b < (n - 1) // B); each hit block's refcount rises by one, and a hit
    block with refcount 0 leaves the free list.  Returns (seq, B * hits).
  * A registered block freed to refcount 0 stays registered at the free-list
    tail; handing it out again (append) unregisters it first (eviction).
  * An append that writes into a registered block in place (no copy due)
    unregisters it first (eviction): cached blocks are never overwritten.
"""

from collections import deque

from .blocks import blocks_needed
from .prefix import FNV_OFFSET, block_hash


class OutOfBlocks(Exception):
    """Raised when an append needs more free blocks than remain (no state change)."""


class RefAllocator:
    def __init__(self, num_blocks, block_size=16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq id -> list of physical block ids (logical order)
        self.lengths = {}  # seq id -> tokens stored
        self.next_id = 0
        self.reg = {}      # registered block -> (hash, parent hash, tokens)
        self.cache = {}    # hash -> registered block
        self.lookups = 0
        self.hit_blocks = 0
        self.evictions = 0

    def _unregister(self, b):
        if b in self.reg:   # eviction: the block is about to be written
            del self.cache[self.reg.pop(b)[0]]
            self.evictions += 1

    def _pop_free(self):
        b = self.free.popleft()
        self._unregister(b)
        return b

    # -- sequence lifetime -------------------------------------------------
    def create(self):
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent, share_tokens):
        if parent not in self.tables:
            raise KeyError(f"unknown sequence {parent}")
        if not 0 <= share_tokens <= self.lengths[parent]:
            raise ValueError("share_tokens must lie in [0, len(parent)]")
        shared = self.tables[parent][: blocks_needed(share_tokens, self.block_size)]
        for b in shared:
            self.refcount[b] += 1
        sid = self.create()
        self.tables[sid] = list(shared)
        self.lengths[sid] = share_tokens
        return sid

    def append(self, seq, n_tokens):
        """Grow ``seq`` by ``n_tokens``; return (slots, cow_pairs)."""
        if seq not in self.tables:
            raise KeyError(f"unknown sequence {seq}")
        if n_tokens < 0:
            raise ValueError("n_tokens must be >= 0")
        B = self.block_size
        table = self.tables[seq]
        start = self.lengths[seq]

        # Count the fresh blocks the append needs before touching any state.
        need = 0
        copied = set()
        for p in range(start, start + n_tokens):
            j = p // B
            if p % B == 0:
                need += 1
            elif j < len(table) and j not in copied and self.refcount[table[j]] > 1:
                need += 1
                copied.add(j)
        if need > len(self.free):
            raise OutOfBlocks(f"append of {n_tokens} needs {need} blocks, {len(self.free)} free")

        slots = []
        cow_pairs = []
        copied = set()
        for p in range(start, start + n_tokens):
            j = p // B
            if p % B != 0 and j not in copied and self.refcount[table[j]] == 1:
                self._unregister(table[j])   # written in place: leaves the cache
            if p % B == 0:
                fresh = self._pop_free()
                self.refcount[fresh] = 1
                table.append(fresh)
            elif j not in copied and self.refcount[table[j]] > 1:
                old = table[j]
                fresh = self._pop_free()
                self.refcount[fresh] = 1
                self.refcount[old] -= 1
                table[j] = fresh
                cow_pairs.append((old, fresh))
                copied.add(j)
            slots.append(table[j] * B + p % B)
        self.lengths[seq] = start + n_tokens
        return slots, cow_pairs

    def free_seq(self, seq):
        if seq not in self.tables:
            raise KeyError(f"unknown sequence {seq}")
        for b in self.tables.pop(seq):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lengths[seq]

    # -- prefix caching ----------------------------------------------------
    def prefix_register(self, seq, tokens, n_tokens=None):
        n = len(tokens) if n_tokens is None else n_tokens
        if seq not in self.tables:
            raise KeyError(f"unknown sequence {seq}")
        if not 0 <= n <= self.lengths[seq]:
            raise ValueError("n_tokens must lie in [0, len(seq)]")
        B = self.block_size
        parent = FNV_OFFSET
        for b in range(n // B):
            blk_tokens = tuple(int(t) for t in tokens[b * B:(b + 1) * B])
            h = block_hash(parent, blk_tokens)
            blk = self.tables[seq][b]
            if blk not in self.reg and h not in self.cache:
                self.reg[blk] = (h, parent, blk_tokens)
                self.cache[h] = blk
            parent = h

    def prefix_lookup(self, tokens, n_tokens=None):
        n = len(tokens) if n_tokens is None else n_tokens
        if n < 0:
            raise ValueError("n_tokens must be >= 0")
        B = self.block_size
        hits, parent = [], FNV_OFFSET
        for b in range(max(n - 1, 0) // B):
            blk_tokens = tuple(int(t) for t in tokens[b * B:(b + 1) * B])
            h = block_hash(parent, blk_tokens)
            blk = self.cache.get(h)
            if blk is None or self.reg[blk][1] != parent or self.reg[blk][2] != blk_tokens:
                break
            hits.append(blk)
            parent = h
        for blk in hits:
            if self.refcount[blk] == 0:
                self.free.remove(blk)
            self.refcount[blk] += 1
        sid = self.create()
        self.tables[sid] = hits
        self.lengths[sid] = len(hits) * B
        self.lookups += 1
        self.hit_blocks += len(hits)
        return sid, len(hits) * B

    def prefix_stats(self):
        return {
            "blocks_registered": len(self.reg),
            "registered_free": sum(1 for b in self.reg if self.refcount[b] == 0),
            "lookups": self.lookups,
            "hit_blocks": self.hit_blocks,
            "evictions": self.evictions,
        }

    # -- inspection --------------------------------------------------------
    def block_table(self, seq):
        return list(self.tables[seq])

    def length(self, seq):
        return self.lengths[seq]

    def stats(self):
        """Counts the pages suggest measuring ([SLAVA], sharing section)."""
        used = sum(1 for r in self.refcount if r > 0)
        return {
            "blocks_total": self.num_blocks,
            "blocks_free": len(self.free),
            "blocks_used": used,
            "blocks_shared": sum(1 for r in self.refcount if r > 1),
            "tokens_logical": sum(self.lengths.values()),
            "slots_logical": sum(len(t) for t in self.tables.values()) * self.block_size,
            "slots_physical": used * self.block_size,
        }
