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

Readings taken where the pages are silent (each is listed in the design doc):
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
"""

from collections import deque

from .blocks import blocks_needed


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
            if p % B == 0:
                fresh = self.free.popleft()
                self.refcount[fresh] = 1
                table.append(fresh)
            elif j not in copied and self.refcount[table[j]] > 1:
                old = table[j]
                fresh = self.free.popleft()
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
