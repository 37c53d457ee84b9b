"""Cache write through a slot mapping, and whole-block copies (oracle side).

Layout (a reading: [SLAVA] section "Ungenutzten Platz in Blöcken berechnen"
says block size and layout depend on the runtime): each of the K and V pools
is ``[num_blocks][num_kv_heads][block_size][head_dim]``.  Slot s names block
``s // block_size`` and row ``s % block_size`` inside it.

Both operations are plain copies of stored bits; no arithmetic on values.
"""

import numpy as np


def ref_write_kv(k_cache, v_cache, k, v, slot_mapping, block_size):
    """Store token t's K/V rows (all KV heads) at slot ``slot_mapping[t]``.

    [SLAVA] lead paragraph: positions reach physical blocks through the block
    table; the per-token slot is that mapping flattened.  A negative slot
    marks a padding token that is skipped.  Two tokens may not name the same
    slot in one call.  Arrays are modified in place: k/v are
    ``[T][Hkv][D]``, caches ``[NB][Hkv][B][D]``, in any one stored format.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    live = slots[keep]
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots in one write")
    num_slots = k_cache.shape[0] * block_size
    if live.size and live.max() >= num_slots:
        raise ValueError("slot beyond the pool")
    blocks = live // block_size
    rows = live % block_size
    k_cache[blocks, :, rows, :] = np.asarray(k)[keep]
    v_cache[blocks, :, rows, :] = np.asarray(v)[keep]


def ref_copy_blocks(k_cache, v_cache, pairs):
    """Copy whole blocks ``src -> dst`` (all heads, all rows) in list order.

    [SLAVA] section "Gemeinsame Nutzung erfordert mehr als Speicherzuweisung"
    and [AIU] sharing question: a shared block is copied before a diverging
    write, leaving the shared original untouched.
    """
    for src, dst in pairs:
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]
