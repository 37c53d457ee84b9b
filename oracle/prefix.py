"""Chained block hashes for prefix caching (test infrastructure; the product never imports this).

[ART] paragraph on prefix caching: blocks of tokens are hashed and kept in
memory; a new request that starts with the same tokens finds the matches and
reuses the stored K/V instead of recomputing them.

The pages name no hash function.  Reading taken here: FNV-1a 64,
a published definition -- start from the offset basis 0xcbf29ce484222325 and,
for each byte, xor it in and multiply by the prime 0x100000001b3 modulo 2^64.
Block b of a token sequence hashes the 8 little-endian bytes of the previous
block's hash (the offset basis before block 0) followed by the 4 little-endian
bytes of each of its token ids, so a block's hash names the whole prefix that
ends with it.
"""

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
_MASK = (1 << 64) - 1


def fnv1a64(data, h=FNV_OFFSET):
    """FNV-1a 64 of ``data`` (bytes), continuing from state ``h``."""
    for byte in bytes(data):
        h ^= byte
        h = (h * FNV_PRIME) & _MASK
    return h


def block_hash(parent, tokens):
    """Hash of a full block with these token ids whose predecessor hashed to ``parent``."""
    data = int(parent).to_bytes(8, "little") + b"".join(
        (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    return fnv1a64(data)


def chain(tokens, block_size=16):
    """Hashes of the full blocks of ``tokens``, in order."""
    out, parent = [], FNV_OFFSET
    for b in range(len(tokens) // block_size):
        parent = block_hash(parent, tokens[b * block_size:(b + 1) * block_size])
        out.append(parent)
    return out
