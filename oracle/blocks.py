"""Block counts and unused-slot accounting (closed forms).

[SLAVA] section "Ungenutzten Platz in Blöcken berechnen": with fixed-size
blocks of B token slots, a sequence of n tokens occupies the fewest blocks that
hold n slots, and only its last block can be partly empty; the empty share
shrinks as the sequence grows.  The section works one case through: 35 tokens
with B = 16 take three blocks (48 slots), leaving 13 of them empty, about 27%.
"""


def blocks_needed(n_tokens, block_size):
    """Number of B-slot blocks a sequence of ``n_tokens`` occupies: ceil(n / B)."""
    if n_tokens < 0 or block_size <= 0:
        raise ValueError("n_tokens must be >= 0 and block_size > 0")
    return -(-n_tokens // block_size)


def unused_slots(n_tokens, block_size):
    """Empty slots left in the last block: B * ceil(n / B) - n, always in [0, B-1]."""
    return blocks_needed(n_tokens, block_size) * block_size - n_tokens


def unused_fraction(n_tokens, block_size):
    """Empty share of the slots allocated to one sequence (0 for an empty sequence)."""
    slots = blocks_needed(n_tokens, block_size) * block_size
    return 0.0 if slots == 0 else unused_slots(n_tokens, block_size) / slots
