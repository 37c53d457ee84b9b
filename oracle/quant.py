"""Quantised (fp8) K/V cache: the cache format and its exact decoding (test infrastructure only).

What the pages fix: [SLAVA] section "Gemeinsame Nutzung erfordert mehr als
Speicherzuweisung" names cache quantisation as a remedy when the raw K/V data
does not fit, and asks that comparisons use the same cache precision; [AIU]
section "L'avenir de PagedAttention et vLLM" expects paged K/V to be combined
with quantisation.  They fix no format.  Readings taken here:

  * Element format: 8-bit floating point "E4M3" in the OCP 8-bit floating
    point specification (the FN variant: 1 sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the codes
    0x7f and 0xff are NaN; no infinities; largest finite value 448).
  * Scale: one power of two per (token, KV head) row of head_dim values,
    stored as an 8-bit biased exponent (the OCP "E8M0" scale format: code c
    means 2^(c - 127)).  The exponent e is the smallest integer with
    max|x| <= 448 * 2^e, limited to [-126, 127]; a row of zeros takes e = 0.
    With a power-of-two scale, x * 2^-e is exact, so the only rounding is the
    one to E4M3.
  * Rounding: to the nearest E4M3 value, ties to an even mantissa (the
    usual IEEE rule).  Because |x * 2^-e| <= 448 nothing saturates.
  * Non-finite inputs: E4M3 FN has no infinity, so a NaN or an infinite
    element is stored as the NaN code (0x7f, with the element's sign bit:
    0xff when it is set), and the row's scale is taken from its finite
    elements only (a row with none takes e = 0).
  * Dequantised value: decode(code) * 2^e, exact in float64.
  * Pool layout: num_blocks * num_kv_heads * (16 * D + 16) bytes in two
    planes.  First the codes, ``[num_blocks][num_kv_heads][16 * D]``: per
    (block, KV head) tile the K codes row-major (byte row * D + d), the V codes
    transposed (byte d * 16 + row).  Then the exponents,
    ``[num_blocks][num_kv_heads][16]``, one byte per row.
"""

import math

import numpy as np

E4M3_MAX = 448.0
EXP_MIN, EXP_MAX = -126, 127
SCALE_BIAS = 127


def decode_e4m3(code):
    """Value of one E4M3 (FN) code, as float64 (NaN for 0x7f / 0xff)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE_TABLE = np.array([decode_e4m3(c) for c in range(256)], dtype=np.float64)


def encode_e4m3(y):
    """E4M3 codes nearest to y (array, |y| <= 448), ties to an even mantissa; the sign of zero is kept.

    Subnormal range (|y| < 2^-6): the code is the number of 2^-9 steps, rounded
    (8 steps give the smallest normal, code 0x08).  Normal range: y = f * 2^E
    with f in [1, 2); the mantissa is (f - 1) * 8 rounded, a carry to 8 moving
    to the next binade.  np.rint rounds half to even.
    """
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.abs(y) <= E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.abs(y)
    sub = a < 2.0 ** -6
    q_sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    m, E = np.frexp(np.where(sub, 1.0, a))          # a = m * 2^E, m in [0.5, 1)
    E = E.astype(np.int64) - 1                      # a = (2m) * 2^E
    q = np.rint((2.0 * m - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    q = np.where(carry, 0, q)
    E = E + carry
    code = np.where(sub, q_sub, ((E + 7) << 3) | q)
    return (sign | code).astype(np.uint8)


def row_exponent(amax):
    """Smallest e in [-126, 127] with amax <= 448 * 2^e, per element (0 where amax = 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    e = np.where(safe <= np.ldexp(E4M3_MAX, e - 1), e - 1, e)     # log2 rounding, either way
    e = np.where(safe > np.ldexp(E4M3_MAX, e), e + 1, e)
    return np.clip(np.where(amax > 0, e, 0), EXP_MIN, EXP_MAX)


def quantize_rows(x):
    """Rows of values (last axis = one row) -> (uint8 codes, uint8 biased exponent per row).

    NaN and infinite elements become the NaN code with their sign bit; the
    scale ignores them.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    e = row_exponent(np.max(np.where(finite, np.abs(x), 0.0), axis=-1))
    codes = encode_e4m3(np.ldexp(np.where(finite, x, 0.0), -e[..., None]))
    nan_codes = np.where(np.signbit(x), 0xFF, 0x7F).astype(np.uint8)
    return np.where(finite, codes, nan_codes), (e + SCALE_BIAS).astype(np.uint8)


def dequantize_rows(codes, exp_codes):
    e = np.asarray(exp_codes, dtype=np.int64) - SCALE_BIAS
    return np.ldexp(DECODE_TABLE[np.asarray(codes, dtype=np.int64)], e[..., None])


class Fp8Pool:
    """One quantised pool: ``flat`` holds the bytes; ``codes`` and ``exps`` are views of its two planes.

    Indexing by block reads or replaces that block's codes and exponents
    together, so a whole-block copy is ``pool[dst] = pool[src]``.
    """

    def __init__(self, num_blocks, num_kv_heads, head_dim, block_size=16, fill=0xFF):
        n = num_blocks * num_kv_heads
        self.flat = np.full(n * (block_size * head_dim + block_size), fill, dtype=np.uint8)
        self.codes = self.flat[:n * block_size * head_dim].reshape(num_blocks, num_kv_heads, block_size * head_dim)
        self.exps = self.flat[n * block_size * head_dim:].reshape(num_blocks, num_kv_heads, block_size)
        self.num_blocks, self.num_kv_heads, self.head_dim, self.block_size = (num_blocks, num_kv_heads,
                                                                              head_dim, block_size)

    def __getitem__(self, blk):
        return self.codes[blk].copy(), self.exps[blk].copy()

    def __setitem__(self, blk, value):
        self.codes[blk], self.exps[blk] = value


def fp8_pool(num_blocks, num_kv_heads, head_dim, block_size=16, fill=0xFF):
    """An empty pool (every byte ``fill``; 0xff is a NaN code and a NaN scale)."""
    return Fp8Pool(num_blocks, num_kv_heads, head_dim, block_size, fill)


def _code_index(kind, rows, D, block_size):
    """Byte index of each (row, d) code inside a tile: ``[len(rows)][D]``."""
    d = np.arange(D)[None, :]
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    return rows * D + d if kind == "k" else d * block_size + rows


def ref_write_kv_fp8(k_pool, v_pool, k, v, slot_mapping, block_size):
    """Quantise and store token t's K/V rows (all KV heads) at slot ``slot_mapping[t]``.

    k, v: float64-exact values ``[T][Hkv][D]`` (e.g. widened bf16).  A
    negative slot is skipped; two tokens may not name the same slot.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    live = slots[keep]
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slots in one write")
    if live.size and live.max() // block_size >= k_pool.num_blocks:
        raise ValueError("slot beyond the pool")
    blk, row = live // block_size, live % block_size
    hkv, D = np.asarray(k).shape[1], np.asarray(k).shape[2]
    heads = np.arange(hkv)[None, :, None]
    for pool, x, kind in ((k_pool, k, "k"), (v_pool, v, "v")):
        codes, exps = quantize_rows(np.asarray(x, dtype=np.float64)[keep])      # [n][Hkv][D], [n][Hkv]
        idx = _code_index(kind, row, D, block_size)[:, None, :]                 # [n][1][D]
        pool.codes[blk[:, None, None], heads, idx] = codes
        pool.exps[blk[:, None], np.arange(hkv)[None, :], row[:, None]] = exps


def gather_logical_fp8(pool, table, length, block_size, kind):
    """Dequantised rows 0..length-1 of one sequence: float64 ``[length][Hkv][D]``.

    ``kind`` is "k" (row-major codes) or "v" (transposed codes).
    """
    hkv, D = pool.num_kv_heads, pool.head_dim
    t = np.arange(length)
    blk = np.asarray(table, dtype=np.int64)[t // block_size]
    row = t % block_size
    idx = _code_index(kind, row, D, block_size)[:, None, :]
    codes = pool.codes[blk[:, None, None], np.arange(hkv)[None, :, None], idx]     # [L][Hkv][D]
    exps = pool.exps[blk[:, None], np.arange(hkv)[None, :], row[:, None]]
    return dequantize_rows(codes, exps)
