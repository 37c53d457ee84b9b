"""Pins for the fp8 cache format of the oracle (oracle/quant.py).

Pages: [SLAVA] section "Gemeinsame Nutzung erfordert mehr als
Speicherzuweisung" (cache quantisation as a remedy; compare at the same cache
precision) and [AIU] "L'avenir de PagedAttention et vLLM" (paged K/V combined
with quantisation).  The element format is the E4M3 (FN) encoding of the OCP
8-bit floating point specification; its published values pin the decoder,
brute force over all codes pins the rounding, closed forms pin the scale
choice, and an independent row-by-row reconstruction pins the pool layout.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from oracle.quant import DECODE_TABLE

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_decode_published_values():
    # OCP 8-bit floating point specification, E4M3: bias 7, max normal 448,
    # min normal 2^-6, min subnormal 2^-9, S.1111.111 is NaN, no infinities.
    assert oracle.decode_e4m3(0x00) == 0.0
    assert math.copysign(1.0, oracle.decode_e4m3(0x80)) == -1.0
    assert oracle.decode_e4m3(0x01) == 2.0 ** -9
    assert oracle.decode_e4m3(0x07) == 7 * 2.0 ** -9
    assert oracle.decode_e4m3(0x08) == 2.0 ** -6
    assert oracle.decode_e4m3(0x38) == 1.0
    assert oracle.decode_e4m3(0xB8) == -1.0
    assert oracle.decode_e4m3(0x7E) == 448.0
    assert oracle.decode_e4m3(0xFE) == -448.0
    assert oracle.decode_e4m3(0x77) == 240.0        # 1.875 * 2^7
    assert math.isnan(oracle.decode_e4m3(0x7F)) and math.isnan(oracle.decode_e4m3(0xFF))
    vals = sorted(DECODE_TABLE[c] for c in FINITE if c < 0x80)
    assert len(set(vals)) == 127 and vals[0] == 0.0 and vals[-1] == 448.0


def test_encode_round_trips_every_code():
    codes = np.array(FINITE, dtype=np.uint8)
    got = oracle.encode_e4m3(DECODE_TABLE[codes])
    assert np.array_equal(got, codes)


def _brute(y):
    """Nearest finite code by exhaustive search; ties to the even mantissa."""
    best = None
    for c in FINITE:
        if (c & 0x80) != (0x80 if math.copysign(1.0, y) < 0 else 0):
            continue
        d = abs(DECODE_TABLE[c] - y)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c)
    return best[1]


def test_encode_is_nearest_ties_to_even_by_brute_force():
    rng = np.random.default_rng(0)
    pos = np.array(sorted(DECODE_TABLE[c] for c in FINITE if c < 0x80))
    mids = (pos[1:] + pos[:-1]) / 2                     # every tie between neighbours
    rand = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 3000))
    ys = np.concatenate([mids, rand, [2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10, 448.0]])
    ys = np.concatenate([ys, -ys])
    got = oracle.encode_e4m3(ys)
    for y, c in zip(ys, got):
        assert c == _brute(float(y)), (y, hex(c))


def test_specific_ties():
    assert oracle.encode_e4m3([1 + 1 / 16])[0] == 0x38           # 1.0 (even) over 1.125
    assert oracle.encode_e4m3([1 + 3 / 16])[0] == 0x3A           # 1.25 (even) over 1.125
    assert oracle.encode_e4m3([2.0 ** -10])[0] == 0x00           # half the smallest subnormal -> 0
    assert oracle.encode_e4m3([3 * 2.0 ** -10])[0] == 0x02       # between 1 and 2 steps -> 2
    assert oracle.encode_e4m3([15 * 2.0 ** -10])[0] == 0x08      # 7.5 steps -> 8 = smallest normal
    with pytest.raises(ValueError):
        oracle.encode_e4m3([448.5])


def test_row_exponent_closed_forms():
    assert list(oracle.row_exponent([448.0, 449.0, 1.0, 1.75, 1.76, 0.0])) == [0, 1, -8, -8, -7, 0]
    assert oracle.row_exponent([2.0 ** -140])[0] == -126         # clamped
    rng = np.random.default_rng(1)
    amax = np.exp(rng.uniform(np.log(2.0 ** -110), np.log(2.0 ** 120), 5000))
    e = oracle.row_exponent(amax)
    assert np.all(amax <= np.ldexp(448.0, e))
    assert np.all(amax > np.ldexp(448.0, e - 1))                 # smallest such e


def test_non_finite_elements():
    """NaN and infinities are stored as the NaN code with their sign; the scale comes from the finite
    elements.  Row [NaN, +inf, -inf, 1, -3]: amax 3 -> e = -7 (448 * 2^-8 = 1.75 < 3 <= 3.5 = 448 * 2^-7),
    so 1 * 2^7 = 128 -> 0x70 and -3 * 2^7 = -384 = -1.5 * 2^8 -> 0xFC; -NaN (sign set) -> 0xFF."""
    row = np.array([[np.nan, np.inf, -np.inf, 1.0, -3.0, -np.nan]])
    codes, exps = oracle.quantize_rows(row)
    assert list(codes[0]) == [0x7F, 0x7F, 0xFF, 0x70, 0xFC, 0xFF]
    assert list(exps) == [127 - 7]
    back = oracle.dequantize_rows(codes, exps)[0]
    assert np.isnan(back[:3]).all() and np.isnan(back[5]) and list(back[3:5]) == [1.0, -3.0]
    # a row with no finite element takes e = 0
    codes, exps = oracle.quantize_rows(np.array([[np.inf, np.nan]]))
    assert list(codes[0]) == [0x7F, 0x7F] and list(exps) == [127]


def test_quantisation_error_bound():
    """Relative error <= 2^-4 in the normal range (half a 3-bit ulp), absolute <= 2^-10 * 2^e below it."""
    rng = np.random.default_rng(2)
    x = workloads.bf16_bits(rng.standard_normal((300, 128)).astype(np.float32) * np.float32(7.0))
    xf = oracle.to_f64(x, "bf16")
    codes, exps = oracle.quantize_rows(xf)
    back = oracle.dequantize_rows(codes, exps)
    scale = np.ldexp(1.0, exps.astype(np.int64) - 127)[:, None]
    normal = np.abs(xf) >= scale * 2.0 ** -6
    err = np.abs(back - xf)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(xf[normal]))
    assert np.all(err[~normal] <= (scale * 2.0 ** -10 * np.ones_like(xf))[~normal])
    # every row uses its range: its largest magnitude, in (224, 448] before rounding, stays in [224, 448]
    top = np.max(np.abs(back / scale), axis=1)
    assert np.all((top >= 224.0) & (top <= 448.0))


def test_write_layout_against_row_by_row_reconstruction():
    rng = np.random.default_rng(3)
    NB, Hkv, D, B = 7, 2, 64, 16
    kp, vp = oracle.fp8_pool(NB, Hkv, D), oracle.fp8_pool(NB, Hkv, D)
    T = 20
    k = oracle.to_f64(workloads.bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32)), "bf16")
    v = oracle.to_f64(workloads.bf16_bits(rng.standard_normal((T, Hkv, D)).astype(np.float32)), "bf16")
    slots = rng.permutation(NB * B)[:T]
    slots[4] = -1                                   # padding token: skipped
    oracle.ref_write_kv_fp8(kp, vp, k, v, slots, B)
    touched = np.zeros(kp.flat.shape, dtype=bool)
    n = NB * Hkv
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, row = s // B, s % B
        for h in range(Hkv):
            kc, ke = oracle.quantize_rows(k[t, h][None])
            vc, ve = oracle.quantize_rows(v[t, h][None])
            tile = (blk * Hkv + h) * B * D                           # code plane: tiles of B*D bytes
            for d in range(D):
                assert kp.flat[tile + row * D + d] == kc[0, d]       # K row-major
                assert vp.flat[tile + d * B + row] == vc[0, d]       # V transposed
                touched[tile + row * D + d] = True
            ex = n * B * D + (blk * Hkv + h) * B + row               # exponent plane after the codes
            assert kp.flat[ex] == ke[0] and vp.flat[ex] == ve[0]
            touched[ex] = True
    assert np.all(kp.flat[~touched] == 0xFF)                         # nothing else written
    # gathering through a table returns each token's own dequantised row
    table = list(range(NB))
    Kg = oracle.gather_logical_fp8(kp, table, NB * B, B, "k")
    Vg = oracle.gather_logical_fp8(vp, table, NB * B, B, "v")
    for t, s in enumerate(slots):
        if s >= 0:
            kc, ke = oracle.quantize_rows(k[t])
            vc, ve = oracle.quantize_rows(v[t])
            assert np.array_equal(Kg[s], oracle.dequantize_rows(kc, ke))
            assert np.array_equal(Vg[s], oracle.dequantize_rows(vc, ve))


def test_fp8_attention_is_attention_on_the_dequantised_values():
    """The fp8 route of ref_paged_attention equals the fp32 route fed the dequantised K/V."""
    rng = np.random.default_rng(4)
    NB, Hkv, Hq, D, B = 9, 2, 4, 64, 16
    kp, vp = oracle.fp8_pool(NB, Hkv, D), oracle.fp8_pool(NB, Hkv, D)
    L = np.array([37, 5, 60])
    n = np.array([1, 5, 3])
    tables = [[3, 0, 7], [5], [1, 8, 2, 6]]
    for i in range(3):
        slots = [tables[i][t // B] * B + t % B for t in range(L[i])]
        k = oracle.to_f64(workloads.bf16_bits(rng.standard_normal((L[i], Hkv, D)).astype(np.float32)), "bf16")
        v = oracle.to_f64(workloads.bf16_bits(rng.standard_normal((L[i], Hkv, D)).astype(np.float32)), "bf16")
        oracle.ref_write_kv_fp8(kp, vp, k, v, slots, B)
    q = workloads.bf16_bits(rng.standard_normal((int(n.sum()), Hq, D)).astype(np.float32))
    qsl = np.concatenate([[0], np.cumsum(n)])
    out8 = oracle.ref_paged_attention(q, kp, vp, tables, L, qsl, L - n, 0.125, True, B, "fp8")
    # the same values as an fp32 pool (dequantised values of this data fit fp32 exactly)
    kf = np.zeros((NB, Hkv, B, D), np.float32)
    vf = np.zeros_like(kf)
    for i in range(3):
        Kg = oracle.gather_logical_fp8(kp, tables[i], L[i], B, "k")
        Vg = oracle.gather_logical_fp8(vp, tables[i], L[i], B, "v")
        for t in range(L[i]):
            kf[tables[i][t // B], :, t % B] = Kg[t]
            vf[tables[i][t // B], :, t % B] = Vg[t]
    qf = oracle.to_f64(q, "bf16").astype(np.float32)
    out32 = oracle.ref_paged_attention(qf, kf, vf, tables, L, qsl, L - n, 0.125, True, B, "f32")
    assert np.array_equal(out8, out32)
