"""Pins for the oracle's widening of stored element formats to float64.

The workloads store K, V and q as IEEE fp32 or as bfloat16 bit patterns; the
oracle widens both to float64 before any arithmetic.  These pins check the
widening against things other than the oracle's own code:

  * torch's own bfloat16 -> float64 conversion, over all 65,536 bit patterns
    (NaN payloads compared by ``isnan`` only);
  * values fixed by the bfloat16 format itself (1 sign bit, 8 exponent bits
    with bias 127, 7 fraction bits): 0x3F80 = 1, 0xC000 = -2, 0x0001 = 2^-133
    (smallest subnormal), 0x0080 = 2^-126 (smallest normal), 0x7F7F =
    (2 - 2^-7) * 2^127 (largest finite), 0x7F80 = +inf, 0xFF80 = -inf,
    0x8000 = -0;
  * fp32: NumPy's own float32 -> float64 cast on random values and on the
    fp32 edge values.
"""

import numpy as np
import torch

import oracle


def torch_bf16_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64 through torch's own dtype conversion."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def test_bf16_all_bit_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits, "bf16")
    want = torch_bf16_to_f64(bits)
    assert got.dtype == np.float64 and got.shape == bits.shape
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127          # exponent all ones, fraction non-zero, both signs
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_bf16_printed_patterns():
    cases = {
        0x3F80: 1.0,
        0xC000: -2.0,
        0x0001: 2.0 ** -133,
        0x0080: 2.0 ** -126,
        0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
        0x3FC0: 1.5,
        0x4049: 3.140625,                 # 1.5703125 * 2
        0x7F80: np.inf,
        0xFF80: -np.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle.to_f64(bits, "bf16")
    assert list(got) == list(cases.values())
    z = oracle.to_f64(np.array([0x0000, 0x8000], dtype=np.uint16), "bf16")
    assert z[0] == 0.0 and not np.signbit(z[0])
    assert z[1] == 0.0 and np.signbit(z[1])
    assert np.isnan(oracle.to_f64(np.array([0x7FC0, 0xFFC1], dtype=np.uint16), "bf16")).all()


def test_bf16_shape_is_kept():
    bits = np.random.default_rng(3).integers(0, 1 << 16, size=(3, 5, 7), dtype=np.uint16)
    got = oracle.to_f64(bits, "bf16")
    assert got.shape == (3, 5, 7)
    assert np.array_equal(got, torch_bf16_to_f64(bits.reshape(-1)).reshape(3, 5, 7), equal_nan=True)


def test_f32_widening():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(1000).astype(np.float32)
    edge = np.array([0.0, -0.0, np.finfo(np.float32).max, np.finfo(np.float32).tiny,
                     np.float32(1e-45), np.inf, -np.inf], dtype=np.float32)
    for arr in (x, edge):
        got = oracle.to_f64(arr, "f32")
        assert got.dtype == np.float64
        assert [float(a) for a in arr] == list(got)


def test_wrong_storage_is_refused():
    import pytest
    with pytest.raises(TypeError):
        oracle.to_f64(np.zeros(3, dtype=np.float32), "bf16")
    with pytest.raises(TypeError):
        oracle.to_f64(np.zeros(3, dtype=np.uint16), "f32")
    with pytest.raises(ValueError):
        oracle.to_f64(np.zeros(3, dtype=np.uint16), "f16")
