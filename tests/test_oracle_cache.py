"""Pins for the oracle's cache write and block copy.

The write defines the mapping in [SLAVA]'s lead paragraph: after storing token
rows at their slots, reading the sequence back through its block table in
logical order returns exactly the rows written, and no other block changes.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import OracleRun, logical_rows, nan_pool


@pytest.mark.parametrize("name", ["decode_f32", "mixed_bf16", "shared_bf16"])
def test_roundtrip_through_block_tables(name):
    wl = workloads.mini(name)
    run = OracleRun(wl, compute_out=False)
    for i, (K, V) in enumerate(logical_rows(wl)):
        L = int(wl.seq_lens[i])
        assert len(K) == L
        gk = oracle.gather_logical(run.k_cache, run.tables[i], L, wl.block_size)
        gv = oracle.gather_logical(run.v_cache, run.tables[i], L, wl.block_size)
        assert np.array_equal(gk.view(np.uint8), K.view(np.uint8))
        assert np.array_equal(gv.view(np.uint8), V.view(np.uint8))


def test_untouched_blocks_unchanged_and_padding_skipped():
    rng = np.random.default_rng(3)
    B, Hkv, D = 16, 2, 8
    kc = rng.standard_normal((10, Hkv, B, D)).astype(np.float32)
    vc = rng.standard_normal((10, Hkv, B, D)).astype(np.float32)
    k0, v0 = kc.copy(), vc.copy()
    k = rng.standard_normal((4, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((4, Hkv, D)).astype(np.float32)
    slots = np.array([3 * B + 5, -1, 7 * B + 0, 7 * B + 15])
    oracle.ref_write_kv(kc, vc, k, v, slots, B)
    assert np.array_equal(kc[3, :, 5], k[0]) and np.array_equal(vc[7, :, 15], v[3])
    mask = np.ones(kc.shape[:3], dtype=bool)
    mask[3, :, 5] = mask[7, :, 0] = mask[7, :, 15] = False
    assert np.array_equal(kc[mask], k0[mask]) and np.array_equal(vc[mask], v0[mask])


def test_duplicate_slots_rejected():
    kc = np.zeros((2, 1, 16, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.ref_write_kv(kc, kc.copy(), np.ones((2, 1, 4), np.float32),
                            np.ones((2, 1, 4), np.float32), np.array([5, 5]), 16)


def test_copy_blocks_copies_whole_block_and_keeps_source():
    rng = np.random.default_rng(4)
    kc = rng.integers(0, 2**16, size=(6, 2, 16, 8), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(6, 2, 16, 8), dtype=np.uint16)
    k0, v0 = kc.copy(), vc.copy()
    oracle.ref_copy_blocks(kc, vc, [(1, 4), (2, 5)])
    assert np.array_equal(kc[4], k0[1]) and np.array_equal(vc[5], v0[2])
    for b in (0, 1, 2, 3):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])


def test_named_workload_sizes():
    # block counts of the five named workloads follow the closed form
    wl = workloads.tiny_decode()
    run = OracleRun(wl, compute_out=False)
    assert [len(t) for t in run.tables] == [3, 1, 1, 4]
    st = run.alloc.stats()
    assert st["blocks_used"] == 9
    assert st["slots_logical"] - st["tokens_logical"] == 42
