"""Random super-batches against the oracle: every dispatcher route on mixed batches.

"Внутреннее устройство vLLM" (artificials.ru), forward-pass and chunked-prefill
paragraphs: one forward pass takes decode tokens and prefill chunks together,
each sequence attending over its own cached tokens and its new ones.  Each
seed draws a batch of 1..24 sequences mixing single-token decode rows, 2..16
token rows (speculative verification) and 17..160 token chunks, on cached
lengths that include 0, block boundaries and arbitrary values, with a random
head grouping, and runs it through the library (C++ allocator, device pools,
pa_write_kv_forward) and through the oracle: slots, tables and both whole
pools bit for bit, every output row within the stated tolerance.  The cache
families rotate over bf16 head_dim 128, bf16 head_dim 64, fp32 and fp8 (bf16
rows on E4M3 codes); the bf16 and fp32 batches also run with the single-token
rows kept apart from the multi-token kernel (PA_VERIFY=split) and with the
multi-token rows sent to the chunked-prefill kernel (PA_VERIFY=prefill).  A
second pass runs each batch with the chunked-prefill work-groups in both
orders (PA_PREFILL_ORDER=sequences / pieces).
"""

import numpy as np
import pytest

import workloads
from test_gpu_parity import _device_run, check_parity

pytestmark = pytest.mark.gpu

FAMILIES = [("bf16", 128, ""), ("bf16", 64, ""), ("f32", 128, ""), ("bf16", 128, "fp8")]


def random_batch(seed):
    rng = np.random.default_rng(9100 + seed)
    dtype, D, cache = FAMILIES[seed % len(FAMILIES)]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    S = int(rng.integers(1, 25))
    new, cached = [], []
    for _ in range(S):
        u = rng.random()
        new.append(1 if u < 0.4 else int(rng.integers(2, 17)) if u < 0.7 else int(rng.integers(17, 161)))
        v = rng.random()
        cached.append(0 if v < 0.15 else 16 * int(rng.integers(1, 60)) if v < 0.4 else int(rng.integers(1, 1200)))
    causal = bool(rng.random() >= 0.25)
    wl = workloads.independent(f"random_mixed_{seed}", 9200 + seed, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype,
                               cached=cached, new=new, pool_extra=3, causal=causal, cache_dtype=cache)
    return wl, f"{dtype}/D{D}/{cache or 'plain'}/G{G}/Hkv{Hkv}/S{S}/causal{int(causal)}"


@pytest.mark.parametrize("seed", range(24))
def test_random_mixed_batch(seed, monkeypatch):
    wl, what = random_batch(seed)
    routes = [None] if wl.cache == "fp8" else [None, "split", "prefill"]
    for route in routes:
        for key in ("PA_VERIFY", "PA_DECODE", "PA_CHECK"):
            monkeypatch.delenv(key, raising=False)
        if route is not None:
            monkeypatch.setenv("PA_VERIFY", route)
        print(f"[random-mixed] seed {seed}: {what}, route {route or 'default'}", flush=True)
        check_parity(wl)


@pytest.mark.parametrize("seed", range(24))
def test_prefill_work_group_orders(seed, monkeypatch):
    """The chunked-prefill work-groups ordered sequences-slowest
    (PA_PREFILL_ORDER=sequences) and pieces-slowest (=pieces): both meet the
    tolerance against the oracle, with bit-identical outputs (the same work
    items, handed to different work-groups).  Multi-token rows go to the
    prefill kernel (PA_VERIFY=prefill) except on fp8 pools."""
    wl, what = random_batch(seed)
    for key in ("PA_VERIFY", "PA_DECODE", "PA_CHECK", "PA_PREFILL_ORDER"):
        monkeypatch.delenv(key, raising=False)
    if wl.cache != "fp8":
        monkeypatch.setenv("PA_VERIFY", "prefill")
    monkeypatch.setenv("PA_PREFILL_ORDER", "sequences")
    print(f"[random-mixed] seed {seed}: {what}, prefill work-group orders", flush=True)
    seq, _ = check_parity(wl)
    monkeypatch.setenv("PA_PREFILL_ORDER", "pieces")
    pieces = _device_run(wl)
    assert np.array_equal(seq.out_f64(), pieces.out_f64())
