"""Every shape pa_forward advertises, against the oracle.

The header promises dtype {f32, bf16} x head_dim {64, 128} x query heads per
KV head {1, 2, 4, 8}.  Each combination runs a batch of single-token decode
rows and a mixed batch (decode rows, a few multi-token rows and prefill
chunks), with ragged lengths: empty cache, exactly one block, one block plus
one token, several tiles with a partial last block.  bf16 with head_dim 128
also runs with the vector decode kernel forced (PA_DECODE=valu).  The
attention definition followed is the one in "PagedAttention et vLLM"
(aiunderstanding.org), section "Plongée profonde", and "Внутреннее
устройство vLLM" (artificials.ru), forward-pass paragraph.
"""

import pytest

import workloads
from helpers import ensure_library
from test_gpu_parity import check_parity

pytestmark = pytest.mark.gpu

HEADS = {1: (4, 4), 2: (8, 4), 4: (8, 2), 8: (16, 2)}     # G -> (Hq, Hkv)
SHAPES = [(dt, D, G) for dt in ("f32", "bf16") for D in (64, 128) for G in (1, 2, 4, 8)]

DECODE_CACHED = [0, 15, 16, 47, 300, 1025, 2]
MIXED_CACHED = [0, 15, 16, 47, 300, 9, 130]
MIXED_NEW = [1, 3, 1, 17, 40, 70, 2]


def _batches(dtype, D, G, seed):
    Hq, Hkv = HEADS[G]
    dec = workloads.independent(f"shape_{dtype}_d{D}_g{G}_decode", seed, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                                cached=DECODE_CACHED, new=[1] * len(DECODE_CACHED), pool_extra=3)
    mix = workloads.independent(f"shape_{dtype}_d{D}_g{G}_mixed", seed + 1, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                                cached=MIXED_CACHED, new=MIXED_NEW, pool_extra=3)
    return dec, mix


@pytest.mark.parametrize("dtype,D,G", SHAPES, ids=[f"{d}-D{h}-G{g}" for d, h, g in SHAPES])
def test_every_advertised_shape(dtype, D, G, monkeypatch):
    for k in ("PA_DECODE", "PA_VERIFY", "PA_SPLIT", "PA_PREFILL_SPLIT"):
        monkeypatch.delenv(k, raising=False)
    ensure_library()
    dec, mix = _batches(dtype, D, G, 200 + 10 * G + D // 64 + (0 if dtype == "f32" else 5))
    check_parity(dec)
    check_parity(mix)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_vector_decode_forced_bf16_d128(G, monkeypatch):
    """PA_DECODE=valu: bf16 head_dim 128 single-token rows on the vector kernel (partitioned, merged),
    alone and beside multi-token rows and chunks (PA_VERIFY=split keeps the single-token rows there)."""
    ensure_library()
    monkeypatch.setenv("PA_DECODE", "valu")
    monkeypatch.setenv("PA_VERIFY", "split")
    dec, mix = _batches("bf16", 128, G, 300 + G)
    check_parity(dec, pools=False)
    check_parity(mix, pools=False)
    monkeypatch.setenv("PA_SPLIT", "64")             # many partitions per sequence through the merge
    check_parity(dec, pools=False)
