"""Prefix caching end to end on the GPU.

[ART] paragraph on prefix caching: a request that starts with tokens already
seen reuses their cached K/V blocks and computes attention only for the rest;
[HADA] bullet "Prefix Caching".  Here one request runs a full prefill and
registers its blocks; later requests with the same prompt look the prompt up
in the library's allocator, store only their own tokens, and run their prefill
with cached_lens = the cached token count.  Their output must equal the
oracle's attention over each request's whole logical sequence, computed from
contiguous rows with no sharing at all.  A K/V row here depends only on the
prefix that ends at it, as in a real model: the prompt's rows are shared,
each suffix has rows of its own.
"""

import math

import numpy as np
import pytest

import oracle
import workloads
from helpers import compare, ensure_library

pytestmark = pytest.mark.gpu

B = 16


def _bits(rng, shape):
    return workloads.bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _logical_pool(rows_per_req, Hkv, D):
    """Oracle-side pool: each request's rows in blocks of their own, tables = consecutive ids."""
    blocks, tables, nb = [], [], 0
    for rows in rows_per_req:
        L = rows.shape[0]
        n = -(-L // B)
        pad = np.zeros((n * B, Hkv, D), dtype=rows.dtype)
        pad[:L] = rows
        blocks.append(pad.reshape(n, B, Hkv, D).transpose(0, 2, 1, 3))
        tables.append(list(range(nb, nb + n)))
        nb += n
    return np.ascontiguousarray(np.concatenate(blocks)), tables


@pytest.mark.parametrize("prompt_len, suffixes", [(150, [1, 7, 33, 64]), (64, [1, 16, 2]), (9, [5, 30])])
def test_prefix_cached_prefill_matches_full_attention(prompt_len, suffixes):
    pa = ensure_library()
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(prompt_len)
    Hq, Hkv, D = 8, 2, 128
    scale = 1.0 / math.sqrt(D)
    num_blocks = 64
    prompt = rng.integers(0, 30000, size=prompt_len).tolist()
    p_k, p_v = _bits(rng, (prompt_len, Hkv, D)), _bits(rng, (prompt_len, Hkv, D))
    reqs = []
    for r, n in enumerate(suffixes):
        toks = prompt + list(range(50000 + 1000 * r, 50000 + 1000 * r + n))
        k = np.concatenate([p_k, _bits(rng, (n, Hkv, D))])
        v = np.concatenate([p_v, _bits(rng, (n, Hkv, D))])
        q = _bits(rng, (len(toks), Hq, D))
        reqs.append((toks, k, v, q))

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    shape = (num_blocks + 1, Hkv, B, D)                 # one guard block past the allocator's range
    k_cache = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    v_cache = torch.full(shape, 0x7FC0, dtype=torch.int16, device=dev).view(torch.bfloat16)
    alloc = pa.BlockAllocator(num_blocks, B)

    def run(batch):
        """Prefill a batch of (request index, sequence id, cached tokens) and return its output rows."""
        tables, seq_lens, cached, qrows = [], [], [], []
        for i, sid, c in batch:
            toks, k, v, q = reqs[i]
            slots, pairs = alloc.append(sid, len(toks) - c)
            assert pairs == []
            pa.pa_write_kv(dev_bf16(k[c:]), dev_bf16(v[c:]), k_cache, v_cache,
                           torch.from_numpy(slots.copy()).to(dev))
            tables.append(alloc.block_table(sid))
            seq_lens.append(len(toks))
            cached.append(c)
            qrows.append(q[c:])
        width = max(len(t) for t in tables)
        bt = np.full((len(tables), width), num_blocks, dtype=np.int32)
        for j, t in enumerate(tables):
            bt[j, :len(t)] = t
        qlens = [len(x) for x in qrows]
        qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
        qd = dev_bf16(np.concatenate(qrows))
        out = torch.full_like(qd, float("nan"))
        ws_n = pa.pa_forward_workspace_size(len(batch), int(qsl[-1]), Hq, max(seq_lens), max(qlens), k_cache)
        ws = pa.new_workspace(ws_n, dev) if ws_n else None
        pa.pa_forward(out, qd, k_cache, v_cache, torch.from_numpy(bt).to(dev),
                      torch.tensor(seq_lens, dtype=torch.int32, device=dev), torch.from_numpy(qsl).to(dev),
                      torch.tensor(cached, dtype=torch.int32, device=dev), max(seq_lens), max(qlens), scale, 1,
                      workspace=ws)
        torch.cuda.synchronize()
        got = out.to(torch.float64).cpu().numpy()

        # oracle: whole logical sequences, laid out with no sharing at all
        kpool, tabs = _logical_pool([reqs[i][1] for i, _, _ in batch], Hkv, D)
        vpool, _ = _logical_pool([reqs[i][2] for i, _, _ in batch], Hkv, D)
        want = oracle.ref_paged_attention(np.concatenate(qrows), kpool, vpool, tabs, seq_lens, qsl, cached,
                                          scale, True, B, "bf16")
        ok, max_abs, mean_abs = compare(got, want, "bf16")
        print(f"[prefix] P={prompt_len} batch={[(i, c) for i, _, c in batch]}: "
              f"max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}", flush=True)
        assert ok, (max_abs, mean_abs)

    # request 0: nothing cached; full prefill, then its blocks are registered and it finishes
    toks0 = reqs[0][0]
    s0, c0 = alloc.prefix_lookup(toks0)
    assert c0 == 0
    run([(0, s0, 0)])
    alloc.prefix_register(s0, toks0)
    alloc.free_seq(s0)                     # its blocks stay cached on the free list
    # the others reuse the prompt's full blocks and prefill only their own tokens, in one batch
    batch = []
    for i in range(1, len(reqs)):
        sid, c = alloc.prefix_lookup(reqs[i][0])
        assert c == min(prompt_len // B, (len(reqs[i][0]) - 1) // B) * B
        batch.append((i, sid, c))
    run(batch)
    st = alloc.prefix_stats()
    assert st["hit_blocks"] == sum(c for _, _, c in batch) // B
    assert st["evictions"] == 0
