"""Test-side helpers: run a workload through the oracle, and rebuild logical K/V rows.

Only tests, smoke() and the bench's CPU-baseline leg use these; they call the
oracle and the workload generator, never the HIP path.
"""

import numpy as np

import oracle
import workloads

BF16_NAN = np.uint16(0x7FC0)


def nan_pool(wl):
    """K and V pools of ``wl.pool_blocks`` blocks, every element NaN (fp8: every code and scale byte 0xff)."""
    if wl.cache == "fp8":
        return (oracle.fp8_pool(wl.pool_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size),
                oracle.fp8_pool(wl.pool_blocks, wl.num_kv_heads, wl.head_dim, wl.block_size))
    shape = (wl.pool_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    if wl.dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32), np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, BF16_NAN, dtype=np.uint16), np.full(shape, BF16_NAN, dtype=np.uint16)


def _write_fp8(k_pool, v_pool, k, v, slots, block_size, chunk=1 << 16):
    """Quantised write of bf16 rows (widened exactly), in chunks of tokens to bound memory."""
    for a in range(0, len(slots), chunk):
        b = min(len(slots), a + chunk)
        oracle.ref_write_kv_fp8(k_pool, v_pool, oracle.to_f64(k[a:b], "bf16"), oracle.to_f64(v[a:b], "bf16"),
                                slots[a:b], block_size)


class OracleRun:
    """Everything the oracle side computes for one workload."""

    def __init__(self, wl, compute_out=True, seqs=None):
        self.wl = wl
        self.alloc = oracle.RefAllocator(wl.num_blocks, wl.block_size, wl.free_order)
        self.ids, self.ctx_slots, self.new_slots, self.cow = workloads.drive(wl, self.alloc)
        self.k_cache, self.v_cache = nan_pool(wl)
        write = _write_fp8 if wl.cache == "fp8" else oracle.ref_write_kv
        write(self.k_cache, self.v_cache, wl.ctx_k, wl.ctx_v, self.ctx_slots, wl.block_size)
        oracle.ref_copy_blocks(self.k_cache, self.v_cache, self.cow)
        write(self.k_cache, self.v_cache, wl.k_new, wl.v_new, self.new_slots, wl.block_size)
        self.tables = [self.alloc.block_table(self.ids[h]) for h in wl.batch]
        self.out = None
        if compute_out:
            self.out = self.attention(seqs)

    def attention(self, seqs=None):
        """Oracle output [T][Hq][D] (float64); with ``seqs`` only those sequences' rows are filled."""
        wl = self.wl
        qsl = wl.query_start_loc
        if seqs is None:
            return oracle.ref_paged_attention(
                wl.q, self.k_cache, self.v_cache, self.tables, wl.seq_lens, qsl,
                wl.cached_lens, wl.scale, wl.causal, wl.block_size, wl.cache)
        out = np.full((wl.num_tokens, wl.num_q_heads, wl.head_dim), np.nan)
        for i in seqs:
            r0, r1 = int(qsl[i]), int(qsl[i + 1])
            sub = oracle.ref_paged_attention(
                wl.q[r0:r1], self.k_cache, self.v_cache, [self.tables[i]],
                wl.seq_lens[i:i + 1], np.array([0, r1 - r0]), wl.cached_lens[i:i + 1],
                wl.scale, wl.causal, wl.block_size, wl.cache)
            out[r0:r1] = sub
        return out


def logical_rows(wl):
    """Each batch sequence's K/V rows in logical order, rebuilt from the trace alone.

    This follows token identity (which generated row a position holds) with
    no blocks, tables or slots: create -> empty, fork -> parent's first k rows,
    append -> extend.  Returns lists of (K, V) arrays per batch sequence.
    """
    rows = {}
    for op in wl.trace:
        kind = op[0]
        if kind == "create":
            rows[op[1]] = []
        elif kind == "fork":
            rows[op[1]] = list(rows[op[2]][: op[3]])
        elif kind == "append_ctx":
            _, s, n, r0 = op
            rows[s].extend(("ctx", r) for r in range(r0, r0 + n))
        elif kind == "append_new":
            _, s, n, r0 = op
            rows[s].extend(("new", r) for r in range(r0, r0 + n))
    out = []
    for h in wl.batch:
        ks = [wl.ctx_k[r] if src == "ctx" else wl.k_new[r] for src, r in rows[h]]
        vs = [wl.ctx_v[r] if src == "ctx" else wl.v_new[r] for src, r in rows[h]]
        out.append((np.stack(ks), np.stack(vs)))
    return out


def oracle_from_rows(rows, q, query_lens, wl):
    """Oracle output for sequences given by their logical K/V rows (``rows[i] = (K, V)``, stored
    format, ``[L_i][Hkv][D]``) and query rows ``q`` (``query_lens[i]`` rows each, the last ones of
    the sequence), with ``wl``'s heads, dtype, cache format, scale and mask.  The rows go into a
    fresh oracle pool, each sequence in blocks of its own, through the oracle's cache write."""
    B = wl.block_size
    lens = np.array([len(k) for k, _ in rows], dtype=np.int64)
    nb = int(sum(-(-L // B) for L in lens)) + 1
    if wl.cache == "fp8":
        kc = oracle.fp8_pool(nb, wl.num_kv_heads, wl.head_dim, B)
        vc = oracle.fp8_pool(nb, wl.num_kv_heads, wl.head_dim, B)
    else:
        kc, vc = (np.zeros((nb, wl.num_kv_heads, B, wl.head_dim), dtype=rows[0][0].dtype) for _ in range(2))
    tables, b0 = [], 0
    write = _write_fp8 if wl.cache == "fp8" else oracle.ref_write_kv
    for K, V in rows:
        n = -(-len(K) // B)
        tables.append(list(range(b0, b0 + n)))
        slots = np.array([(b0 + t // B) * B + t % B for t in range(len(K))], dtype=np.int64)
        write(kc, vc, K, V, slots, B)
        b0 += n
    query_lens = np.asarray(query_lens, dtype=np.int64)
    qsl = np.concatenate([[0], np.cumsum(query_lens)])
    return oracle.ref_paged_attention(q, kc, vc, tables, lens, qsl, lens - query_lens, wl.scale, wl.causal,
                                      B, wl.cache)


def compare(got, want, dtype):
    """Max-abs / mean-abs error and the pass/fail of the stated tolerance.

    bf16 data: max-abs <= 2e-2 and mean-abs <= 2e-3; fp32 data: max-abs <= 1e-4.
    """
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    mean_abs = float(err.mean()) if err.size else 0.0
    if not np.all(np.isfinite(got)):
        return False, max_abs, mean_abs
    if dtype == "bf16":
        ok = max_abs <= 2e-2 and mean_abs <= 2e-3
    else:
        ok = max_abs <= 1e-4
    return ok, max_abs, mean_abs


def ensure_library():
    """Import the binding, building libpagedattn.so first if it is not there."""
    import os
    from paged_kv_cache_forward_amd import build as _build
    if not os.path.exists(_build.LIB):
        _build.build()
    import paged_kv_cache_forward_amd as pa
    return pa
