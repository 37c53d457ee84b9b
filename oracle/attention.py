"""Paged attention over a flattened variable-length super-batch (oracle side).

What the pages fix:
  * [AIU] "Plongée profonde" and FAQ (KV-cache question): the cache keeps a
    key and a value vector for every token already seen so the next token can
    attend to the whole previous context without recomputing it.
  * [SLAVA] lead paragraph / [AIU] "Plongée profonde": those vectors sit in
    fixed-size blocks anywhere in memory, found through a per-request table
    from logical positions to physical blocks.  Paging does not change the
    K/V data stored per token.
  * [ART] forward-pass paragraph: all sequences of one step form a single
    super-batch without padding; masks and exact position indices keep each
    sequence to its own tokens.  Decode and prefill rows mix in one step
    ([ART] engine paragraph).
  * [HADA] "Chunked Prefill" / [ART] chunked-prefill paragraph: a long prompt's
    prefill is cut into chunks processed over several steps on top of the
    tokens already cached.

The pages print no attention formula.  Reading taken: scaled dot-product
attention with a softmax over each query's visible keys, computed in float64:

  for sequence i, query row j (absolute position c_i + j), query head h,
  KV head g = floor(h / G) with G = Hq / Hkv:
      visible t:  t <= c_i + j          (causal)
                  t <  L_i              (non-causal)
      s_t   = scale * <q, K_t>
      out   = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)

with L_i = c_i + n_i the tokens in cache after this step's write (the new
tokens are written before attention), K_t / V_t row t of sequence i read
through its block table, and n_i = query_start_loc[i+1] - query_start_loc[i].
"""

import numpy as np

from .numerics import to_f64
from .quant import gather_logical_fp8


def gather_logical(cache, table, length, block_size):
    """Rows 0..length-1 of one sequence in logical order: ``[length][Hkv][D]``.

    Token t lives in physical block ``table[t // block_size]`` at row
    ``t % block_size`` ([SLAVA] lead paragraph).  Only the sequence's own
    ``length`` rows are read; slots past it are never touched.
    """
    t = np.arange(length)
    blocks = np.asarray(table, dtype=np.int64)[t // block_size]
    return cache[blocks, :, t % block_size, :]


def ref_paged_attention(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                        cached_lens, scale, causal, block_size, dtype):
    """Attention output in float64, ``[num_tokens][Hq][D]``.

    ``q`` is ``[num_tokens][Hq][D]``, the caches ``[NB][Hkv][B][D]``, all stored
    as ``dtype`` ("f32" or "bf16" bit patterns).  With ``dtype`` "fp8" the
    caches are quantised pools
    read as their exact dequantised values (``oracle.quant.Fp8Pool``), and ``q`` is bf16.  ``block_tables[i]`` lists the
    physical blocks of sequence i in logical order.  Rows of every sequence
    are attended independently; rows belonging to no sequence stay zero.
    """
    q = np.asarray(q)
    num_tokens, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.num_kv_heads if dtype == "fp8" else k_cache.shape[1]
    q_dtype = "bf16" if dtype == "fp8" else dtype
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_tokens, num_q_heads, head_dim), dtype=np.float64)

    for i in range(len(seq_lens)):
        r0, r1 = int(query_start_loc[i]), int(query_start_loc[i + 1])
        n, L, c = r1 - r0, int(seq_lens[i]), int(cached_lens[i])
        if L != c + n:
            raise ValueError(f"sequence {i}: seq_len {L} != cached {c} + new {n}")
        if n == 0:
            continue
        if dtype == "fp8":
            K = gather_logical_fp8(k_cache, block_tables[i], L, block_size, "k")
            V = gather_logical_fp8(v_cache, block_tables[i], L, block_size, "v")
        else:
            K = to_f64(gather_logical(k_cache, block_tables[i], L, block_size), dtype)
            V = to_f64(gather_logical(v_cache, block_tables[i], L, block_size), dtype)
        Q = to_f64(q[r0:r1], q_dtype)

        pos = c + np.arange(n)[:, None]          # absolute position of each row
        t = np.arange(L)[None, :]
        visible = (t <= pos) if causal else np.ones((n, L), dtype=bool)

        for h in range(num_q_heads):
            g = h // group
            s = scale * (Q[:, h, :] @ K[:, g, :].T)           # [n][L]
            s = np.where(visible, s, -np.inf)
            w = np.exp(s - s.max(axis=1, keepdims=True))      # masked -> 0
            out[r0:r1, h, :] = (w @ V[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out


# -- split-KV pieces (used to pin the partition/merge identity) ---------------

def ref_partition_state(q_vec, K, V, scale):
    """Softmax state of one query vector over one partition of keys.

    Returns (m, l, acc): m = max score, l = sum exp(s - m), acc = sum exp(s - m) V.
    ``K``/``V`` are ``[n][D]`` float64 rows of the partition (n >= 1).
    """
    s = scale * (K @ q_vec)
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ V


def ref_lse_merge(states):
    """Combine partition states: rescale each by exp(m_p - M), M = max_p m_p."""
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den


def ref_split_attention_row(q_vec, K, V, scale, part):
    """One query over keys 0..len(K)-1 cut into consecutive partitions of ``part``."""
    L = K.shape[0]
    states = [ref_partition_state(q_vec, K[a:a + part], V[a:a + part], scale)
              for a in range(0, L, part)]
    return ref_lse_merge(states)
