"""Seeded synthetic workloads for paged KV-cache attention.

This module only makes inputs: sequence lengths, N(0,1) values, free-list
orders and allocator operation traces.  It holds none of the method's
arithmetic (no block tables, slots, or attention); both the CPU oracle side
and the GPU side consume what it returns, each running its own allocator and
cache writes on the same trace.

All values are float32 N(0,1) drawn from NumPy's PCG64 with the workload's
seed, then rounded to bfloat16 (round-to-nearest-even) where the workload is
bf16.  bf16 data is carried as uint16 bit patterns.  Lengths are uniform over
inclusive integer ranges.

Trace operations (replayed in order by ``drive``):
  ("create", s)                    new empty sequence, handle s
  ("fork", s, parent, k)           new sequence sharing parent's first k tokens
  ("append_ctx", s, n, row0)       n cached tokens; K/V rows ctx_k[row0:row0+n]
  ("append_new", s, n, row0)       n tokens of this step; rows k_new[row0:row0+n]
"""

from dataclasses import dataclass, field
import math

import numpy as np

BLOCK_SIZE = 16


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even) and return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def _normal(rng, shape, dtype, chunk_rows=1 << 16):
    """N(0,1) values of ``shape`` stored as dtype ("f32" or "bf16" bits), drawn row-chunk by row-chunk."""
    out = np.empty(shape, dtype=np.float32 if dtype == "f32" else np.uint16)
    rows = shape[0]
    for a in range(0, rows, chunk_rows):
        b = min(rows, a + chunk_rows)
        v = rng.standard_normal((b - a,) + tuple(shape[1:]), dtype=np.float32)
        out[a:b] = v if dtype == "f32" else bf16_bits(v)
    return out


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                    # "f32" or "bf16"
    scale: float
    causal: bool
    num_blocks: int               # blocks the allocator manages
    free_order: np.ndarray        # int32 permutation of 0..num_blocks-1
    batch: list                   # trace handle of each super-batch sequence, in batch order
    seq_lens: np.ndarray          # int32 [S]: tokens in cache after this step's write
    cached_lens: np.ndarray       # int32 [S]: tokens in cache before it
    query_lens: np.ndarray        # int32 [S]: this step's query tokens
    q: np.ndarray                 # [T][Hq][D]
    k_new: np.ndarray             # [T][Hkv][D]
    v_new: np.ndarray
    ctx_k: np.ndarray             # [Nctx][Hkv][D] cached tokens' rows
    ctx_v: np.ndarray
    trace: list
    block_size: int = BLOCK_SIZE
    notes: dict = field(default_factory=dict)
    cache_dtype: str = ""         # "" = the same as dtype; "fp8" = quantised pools, bf16 rows

    @property
    def cache(self):
        return self.cache_dtype or self.dtype

    @property
    def num_seqs(self):
        return len(self.batch)

    @property
    def num_tokens(self):
        return int(self.query_lens.sum())

    @property
    def query_start_loc(self):
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    @property
    def guard_block(self):
        """Extra pool block past the allocator's range; used as block-table padding."""
        return self.num_blocks

    @property
    def pool_blocks(self):
        return self.num_blocks + 1

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    @property
    def max_query_len(self):
        return int(self.query_lens.max()) if len(self.query_lens) else 0


def drive(wl, alloc):
    """Replay ``wl.trace`` on ``alloc`` (create / fork / append API).

    Returns (handles, ctx_slots, new_slots, step_cow_pairs): the allocator's id
    for each trace handle, the slot of every cached row and every new row, and
    the copy-on-write pairs the step's appends produced.  Appends of cached
    rows must produce no copies (checked).
    """
    ids = {}
    ctx_slots = np.full(len(wl.ctx_k), -1, dtype=np.int64)
    new_slots = np.full(len(wl.k_new), -1, dtype=np.int64)
    cow = []
    for op in wl.trace:
        kind = op[0]
        if kind == "create":
            ids[op[1]] = alloc.create()
        elif kind == "fork":
            ids[op[1]] = alloc.fork(ids[op[2]], op[3])
        elif kind in ("append_ctx", "append_new"):
            _, s, n, row0 = op
            slots, pairs = alloc.append(ids[s], n)
            if kind == "append_ctx":
                if pairs:
                    raise RuntimeError("cached-token append produced copy-on-write pairs")
                ctx_slots[row0:row0 + n] = slots
            else:
                new_slots[row0:row0 + n] = slots
                cow.extend(pairs)
        else:
            raise ValueError(f"unknown trace op {op!r}")
    return ids, ctx_slots, new_slots, cow


def block_table_array(wl, alloc, ids, stride=None):
    """Batch-ordered block tables as int32 ``[S][stride]``, padded with the guard block."""
    tables = [alloc.block_table(ids[h]) for h in wl.batch]
    width = max([len(t) for t in tables] + [1]) if stride is None else stride
    out = np.full((len(tables), width), wl.guard_block, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, :len(t)] = t
    return out


# -- builders ----------------------------------------------------------------

def independent(name, seed, *, Hq, Hkv, D, dtype, cached, new, num_blocks=None,
                pool_factor=None, pool_extra=0, causal=True, scale=None, notes=None, cache_dtype=""):
    """Sequences with private blocks: sequence i holds cached[i] tokens and adds new[i].

    The trace creates every sequence and appends its cached tokens in batch
    order, then appends each sequence's new tokens (this step).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cached = np.asarray(cached, dtype=np.int64)
    new = np.asarray(new, dtype=np.int64)
    S = len(cached)
    blocks = int(sum(math.ceil((c + n) / BLOCK_SIZE) for c, n in zip(cached, new)))
    if num_blocks is None:
        num_blocks = (math.ceil(pool_factor * blocks) if pool_factor else blocks) + pool_extra
    free_order = rng.permutation(num_blocks).astype(np.int32)
    T, Nctx = int(new.sum()), int(cached.sum())
    q = _normal(rng, (T, Hq, D), dtype)
    k_new = _normal(rng, (T, Hkv, D), dtype)
    v_new = _normal(rng, (T, Hkv, D), dtype)
    ctx_k = _normal(rng, (Nctx, Hkv, D), dtype)
    ctx_v = _normal(rng, (Nctx, Hkv, D), dtype)
    trace, row = [], 0
    for i in range(S):
        trace.append(("create", i))
        if cached[i]:
            trace.append(("append_ctx", i, int(cached[i]), row))
        row += int(cached[i])
    row = 0
    for i in range(S):
        if new[i]:
            trace.append(("append_new", i, int(new[i]), row))
        row += int(new[i])
    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
        scale=(1.0 / math.sqrt(D)) if scale is None else scale, causal=causal,
        num_blocks=num_blocks, free_order=free_order, batch=list(range(S)),
        seq_lens=(cached + new).astype(np.int32), cached_lens=cached.astype(np.int32),
        query_lens=new.astype(np.int32), q=q, k_new=k_new, v_new=v_new,
        ctx_k=ctx_k, ctx_v=ctx_v, trace=trace, notes=dict(notes or {}), cache_dtype=cache_dtype)


def shared_prefix(name, seed, *, Hq, Hkv, D, dtype, num_seqs, prefix, suffix_max,
                  num_blocks, causal=True, notes=None):
    """Fan-out over one shared prefix, with one sequence diverging inside a shared block.

    Sequence 0 stores ``prefix`` tokens; sequences 1..S-2 fork it at the full
    prefix; sequence S-1 forks it at ``prefix - r`` with r ~ U{1..15}, so its
    next token lands inside the last shared block (a copy-on-write).  Sequences
    0..S-2 then add private suffixes of U{0..suffix_max} tokens.  This step
    adds one token to every sequence.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    S = num_seqs
    suffix = rng.integers(0, suffix_max + 1, size=S - 1)
    r = int(rng.integers(1, BLOCK_SIZE))          # 1..15
    cached = np.concatenate([prefix + suffix, [prefix - r]]).astype(np.int64)
    new = np.ones(S, dtype=np.int64)
    T, Nctx = S, int(prefix + suffix.sum())
    q = _normal(rng, (T, Hq, D), dtype)
    k_new = _normal(rng, (T, Hkv, D), dtype)
    v_new = _normal(rng, (T, Hkv, D), dtype)
    ctx_k = _normal(rng, (Nctx, Hkv, D), dtype)
    ctx_v = _normal(rng, (Nctx, Hkv, D), dtype)
    trace = [("create", 0), ("append_ctx", 0, prefix, 0)]
    for i in range(1, S - 1):
        trace.append(("fork", i, 0, prefix))
    trace.append(("fork", S - 1, 0, prefix - r))
    row = prefix
    for i in range(S - 1):
        if suffix[i]:
            trace.append(("append_ctx", i, int(suffix[i]), row))
        row += int(suffix[i])
    for i in range(S):
        trace.append(("append_new", i, 1, i))
    info = {"prefix": prefix, "diverge_r": r, "suffix": suffix.tolist()}
    info.update(notes or {})
    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
        scale=1.0 / math.sqrt(D), causal=causal, num_blocks=num_blocks,
        free_order=free_order, batch=list(range(S)),
        seq_lens=(cached + new).astype(np.int32), cached_lens=cached.astype(np.int32),
        query_lens=new.astype(np.int32), q=q, k_new=k_new, v_new=v_new,
        ctx_k=ctx_k, ctx_v=ctx_v, trace=trace, notes=info)


def unshared(wl, name=None, seed_offset=1000):
    """The same batch with every sequence holding private copies of its rows: no forks.

    Each batch sequence gets the same logical rows (token by token: the same
    cached K/V rows, then the same new rows) as in ``wl``, but stored by its
    own create + append_ctx + append_new, so no block is shared and no
    copy-on-write happens.  q, the new rows, lengths and batch order are
    unchanged; the pool gets a fresh free-list order (seeded).  This only
    rearranges the trace and duplicates input rows.
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
    ctx_idx, trace, new_ops = [], [], []
    for i, h in enumerate(wl.batch):
        lr = rows[h]
        n = int(wl.query_lens[i])
        cached = lr[:len(lr) - n]
        if any(src != "ctx" for src, _ in cached) or any(src != "new" for src, _ in lr[len(lr) - n:]):
            raise ValueError("a sequence's new rows must come after all of its cached rows")
        trace.append(("create", i))
        if cached:
            trace.append(("append_ctx", i, len(cached), len(ctx_idx)))
            ctx_idx.extend(r for _, r in cached)
        if n:
            new_ops.append(("append_new", i, n, int(lr[len(lr) - n][1])))
    trace.extend(new_ops)
    ctx_idx = np.asarray(ctx_idx, dtype=np.int64)
    blocks = int(sum(math.ceil(int(L) / BLOCK_SIZE) for L in wl.seq_lens))
    num_blocks = max(wl.num_blocks, blocks + 1)
    rng = np.random.Generator(np.random.PCG64(wl.seed + seed_offset))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return Workload(
        name=name or wl.name + "_unshared", seed=wl.seed, num_q_heads=wl.num_q_heads,
        num_kv_heads=wl.num_kv_heads, head_dim=wl.head_dim, dtype=wl.dtype, scale=wl.scale,
        causal=wl.causal, num_blocks=num_blocks, free_order=free_order, batch=list(range(wl.num_seqs)),
        seq_lens=wl.seq_lens.copy(), cached_lens=wl.cached_lens.copy(), query_lens=wl.query_lens.copy(),
        q=wl.q, k_new=wl.k_new, v_new=wl.v_new, ctx_k=wl.ctx_k[ctx_idx], ctx_v=wl.ctx_v[ctx_idx],
        trace=trace, notes=dict(wl.notes, unshared_from=wl.name), cache_dtype=wl.cache_dtype)


def fork_tree(name, seed, *, Hq, Hkv, D, dtype, root, forks, suffix_max, num_blocks=None, pool_extra=4):
    """Sequences forked from each other, one decode token each, in batch order.

    ``root`` tokens are stored for sequence 0; sequence i >= 1 forks
    ``forks[i-1] = (parent, k)`` (parent < i, k <= the parent's length at that
    point: the parent's first k tokens are shared); then every sequence whose
    length is a whole number of blocks adds a private suffix of
    U{0..suffix_max} cached tokens (the others may share their last, partial
    block, which a cached append must not write into), and finally one new
    token each (a sequence whose next token lands inside a shared block copies
    it first).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S = len(forks) + 1
    trace = [("create", 0), ("append_ctx", 0, root, 0)]
    lens = [root]
    row = root
    for i, (p, k) in enumerate(forks, start=1):
        if not (0 <= p < i and 0 <= k <= lens[p]):
            raise ValueError(f"fork {i}: parent {p}, {k} tokens")
        trace.append(("fork", i, p, k))
        lens.append(k)
    suffix = rng.integers(0, suffix_max + 1, size=S)
    suffix[[L % BLOCK_SIZE != 0 for L in lens]] = 0
    for i in range(S):
        if suffix[i]:
            trace.append(("append_ctx", i, int(suffix[i]), row))
            row += int(suffix[i])
            lens[i] += int(suffix[i])
    for i in range(S):
        trace.append(("append_new", i, 1, i))
    cached = np.asarray(lens, dtype=np.int64)
    new = np.ones(S, dtype=np.int64)
    blocks = int(sum(math.ceil((c + 1) / BLOCK_SIZE) for c in cached))
    if num_blocks is None:
        num_blocks = blocks + pool_extra
    free_order = rng.permutation(num_blocks).astype(np.int32)
    q = _normal(rng, (S, Hq, D), dtype)
    k_new = _normal(rng, (S, Hkv, D), dtype)
    v_new = _normal(rng, (S, Hkv, D), dtype)
    ctx_k = _normal(rng, (row, Hkv, D), dtype)
    ctx_v = _normal(rng, (row, Hkv, D), dtype)
    return Workload(
        name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
        scale=1.0 / math.sqrt(D), causal=True, num_blocks=num_blocks, free_order=free_order,
        batch=list(range(S)), seq_lens=(cached + new).astype(np.int32), cached_lens=cached.astype(np.int32),
        query_lens=new.astype(np.int32), q=q, k_new=k_new, v_new=v_new, ctx_k=ctx_k, ctx_v=ctx_v,
        trace=trace, notes={"forks": list(forks), "suffix": suffix.tolist()})


# -- the five named workloads ------------------------------------------------

def _lengths(seed_offset_rng, lo, hi, n):
    return seed_offset_rng.integers(lo, hi + 1, size=n)


def tiny_decode():
    """4 sequences of context {35,16,1,50}, 1 new token each; 2/2 heads, D 64, fp32; pool 32."""
    L = np.array([35, 16, 1, 50])
    return independent("tiny_decode", 1, Hq=2, Hkv=2, D=64, dtype="f32",
                       cached=L - 1, new=np.ones(4, dtype=np.int64), num_blocks=32,
                       scale=1.0 / 8.0)


def batched_decode():
    """64 sequences, context U{128..4096}, 1 new token; 32/8 heads, D 128, bf16; pool 20000."""
    L = _lengths(np.random.Generator(np.random.PCG64(1002)), 128, 4096, 64)
    return independent("batched_decode", 2, Hq=32, Hkv=8, D=128, dtype="bf16",
                       cached=L - 1, new=np.ones(64, dtype=np.int64), num_blocks=20000)


def long_context_decode():
    """8 sequences, context U{32768..131072}, 1 new token; 64/8 heads, D 128, bf16."""
    L = _lengths(np.random.Generator(np.random.PCG64(1003)), 32768, 131072, 8)
    return independent("long_context_decode", 3, Hq=64, Hkv=8, D=128, dtype="bf16",
                       cached=L - 1, new=np.ones(8, dtype=np.int64), pool_extra=1024)


def mixed_superbatch():
    """16 decode sequences (context U{256..4096}) then 4 prefill chunks of 512 on 0/1024/4096/8192 cached."""
    L = _lengths(np.random.Generator(np.random.PCG64(1004)), 256, 4096, 16)
    cached = np.concatenate([L - 1, [0, 1024, 4096, 8192]])
    new = np.concatenate([np.ones(16, dtype=np.int64), [512] * 4])
    return independent("mixed_superbatch", 4, Hq=32, Hkv=8, D=128, dtype="bf16",
                       cached=cached, new=new, pool_factor=1.25)


def shared_prefix_cow():
    """256 sequences over a 2048-token shared prefix, suffixes U{0..512}, one diverging; pool 8192."""
    return shared_prefix("shared_prefix_cow", 5, Hq=32, Hkv=8, D=128, dtype="bf16",
                         num_seqs=256, prefix=2048, suffix_max=512, num_blocks=8192)


def spec_verify():
    """64 sequences, context U{128..4096} after the step, each verifying U{2..8} new tokens
    (speculative decoding: the draft tokens plus one), causal; 32/8 heads, D 128, bf16; pool 20000."""
    rng = np.random.Generator(np.random.PCG64(1006))
    L = _lengths(rng, 128, 4096, 64)
    n = _lengths(rng, 2, 8, 64)
    return independent("spec_verify", 6, Hq=32, Hkv=8, D=128, dtype="bf16",
                       cached=L - n, new=n, num_blocks=20000)


def batched_decode_fp8():
    """batched_decode on a quantised (fp8) cache: the same rows, stored as E4M3 codes with row scales."""
    L = _lengths(np.random.Generator(np.random.PCG64(1002)), 128, 4096, 64)
    return independent("batched_decode_fp8", 2, Hq=32, Hkv=8, D=128, dtype="bf16",
                       cached=L - 1, new=np.ones(64, dtype=np.int64), num_blocks=20000, cache_dtype="fp8")


def mixed_superbatch_fp8():
    """mixed_superbatch on a quantised (fp8) cache: 16 decode rows and four 512-token chunks."""
    L = _lengths(np.random.Generator(np.random.PCG64(1004)), 256, 4096, 16)
    cached = np.concatenate([L - 1, [0, 1024, 4096, 8192]])
    new = np.concatenate([np.ones(16, dtype=np.int64), [512] * 4])
    return independent("mixed_superbatch_fp8", 4, Hq=32, Hkv=8, D=128, dtype="bf16",
                       cached=cached, new=new, pool_factor=1.25, cache_dtype="fp8")


NAMED = {
    "tiny_decode": tiny_decode,
    "batched_decode": batched_decode,
    "long_context_decode": long_context_decode,
    "mixed_superbatch": mixed_superbatch,
    "shared_prefix_cow": shared_prefix_cow,
    "spec_verify": spec_verify,
    "batched_decode_fp8": batched_decode_fp8,
    "mixed_superbatch_fp8": mixed_superbatch_fp8,
}


def named(name):
    return NAMED[name]()


# -- small variants of the same shapes (the oracle finishes them in seconds) --

def mini(name):
    """Reduced-size workloads with the named workloads' structure, spanning several tiles and ragged tails."""
    if name == "decode_f32":
        rng = np.random.Generator(np.random.PCG64(11))
        L = rng.integers(1, 700, size=5)
        return independent(name, 11, Hq=4, Hkv=2, D=64, dtype="f32", cached=L - 1,
                           new=np.ones(5, dtype=np.int64), pool_extra=7)
    if name == "decode_bf16":
        rng = np.random.Generator(np.random.PCG64(12))
        L = np.concatenate([[1, 16, 17, 513], rng.integers(2, 2500, size=4)])
        return independent(name, 12, Hq=32, Hkv=8, D=128, dtype="bf16", cached=L - 1,
                           new=np.ones(len(L), dtype=np.int64), pool_extra=5)
    if name == "decode_gqa8":
        rng = np.random.Generator(np.random.PCG64(13))
        L = rng.integers(1500, 6000, size=3)
        return independent(name, 13, Hq=64, Hkv=8, D=128, dtype="bf16", cached=L - 1,
                           new=np.ones(3, dtype=np.int64), pool_extra=3)
    if name == "decode_mha":
        # one query head per KV head: the balanced decode and its merge at G = 1
        rng = np.random.Generator(np.random.PCG64(31))
        L = np.concatenate([[1, 16, 17, 48], rng.integers(2, 3000, size=4)])
        return independent(name, 31, Hq=8, Hkv=8, D=128, dtype="bf16", cached=L - 1,
                           new=np.ones(len(L), dtype=np.int64), pool_extra=4)
    if name == "decode_d64_bf16":
        rng = np.random.Generator(np.random.PCG64(14))
        L = rng.integers(1, 1200, size=5)
        return independent(name, 14, Hq=8, Hkv=8, D=64, dtype="bf16", cached=L - 1,
                           new=np.ones(5, dtype=np.int64))
    if name == "decode_d128_f32":
        rng = np.random.Generator(np.random.PCG64(15))
        L = rng.integers(1, 1200, size=4)
        return independent(name, 15, Hq=8, Hkv=1, D=128, dtype="f32", cached=L - 1,
                           new=np.ones(4, dtype=np.int64))
    if name == "mixed_bf16":
        cached = np.array([300, 1, 2000, 15, 0, 45, 700, 129])
        new = np.array([1, 1, 1, 1, 37, 130, 200, 64])
        return independent(name, 16, Hq=32, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_factor=1.25)
    if name == "mixed_gqa8":
        cached = np.array([0, 900, 33, 5])
        new = np.array([200, 77, 1, 16])
        return independent(name, 17, Hq=64, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2)
    if name == "mixed_mha_d64":
        cached = np.array([0, 250, 3])
        new = np.array([150, 90, 1])
        return independent(name, 18, Hq=4, Hkv=4, D=64, dtype="bf16", cached=cached,
                           new=new, pool_extra=2)
    if name == "prefill_f32":
        cached = np.array([0, 40, 7])
        new = np.array([33, 20, 1])
        return independent(name, 19, Hq=4, Hkv=2, D=64, dtype="f32", cached=cached,
                           new=new, pool_extra=2)
    if name == "noncausal_bf16":
        cached = np.array([10, 0, 64])
        new = np.array([50, 70, 1])
        return independent(name, 20, Hq=32, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2, causal=False)
    if name == "verify_bf16":
        # multi-token decode: 2..16 query tokens per sequence, ragged tails, a sequence with no cache
        cached = np.array([0, 1, 15, 16, 300, 1021, 2500, 47, 5])
        new = np.array([2, 3, 8, 16, 5, 4, 7, 2, 1])
        return independent(name, 22, Hq=32, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=3)
    if name == "verify_gqa8":
        cached = np.array([700, 3, 2047, 64])
        new = np.array([8, 6, 2, 9])
        return independent(name, 23, Hq=64, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2)
    if name == "verify_mha":
        cached = np.array([130, 0, 999])
        new = np.array([16, 4, 11])
        return independent(name, 24, Hq=8, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2)
    if name == "decode_fp8":
        rng = np.random.Generator(np.random.PCG64(25))
        L = np.concatenate([[1, 16, 17, 513], rng.integers(2, 2500, size=4)])
        return independent(name, 25, Hq=32, Hkv=8, D=128, dtype="bf16", cached=L - 1,
                           new=np.ones(len(L), dtype=np.int64), pool_extra=5, cache_dtype="fp8")
    if name == "verify_fp8":
        cached = np.array([0, 1, 15, 16, 300, 1021, 47, 5])
        new = np.array([2, 3, 8, 16, 1, 4, 2, 1])
        return independent(name, 26, Hq=32, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=3, cache_dtype="fp8")
    if name == "fp8_gqa8":
        cached = np.array([700, 3, 2047, 64, 0])
        new = np.array([1, 6, 2, 8, 1])
        return independent(name, 27, Hq=64, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2, cache_dtype="fp8")
    if name == "fp8_mha_noncausal":
        cached = np.array([130, 0, 999])
        new = np.array([16, 4, 1])
        return independent(name, 28, Hq=8, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2, cache_dtype="fp8", causal=False)
    if name == "mixed_fp8":
        # decode rows, multi-token rows and prefill chunks (ragged, one starting at 0) on an fp8 cache
        cached = np.array([300, 1, 2000, 15, 0, 45, 700, 129, 33])
        new = np.array([1, 1, 3, 1, 37, 130, 200, 64, 17])
        return independent(name, 29, Hq=32, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_factor=1.25, cache_dtype="fp8")
    if name == "prefill_fp8_gqa8_noncausal":
        cached = np.array([0, 900, 33, 5])
        new = np.array([200, 77, 1, 16])
        return independent(name, 30, Hq=64, Hkv=8, D=128, dtype="bf16", cached=cached,
                           new=new, pool_extra=2, cache_dtype="fp8", causal=False)
    if name == "shared_bf16":
        return shared_prefix(name, 21, Hq=32, Hkv=8, D=128, dtype="bf16", num_seqs=9,
                             prefix=160, suffix_max=70, num_blocks=200)
    raise KeyError(name)


MINI = ["decode_f32", "decode_bf16", "decode_gqa8", "decode_mha", "decode_d64_bf16", "decode_d128_f32",
        "mixed_bf16", "mixed_gqa8", "mixed_mha_d64", "prefill_f32", "noncausal_bf16",
        "shared_bf16", "verify_bf16", "verify_gqa8", "verify_mha", "decode_fp8", "verify_fp8", "fp8_gqa8",
        "fp8_mha_noncausal", "mixed_fp8", "prefill_fp8_gqa8_noncausal"]
