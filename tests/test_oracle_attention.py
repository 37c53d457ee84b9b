"""Pins for the attention oracle.

The pages print no attention values, so the oracle is pinned by:
  * a float64 library routine on contiguous data (torch's
    scaled_dot_product_attention on the CPU with an explicit boolean mask),
    fed K/V rebuilt in logical order from the trace with no blocks involved;
  * closed forms (one visible token, zero scale, equal values, one dominant key);
  * invariances the pages imply: blocks may sit anywhere ([AIU] "Plongée
    profonde"), block size is a runtime choice ([SLAVA] "Ungenutzten Platz in
    Blöcken berechnen"), shared blocks give what private copies give ([SLAVA]
    "Gemeinsame Nutzung ..."), each sequence sees only its own tokens ([ART]
    forward-pass paragraph), chunked prefill splits work without changing it
    ([HADA] "Chunked Prefill", [ART] chunked-prefill paragraph);
  * the split-KV partition/merge identity.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import OracleRun, logical_rows


def sdpa_f64(Q, K, V, cached, scale, causal):
    """torch SDPA in float64: Q [n][Hq][D], K/V [L][Hkv][D], query row j at position cached+j."""
    n, Hq, D = Q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    q = torch.from_numpy(np.ascontiguousarray(Q.transpose(1, 0, 2)))[None]
    k = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, dim=0)[None]
    v = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, dim=0)[None]
    if causal:
        mask = torch.arange(L)[None, :] <= (cached + torch.arange(n))[:, None]
    else:
        mask = torch.ones(n, L, dtype=torch.bool)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return out[0].numpy().transpose(1, 0, 2)


def paged(seqs, Hkv, D, B, rng, dtype="f32", extra_blocks=3):
    """Place contiguous per-sequence K/V ([L][Hkv][D]) into a NaN pool through RefAllocator."""
    nb = sum(oracle.blocks_needed(len(k), B) for k, _ in seqs) + extra_blocks
    a = oracle.RefAllocator(nb, B, rng.permutation(nb))
    fill = np.float32(np.nan)
    kc = np.full((nb, Hkv, B, D), fill, dtype=np.float32)
    vc = np.full((nb, Hkv, B, D), fill, dtype=np.float32)
    tables = []
    for K, V in seqs:
        s = a.create()
        slots, _ = a.append(s, len(K))
        oracle.ref_write_kv(kc, vc, K, V, slots, B)
        tables.append(a.block_table(s))
    return kc, vc, tables


def run_paged(seqs, Qs, cached, Hkv, D, B, scale, causal, rng):
    kc, vc, tables = paged(seqs, Hkv, D, B, rng)
    q = np.concatenate(Qs).astype(np.float32)
    qsl = np.concatenate([[0], np.cumsum([len(x) for x in Qs])])
    L = np.array([len(k) for k, _ in seqs])
    return oracle.ref_paged_attention(q, kc, vc, tables, L, qsl, np.asarray(cached), scale,
                                      causal, B, "f32")


def rand_case(rng, Hq, Hkv, D, lens_new, lens_cached):
    seqs, Qs = [], []
    for n, c in zip(lens_new, lens_cached):
        L = n + c
        seqs.append((rng.standard_normal((L, Hkv, D)).astype(np.float32),
                     rng.standard_normal((L, Hkv, D)).astype(np.float32)))
        Qs.append(rng.standard_normal((n, Hq, D)).astype(np.float32))
    return seqs, Qs


CASES = [
    # Hq, Hkv, D, B, causal, new lens, cached lens
    (1, 1, 8, 1, True, [1, 3], [0, 5]),
    (2, 1, 8, 2, True, [17, 1], [4, 30]),
    (4, 2, 64, 16, True, [3, 1, 17], [50, 0, 13]),
    (8, 2, 8, 32, False, [3, 17], [9, 40]),
    (8, 8, 64, 16, False, [1, 1], [70, 2]),
    (4, 1, 64, 4, True, [17], [0]),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_library_sdpa(case):
    Hq, Hkv, D, B, causal, new, cached = case
    rng = np.random.default_rng(100 + D + B)
    seqs, Qs = rand_case(rng, Hq, Hkv, D, new, cached)
    scale = 0.37
    got = run_paged(seqs, Qs, cached, Hkv, D, B, scale, causal, rng)
    r = 0
    for (K, V), Q, c in zip(seqs, Qs, cached):
        want = sdpa_f64(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64), c, scale, causal)
        assert np.max(np.abs(got[r:r + len(Q)] - want)) <= 1e-12
        r += len(Q)


def widen_by_torch(x, dtype):
    """Stored rows -> float64 through torch's own dtype conversions (not the oracle's widening)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float64).numpy()
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("name", ["decode_f32", "mixed_bf16", "shared_bf16", "noncausal_bf16"])
def test_workload_matches_library_sdpa(name):
    wl = workloads.mini(name)
    run = OracleRun(wl)
    rows = logical_rows(wl)
    qsl = wl.query_start_loc
    for i, (K, V) in enumerate(rows):
        Q = widen_by_torch(wl.q[qsl[i]:qsl[i + 1]], wl.dtype)
        want = sdpa_f64(Q, widen_by_torch(K, wl.dtype), widen_by_torch(V, wl.dtype),
                        int(wl.cached_lens[i]), wl.scale, wl.causal)
        assert np.max(np.abs(run.out[qsl[i]:qsl[i + 1]] - want)) <= 1e-12


def test_tiny_decode_single_token_sequence_returns_its_value():
    wl = workloads.tiny_decode()
    run = OracleRun(wl)
    i = 2                                             # context length 1
    assert wl.seq_lens[i] == 1
    v = oracle.to_f64(wl.v_new[i], wl.dtype)          # [Hkv][D]; Hq == Hkv here
    assert np.array_equal(run.out[i], v)


def test_closed_forms():
    rng = np.random.default_rng(5)
    Hq, Hkv, D, B = 4, 2, 8, 4
    seqs, Qs = rand_case(rng, Hq, Hkv, D, [5], [20])
    K, V = seqs[0]
    # zero scale: every visible key weighs the same -> mean of visible values
    out = run_paged(seqs, Qs, [20], Hkv, D, B, 0.0, True, rng)
    for j in range(5):
        for h in range(Hq):
            want = V[: 21 + j, h // 2, :].astype(np.float64).mean(axis=0)
            assert np.max(np.abs(out[j, h] - want)) <= 1e-12
    # zero query: same
    Qz = [np.zeros_like(Qs[0])]
    out = run_paged(seqs, Qz, [20], Hkv, D, B, 0.9, True, rng)
    assert np.max(np.abs(out[4, 3] - V[:25, 1].astype(np.float64).mean(axis=0))) <= 1e-12
    # all values equal -> that value
    Vc = np.broadcast_to(np.arange(D, dtype=np.float32), V.shape).copy()
    out = run_paged([(K, Vc)], Qs, [20], Hkv, D, B, 0.7, True, rng)
    assert np.max(np.abs(out - np.arange(D))) <= 1e-12
    # one key aligned with the query and much larger: output -> that key's value
    Kd = K.copy()
    t = 7
    Kd[t, 0] = 50.0 * Qs[0][0, 0] / np.linalg.norm(Qs[0][0, 0])
    out = run_paged([(Kd, V)], [Qs[0][:1]], [24], Hkv, D, B, 1.0, True, rng)
    assert np.max(np.abs(out[0, 0] - V[t, 0])) <= 1e-6


def test_invariant_under_physical_placement_and_block_size():
    rng = np.random.default_rng(9)
    seqs, Qs = rand_case(rng, 8, 2, 16, [1, 4, 9], [60, 0, 33])
    ref = run_paged(seqs, Qs, [60, 0, 33], 2, 16, 16, 0.25, True, np.random.default_rng(1))
    for B in (1, 2, 4, 16, 32, 64):
        for perm_seed in (2, 3):
            got = run_paged(seqs, Qs, [60, 0, 33], 2, 16, B, 0.25, True,
                            np.random.default_rng(perm_seed))
            assert np.array_equal(got, ref)


def test_isolation_order_and_other_sequences():
    rng = np.random.default_rng(11)
    seqs, Qs = rand_case(rng, 4, 4, 8, [1, 3, 1], [30, 7, 2])
    ref = run_paged(seqs, Qs, [30, 7, 2], 4, 8, 16, 0.5, True, rng)
    # reversed batch order
    got = run_paged(seqs[::-1], Qs[::-1], [2, 7, 30], 4, 8, 16, 0.5, True, rng)
    assert np.array_equal(got[0:1], ref[4:5])
    assert np.array_equal(got[1:4], ref[1:4])
    assert np.array_equal(got[4:5], ref[0:1])
    # perturb the other sequences' K/V: sequence 1 unchanged
    pert = [(k + 3.0, v - 2.0) for k, v in seqs]
    pert[1] = seqs[1]
    got = run_paged(pert, Qs, [30, 7, 2], 4, 8, 16, 0.5, True, rng)
    assert np.array_equal(got[1:4], ref[1:4])


def test_stale_slots_never_read():
    # The pool is NaN everywhere the writes do not reach; outputs must stay finite
    # and equal a zero-filled pool's.
    rng = np.random.default_rng(12)
    seqs, Qs = rand_case(rng, 2, 1, 8, [1, 1], [18, 3])
    kc, vc, tables = paged(seqs, 1, 8, 16, np.random.default_rng(0))
    q = np.concatenate(Qs)
    args = (tables, np.array([19, 4]), np.array([0, 1, 2]), np.array([18, 3]), 0.5, True, 16, "f32")
    out_nan = oracle.ref_paged_attention(q, kc, vc, *args)
    assert np.all(np.isfinite(out_nan))
    kz, vz = np.nan_to_num(kc, nan=0.0), np.nan_to_num(vc, nan=0.0)
    assert np.array_equal(out_nan, oracle.ref_paged_attention(q, kz, vz, *args))


def test_shared_prefix_equals_private_copies():
    wl = workloads.mini("shared_bf16")
    shared = OracleRun(wl)
    assert shared.cow, "the diverging sequence must copy a block"
    # private copies: same logical rows, every sequence in its own blocks
    rows = logical_rows(wl)
    B = wl.block_size
    nb = sum(oracle.blocks_needed(len(k), B) for k, _ in rows) + 1
    a = oracle.RefAllocator(nb, B, np.random.default_rng(4).permutation(nb))
    kc = np.full((nb, wl.num_kv_heads, B, wl.head_dim), np.uint16(0x7FC0), dtype=np.uint16)
    vc = kc.copy()
    tables = []
    for K, V in rows:
        s = a.create()
        slots, _ = a.append(s, len(K))
        oracle.ref_write_kv(kc, vc, K, V, slots, B)
        tables.append(a.block_table(s))
    private = oracle.ref_paged_attention(wl.q, kc, vc, tables, wl.seq_lens, wl.query_start_loc,
                                         wl.cached_lens, wl.scale, wl.causal, B, wl.dtype)
    assert np.array_equal(private, shared.out)


@pytest.mark.parametrize("part", [16, 512, 37, 1, 100000])
def test_split_merge_identity(part):
    rng = np.random.default_rng(21)
    L, D = 1300, 32
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    q = rng.standard_normal(D)
    s = 0.3 * (K @ q)
    w = np.exp(s - s.max())
    plain = (w @ V) / w.sum()
    got = oracle.ref_split_attention_row(q, K, V, 0.3, part)
    assert np.max(np.abs(got - plain)) <= 1e-12
    if part >= L:   # a single partition merges to itself
        m, l, acc = oracle.ref_partition_state(q, K, V, 0.3)
        assert np.array_equal(oracle.ref_lse_merge([(m, l, acc)]), acc / l)


def test_chunked_prefill_equals_one_chunk_and_decode_equals_prefill_row():
    rng = np.random.default_rng(31)
    Hq, Hkv, D, N = 4, 2, 16, 90
    K = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    Q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    whole = run_paged([(K, V)], [Q], [0], Hkv, D, 16, 0.3, True, rng)
    # chunks 0:25, 25:64, 64:90 -- each written before it attends, on top of the cached part
    for a, b in [(0, 25), (25, 64), (64, 90)]:
        part = run_paged([(K[:b], V[:b])], [Q[a:b]], [a], Hkv, D, 16, 0.3, True, rng)
        assert np.max(np.abs(part - whole[a:b])) <= 1e-12
    # a single-token decode at position p equals prefill row p
    for p in (0, 1, 15, 16, 89):
        dec = run_paged([(K[:p + 1], V[:p + 1])], [Q[p:p + 1]], [p], Hkv, D, 16, 0.3, True, rng)
        assert np.max(np.abs(dec[0] - whole[p])) <= 1e-12
