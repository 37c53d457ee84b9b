"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Each case replays one seeded workload twice -- on the library (C++ allocator,
device pools, pa_copy_blocks / pa_write_kv_forward) and on the oracle
(RefAllocator, NumPy pools, fp64 attention) -- and compares:
  * slots, block tables and copy pairs: bit-exact;
  * the whole K and V pools after the writes: bit-exact (NaN-poisoned
    everywhere no write reaches);
  * attention outputs: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3, fp32
    max-abs <= 1e-4, and every output finite.
"""

import os

import numpy as np
import pytest

import oracle
import workloads
from helpers import OracleRun, compare, ensure_library

pytestmark = pytest.mark.gpu


def _device_run(wl, **kw):
    ensure_library()
    from workloads.device import DeviceRun
    run = DeviceRun(wl, **kw)
    run.step()
    import torch
    torch.cuda.synchronize()
    return run


def check_parity(wl, seqs=None, pools=True):
    ref = OracleRun(wl, seqs=seqs)
    gpu = _device_run(wl)
    # allocator results
    assert np.array_equal(gpu.ctx_slots, ref.ctx_slots)
    assert np.array_equal(gpu.new_slots, ref.new_slots)
    assert [tuple(p) for p in gpu.cow] == [tuple(p) for p in ref.cow]
    assert gpu.tables == ref.tables
    # pools, bit for bit (allocator range; the extra guard block stays NaN on both sides)
    if pools:
        for dev_pool, ref_pool in ((gpu.k_cache, ref.k_cache), (gpu.v_cache, ref.v_cache)):
            h = gpu.host(dev_pool)
            if wl.cache == "fp8":       # two planes (codes, then row exponents), compared byte for byte
                assert np.array_equal(h.reshape(-1), ref_pool.flat)
                continue
            assert h.shape == ref_pool.shape
            assert np.array_equal(h.view(np.uint8), ref_pool.view(np.uint8))
    got = gpu.out_f64()
    want = ref.out
    if seqs is not None:
        qsl = wl.query_start_loc
        rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in seqs])
        got, want = got[rows], want[rows]
    ok, max_abs, mean_abs = compare(got, want, wl.dtype)
    print(f"[parity] {wl.name}: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}", flush=True)
    assert ok, f"{wl.name}: max_abs={max_abs} mean_abs={mean_abs}"
    return gpu, ref


@pytest.mark.parametrize("name", workloads.MINI)
def test_mini_workloads(name):
    check_parity(workloads.mini(name))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_decode", "batched_decode", "mixed_superbatch", "shared_prefix_cow",
                                  "spec_verify", "batched_decode_fp8", "mixed_superbatch_fp8"])
def test_named_workloads_full_size(name):
    """Every output row against the oracle, and both whole pools byte for byte."""
    check_parity(workloads.named(name))


@pytest.mark.timeout(1200)
def test_long_context_full_size():
    """All eight 32K-128K-token sequences against the oracle (split-KV decode + merge), whole pools
    byte for byte."""
    wl = workloads.long_context_decode()
    check_parity(wl)


def _permuted_batch(wl, perm):
    """Same trace and values, super-batch order permuted: query rows, new K/V rows and the
    trace's new-row indices move with their sequences."""
    import copy
    w2 = copy.copy(wl)
    qsl = wl.query_start_loc
    w2.batch = [wl.batch[p] for p in perm]
    w2.seq_lens = wl.seq_lens[perm]
    w2.cached_lens = wl.cached_lens[perm]
    w2.query_lens = wl.query_lens[perm]
    w2.q = np.concatenate([wl.q[qsl[p]:qsl[p + 1]] for p in perm])
    w2.k_new = np.concatenate([wl.k_new[qsl[p]:qsl[p + 1]] for p in perm])
    w2.v_new = np.concatenate([wl.v_new[qsl[p]:qsl[p + 1]] for p in perm])
    start, pos = {}, 0
    for p in perm:
        start[int(qsl[p])] = pos
        pos += int(qsl[p + 1] - qsl[p])
    w2.trace = [("append_new", op[1], op[2], start[int(op[3])]) if op[0] == "append_new" else op
                for op in wl.trace]
    return w2, qsl


@pytest.mark.parametrize("mode", ["balanced", "partition"])
@pytest.mark.parametrize("name", ["decode_bf16", "mixed_bf16", "decode_f32"])
def test_bit_identical_invariances(name, mode, monkeypatch):
    """Deterministic kernels: placement, batch order and stale-slot contents change no output bit.

    The balanced decode cuts each KV head's concatenated tiles at equal
    counts, so where a sequence is cut depends on its position in the batch:
    there a reordered batch is held to the oracle tolerance instead of bits."""
    if mode == "partition":
        # single-token rows to the partitioned decode kernel, also in batches with longer rows
        monkeypatch.setenv("PA_DECODE", "partition")
        monkeypatch.setenv("PA_VERIFY", "split")
    else:
        monkeypatch.delenv("PA_DECODE", raising=False)
        monkeypatch.delenv("PA_VERIFY", raising=False)
    wl = workloads.mini(name)
    base = _device_run(wl)
    ref_bits = base.host(base.out)
    # other physical placement
    alt = np.random.default_rng(99).permutation(wl.num_blocks).astype(np.int32)
    moved = _device_run(wl, free_order=alt)
    assert moved.tables != base.tables
    assert np.array_equal(moved.host(moved.out), ref_bits)
    # zero-filled pool instead of NaN-filled: stale slots are never read
    zero = _device_run(wl, fill="zero")
    assert np.array_equal(zero.host(zero.out), ref_bits)
    # reversed super-batch order
    perm = np.arange(wl.num_seqs)[::-1]
    w2, qsl = _permuted_batch(wl, perm)
    rev = _device_run(w2)
    rev_bits = rev.host(rev.out)
    qsl2 = w2.query_start_loc
    order_exact = mode == "partition" or wl.dtype != "bf16"
    for k, p in enumerate(perm):
        a, b = rev_bits[qsl2[k]:qsl2[k + 1]], ref_bits[qsl[p]:qsl[p + 1]]
        if order_exact:
            assert np.array_equal(a, b)
        else:
            ok, max_abs, mean_abs = compare(rev.out_f64()[qsl2[k]:qsl2[k + 1]], base.out_f64()[qsl[p]:qsl[p + 1]],
                                            wl.dtype)
            assert ok, (k, max_abs, mean_abs)
    # a wider block table (more padding) changes nothing
    wide = _device_run(wl, table_stride=max(len(t) for t in base.tables) + 7)
    assert np.array_equal(wide.host(wide.out), ref_bits)


@pytest.mark.parametrize("split", ["off", "16", "64", "256", "512", "1024"])
def test_split_sizes(split, monkeypatch):
    """Every decode partition size meets the tolerance (the merge is exercised hard at 16)."""
    monkeypatch.setenv("PA_DECODE", "partition")
    monkeypatch.setenv("PA_SPLIT", split)
    check_parity(workloads.mini("decode_gqa8"), pools=False)
    check_parity(workloads.mini("decode_bf16"), pools=False)


@pytest.mark.parametrize("waves,depth", [("1", "2"), ("7", "3"), ("64", "4"), ("1024", "4"), ("2048", "2"),
                                         ("65536", "3")])
def test_balanced_wave_counts(waves, depth, monkeypatch):
    """The balanced decode meets the tolerance for any number of waves per KV head (one
    wave for everything, ragged cuts, one tile per wave, more waves than tiles) and any
    number of tiles in flight."""
    monkeypatch.delenv("PA_DECODE", raising=False)
    monkeypatch.setenv("PA_DECODE_TOTAL_WAVES", waves)
    monkeypatch.setenv("PA_DECODE_DEPTH", depth)
    for name in ("decode_gqa8", "decode_bf16", "decode_mha", "mixed_bf16", "shared_bf16"):
        check_parity(workloads.mini(name), pools=False)


VERIFY_MINIS = ("verify_bf16", "verify_gqa8", "verify_mha")


@pytest.mark.parametrize("waves", ["1", "7", "64", "1024", "65536"])
def test_multi_token_decode_wave_counts(waves, monkeypatch):
    """The multi-token decode meets the tolerance for any number of waves per KV head
    (one wave for everything, ragged cuts, one tile per wave, more waves than tiles)."""
    monkeypatch.delenv("PA_VERIFY", raising=False)
    monkeypatch.setenv("PA_VERIFY_TOTAL_WAVES", waves)
    for name in VERIFY_MINIS:
        check_parity(workloads.mini(name), pools=False)


@pytest.mark.parametrize("weight", ["500", "1000", "2000"])
def test_multi_token_decode_first_wave_weights(weight, monkeypatch):
    """fp8 decode at two waves per SIMD (2048 in all): the ranks of the waves
    dispatched first on each SIMD take `weight` tiles per 1000 of the others'
    (PA_VERIFY_FIRST_WEIGHT); any weight meets the tolerance.  16 sequences of
    1000-3000 tokens, so every rank keeps a non-empty range at each weight."""
    ensure_library()
    monkeypatch.delenv("PA_VERIFY", raising=False)
    monkeypatch.delenv("PA_VERIFY_TOTAL_WAVES", raising=False)
    monkeypatch.setenv("PA_VERIFY_FIRST_WEIGHT", weight)
    rng = np.random.default_rng(61)
    lens = rng.integers(1000, 3001, size=16)
    wl = workloads.independent("verify_fp8_weights", 61, Hq=32, Hkv=8, D=128, dtype="bf16",
                               cached=(lens - 1).tolist(), new=[1] * 16, pool_extra=2, cache_dtype="fp8")
    check_parity(wl, pools=False)


def test_multi_token_decode_routes():
    """Sequences of 2 .. 16 query tokens: column groups 1, 2 and 4 (set by the longest
    one), the cap per group size (longer sequences go to prefill in the same call),
    non-causal rows, and a batch whose longest sequence picks one column group."""
    ensure_library()
    cases = [
        ("verify_g4_cg1", dict(Hq=32, Hkv=8, cached=[40, 0, 700], new=[2, 4, 3])),
        ("verify_g4_cg2", dict(Hq=32, Hkv=8, cached=[40, 1, 2000, 17], new=[5, 8, 2, 1])),
        ("verify_g8_cap", dict(Hq=64, Hkv=8, cached=[100, 9, 300], new=[8, 9, 2])),
        ("verify_g2", dict(Hq=16, Hkv=8, cached=[64, 129, 5], new=[16, 3, 11])),
        ("verify_g1_long", dict(Hq=8, Hkv=8, cached=[3000, 16], new=[16, 17])),
    ]
    for k, (name, kw) in enumerate(cases):
        wl = workloads.independent(name, 40 + k, D=128, dtype="bf16", pool_extra=2, **kw)
        check_parity(wl, pools=False)
    wl = workloads.independent("verify_noncausal", 46, Hq=32, Hkv=8, D=128, dtype="bf16",
                               cached=[20, 500, 0], new=[6, 3, 16], pool_extra=2, causal=False)
    check_parity(wl, pools=False)


def test_multi_token_decode_against_the_prefill_route(monkeypatch):
    """PA_VERIFY=prefill sends the same sequences through the chunked-prefill kernel; both routes meet the tolerance."""
    monkeypatch.setenv("PA_VERIFY", "prefill")
    for name in VERIFY_MINIS:
        check_parity(workloads.mini(name), pools=False)


def test_single_token_rows_through_the_multi_token_kernel(monkeypatch):
    """PA_VERIFY=all sends single-token sequences through the multi-token decode kernel even in
    batches of single-token sequences only (by default those keep the single-token decode)."""
    monkeypatch.setenv("PA_VERIFY", "all")
    for name in ("decode_bf16", "decode_gqa8", "mixed_bf16", "shared_bf16") + VERIFY_MINIS:
        check_parity(workloads.mini(name), pools=False)


def test_single_token_rows_kept_apart(monkeypatch):
    """PA_VERIFY=split keeps the single-token sequences of a batch that also holds longer ones in
    the single-token decode launch (by default the multi-token launch takes them)."""
    monkeypatch.setenv("PA_VERIFY", "split")
    for name in ("mixed_bf16", "mixed_gqa8", "verify_bf16", "verify_gqa8", "verify_mha"):
        check_parity(workloads.mini(name), pools=False)


def test_multi_token_decode_invariances():
    """Placement, stale-slot contents and table padding change no output bit of the multi-token decode."""
    wl = workloads.mini("verify_bf16")
    base = _device_run(wl)
    ref_bits = base.host(base.out)
    alt = np.random.default_rng(98).permutation(wl.num_blocks).astype(np.int32)
    moved = _device_run(wl, free_order=alt)
    assert moved.tables != base.tables
    assert np.array_equal(moved.host(moved.out), ref_bits)
    zero = _device_run(wl, fill="zero")
    assert np.array_equal(zero.host(zero.out), ref_bits)
    wide = _device_run(wl, table_stride=max(len(t) for t in base.tables) + 7)
    assert np.array_equal(wide.host(wide.out), ref_bits)


@pytest.mark.parametrize("split", ["off", "64", "192", "1024"])
def test_prefill_split_sizes(split, monkeypatch):
    """Every prefill key-range split meets the tolerance (pieces merged by the prefill merge kernel)."""
    monkeypatch.setenv("PA_PREFILL_SPLIT", split)
    for name in ("mixed_bf16", "mixed_gqa8", "noncausal_bf16", "mixed_mha_d64", "mixed_fp8",
                 "prefill_fp8_gqa8_noncausal"):
        check_parity(workloads.mini(name), pools=False)


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("split", ["auto", "64"])
def test_prefill_waves_per_work_group(waves, split, monkeypatch):
    """Both prefill work-group shapes (4 waves = 128 rows, 8 waves = 256 rows) meet the tolerance,
    with and without split key ranges, whichever the host rule would pick for the batch."""
    monkeypatch.setenv("PA_PREFILL_WAVES", waves)
    if split == "auto":
        monkeypatch.delenv("PA_PREFILL_SPLIT", raising=False)
    else:
        monkeypatch.setenv("PA_PREFILL_SPLIT", split)
    for name in ("mixed_bf16", "mixed_gqa8", "noncausal_bf16", "mixed_mha_d64", "mixed_fp8"):
        check_parity(workloads.mini(name), pools=False)
    wl = workloads.independent("long_chunks", 41, Hq=32, Hkv=8, D=128, dtype="bf16",
                               cached=[0, 700, 1500], new=[300, 257, 129], pool_extra=4)
    check_parity(wl, pools=False)
    # one and two query heads per KV head: 256 rows are 256 or 128 tokens per work-group
    for seed, hq, hkv in ((42, 4, 4), (43, 8, 4)):
        wl = workloads.independent(f"chunks_g{hq // hkv}", seed, Hq=hq, Hkv=hkv, D=128, dtype="bf16",
                                   cached=[3, 0, 400, 1], new=[1, 300, 270, 2], pool_extra=4)
        check_parity(wl, pools=False)


@pytest.mark.parametrize("route", ["default", "split"])
def test_two_query_heads_per_kv_head(route, monkeypatch):
    """G = 2 on every decode path: single-token decode, multi-token decode (which takes the
    single-token rows by default and leaves them to the single-token decode under split),
    chunks, and an fp8 cache -- ragged lengths, a length-1 context, a partial last block."""
    if route == "split":
        monkeypatch.setenv("PA_VERIFY", "split")
    else:
        monkeypatch.delenv("PA_VERIFY", raising=False)
    cached = [0, 15, 16, 33, 200, 517, 1029, 3]
    check_parity(workloads.independent("g2_decode", 51, Hq=16, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[1] * len(cached), pool_extra=3))
    check_parity(workloads.independent("g2_mixed", 52, Hq=16, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[1, 3, 1, 16, 1, 40, 2, 1], pool_extra=3))
    check_parity(workloads.independent("g2_fp8", 53, Hq=16, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[1, 5, 1, 1, 30, 1, 1, 2], pool_extra=3,
                                       cache_dtype="fp8"))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.5])
def test_softmax_scales(scale, monkeypatch):
    """Scales other than 1/sqrt(D): a negative one (the prefill folds it into Q by exact sign
    flips), zero (uniform weights: the mean of the visible V rows) and a sharp one, on the
    single-token, multi-token and prefill paths and an fp8 cache."""
    monkeypatch.delenv("PA_VERIFY", raising=False)
    cached = [0, 40, 300, 1100]
    check_parity(workloads.independent("scale_decode", 61, Hq=32, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[1, 1, 1, 1], scale=scale, pool_extra=2),
                 pools=False)
    check_parity(workloads.independent("scale_mixed", 62, Hq=32, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[70, 1, 5, 200], scale=scale, pool_extra=2),
                 pools=False)
    check_parity(workloads.independent("scale_fp8", 63, Hq=32, Hkv=8, D=128, dtype="bf16",
                                       cached=cached, new=[1, 3, 90, 1], scale=scale, pool_extra=2,
                                       cache_dtype="fp8"), pools=False)
    check_parity(workloads.independent("scale_f32", 64, Hq=4, Hkv=2, D=64, dtype="f32",
                                       cached=cached, new=[1, 1, 1, 1], scale=scale, pool_extra=2),
                 pools=False)


def test_over_1024_sequences(monkeypatch):
    """Past the balanced launches' 1024 sequences the partitioned decode takes the single-token
    rows and the chunked-prefill kernel the multi-token ones (the multi-token decode is off)."""
    monkeypatch.delenv("PA_DECODE", raising=False)
    monkeypatch.delenv("PA_VERIFY", raising=False)
    rng = np.random.default_rng(71)
    S = 1100
    cached = rng.integers(0, 300, size=S)
    check_parity(workloads.independent("s1100_decode", 72, Hq=8, Hkv=2, D=128, dtype="bf16",
                                       cached=cached, new=np.ones(S, dtype=np.int64), pool_extra=4),
                 pools=False)
    new = np.ones(S, dtype=np.int64)
    new[::97] = rng.integers(2, 40, size=len(new[::97]))
    check_parity(workloads.independent("s1100_mixed", 73, Hq=8, Hkv=2, D=128, dtype="bf16",
                                       cached=cached, new=new, pool_extra=4), pools=False)


def test_degenerate_batches():
    ensure_library()
    # sequences with no query rows between others, a length-1 context, and a 1-token chunk
    wl = workloads.independent("degenerate", 31, Hq=8, Hkv=2, D=128, dtype="bf16",
                               cached=[5, 0, 33, 0, 16], new=[0, 1, 0, 2, 1], pool_extra=2)
    check_parity(wl)
    wl = workloads.independent("all_len1", 32, Hq=4, Hkv=4, D=64, dtype="f32",
                               cached=[0] * 9, new=[1] * 9)
    check_parity(wl)
    # a lone long prefill with no decode rows (G = 1, D = 128)
    wl = workloads.independent("lone_prefill", 33, Hq=2, Hkv=2, D=128, dtype="bf16",
                               cached=[300], new=[333], pool_extra=1)
    check_parity(wl)


def test_write_kv_padding_and_out_of_pool_slots():
    pa = ensure_library()
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    nb, Hkv, D = 6, 2, 64
    k = rng.standard_normal((5, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((5, Hkv, D)).astype(np.float32)
    slots = np.array([3, -1, 95, nb * 16 + 4, 17], dtype=np.int64)   # pad, last slot, beyond pool
    kc = np.zeros((nb, Hkv, 16, D), np.float32)
    vc = np.zeros_like(kc)
    keep = np.array([True, False, True, False, True])
    oracle.ref_write_kv(kc, vc, k[keep], v[keep], slots[keep], 16)
    kd = torch.zeros(kc.shape, dtype=torch.float32, device=dev)
    vd = torch.zeros_like(kd)
    pa.pa_write_kv(torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), kd, vd,
                   torch.from_numpy(slots).to(dev))
    assert np.array_equal(kd.cpu().numpy(), kc) and np.array_equal(vd.cpu().numpy(), vc)
    # zero tokens is a no-op
    pa.pa_write_kv(torch.empty((0, Hkv, D), device=dev), torch.empty((0, Hkv, D), device=dev), kd, vd,
                   torch.empty((0,), dtype=torch.int64, device=dev))
    assert np.array_equal(kd.cpu().numpy(), kc)


def test_copy_blocks_bit_exact():
    pa = ensure_library()
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(6)
    kc = rng.integers(0, 2**16, size=(9, 8, 16, 128), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(9, 8, 16, 128), dtype=np.uint16)
    pairs = [(1, 4), (2, 7), (8, 0)]
    kd = torch.from_numpy(kc.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(vc.view(np.int16)).to(dev).view(torch.bfloat16)
    pa.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device=dev))
    oracle.ref_copy_blocks(kc, vc, pairs)
    assert np.array_equal(kd.view(torch.int16).cpu().numpy().view(np.uint16), kc)
    assert np.array_equal(vd.view(torch.int16).cpu().numpy().view(np.uint16), vc)


def test_error_paths(monkeypatch):
    pa = ensure_library()
    import torch
    from workloads.device import DeviceRun
    wl = workloads.mini("decode_bf16")
    run = DeviceRun(wl)
    run.step_writes()
    # workspace smaller than required
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pa_forward(run.out, run.q, run.k_cache, run.v_cache, run.block_tables, run.seq_lens, run.qsl,
                      run.cached_lens, wl.max_seq_len, 1, wl.scale, True,
                      workspace=torch.empty(16, dtype=torch.uint8, device=run.dev))
    assert e.value.status == pa.PA_ERR_ARG
    # check mode catches metadata violations before launching
    monkeypatch.setenv("PA_CHECK", "1")
    bad = run.block_tables.clone()
    bad[0, 0] = wl.pool_blocks + 5
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pa_forward(run.out, run.q, run.k_cache, run.v_cache, bad, run.seq_lens, run.qsl,
                      run.cached_lens, wl.max_seq_len, 1, wl.scale, True, workspace=run.workspace)
    assert e.value.status == pa.PA_ERR_RANGE
    with pytest.raises(pa.PagedAttnError) as e:   # max_seq_len below a real length
        pa.pa_forward(run.out, run.q, run.k_cache, run.v_cache, run.block_tables, run.seq_lens, run.qsl,
                      run.cached_lens, 3, 1, wl.scale, True, workspace=run.workspace)
    assert e.value.status == pa.PA_ERR_RANGE
    dup = torch.tensor([7, 7], dtype=torch.int64, device=run.dev)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pa_write_kv(run.k_new[:2], run.v_new[:2], run.k_cache, run.v_cache, dup)
    assert e.value.status == pa.PA_ERR_RANGE
    # the valid call still passes in check mode
    run.forward()
    torch.cuda.synchronize()
    # without check mode an out-of-range table entry is clamped: finite output, no fault
    monkeypatch.setenv("PA_CHECK", "0")
    pa.pa_forward(run.out, run.q, run.k_cache, run.v_cache, bad, run.seq_lens, run.qsl,
                  run.cached_lens, wl.max_seq_len, 1, wl.scale, True, workspace=run.workspace)
    torch.cuda.synchronize()


# -- quantised (fp8) cache ------------------------------------------------------

FP8_MINIS = ("decode_fp8", "verify_fp8", "fp8_gqa8", "fp8_mha_noncausal", "mixed_fp8")


def test_fp8_write_edge_rows():
    """Quantised write, bit for bit against the oracle: zero rows, -0, bf16 subnormals, the
    largest bf16 values, exact rounding ties, NaN and infinite elements, padding and
    out-of-pool slots."""
    pa = ensure_library()
    import torch
    from helpers import _write_fp8
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    NB, Hkv, D, B = 5, 2, 128, 16
    rows = [np.zeros(D), -np.zeros(D), np.full(D, 2.0 ** -130), np.linspace(-3e38, 3e38, D),
            np.concatenate([[448.0], 1 + np.arange(1, D) / 16.0 * 0.0625]),        # amax 448: ties at 1/16 steps
            np.concatenate([[1.0], np.full(D - 1, 1 + 1 / 16)]),
            np.concatenate([[2.0 ** -120], np.full(D - 1, 3 * 2.0 ** -130)]),
            rng.standard_normal(D) * 1e-3, rng.standard_normal(D) * 1e3,
            # non-finite elements: the NaN code with their sign, the scale from the finite ones
            np.concatenate([[np.nan, np.inf, -np.inf], rng.standard_normal(D - 3) * 5.0]),
            np.full(D, np.inf)]
    T = len(rows)
    x = np.stack(rows)[:, None, :].repeat(Hkv, axis=1)
    x[:, 1] *= -0.75
    k = workloads.bf16_bits(x.astype(np.float32))
    v = workloads.bf16_bits((x[:, :, ::-1] * 0.5).astype(np.float32))
    slots = np.array([3, -1, 17, 79, 40, NB * B + 2, 65, 0, 50, 22, 33], dtype=np.int64)
    kp = oracle.fp8_pool(NB, Hkv, D)
    vp = oracle.fp8_pool(NB, Hkv, D)
    keep = slots < NB * B
    _write_fp8(kp, vp, k[keep], v[keep], slots[keep], B)
    kd = torch.full(pa.fp8_pool_shape(NB, Hkv, D), 0xFF, dtype=torch.uint8, device=dev)
    vd = torch.full_like(kd, 0xFF)
    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    pa.pa_write_kv(dev_bf16(k), dev_bf16(v), kd, vd, torch.from_numpy(slots).to(dev))
    assert np.array_equal(kd.cpu().numpy().reshape(-1), kp.flat)
    assert np.array_equal(vd.cpu().numpy().reshape(-1), vp.flat)


def test_fp8_copy_blocks_bit_exact():
    pa = ensure_library()
    import torch
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(8)
    kc, vc = oracle.fp8_pool(9, 8, 128), oracle.fp8_pool(9, 8, 128)
    kc.flat[:] = rng.integers(0, 256, size=kc.flat.shape, dtype=np.uint8)
    vc.flat[:] = rng.integers(0, 256, size=vc.flat.shape, dtype=np.uint8)
    pairs = [(1, 4), (2, 7), (8, 0)]
    shape = pa.fp8_pool_shape(9, 8, 128)
    kd = torch.from_numpy(kc.flat.reshape(shape).copy()).to(dev)
    vd = torch.from_numpy(vc.flat.reshape(shape).copy()).to(dev)
    pa.pa_copy_blocks(kd, vd, torch.tensor(pairs, dtype=torch.int32, device=dev))
    oracle.ref_copy_blocks(kc, vc, pairs)
    assert np.array_equal(kd.cpu().numpy().reshape(-1), kc.flat)
    assert np.array_equal(vd.cpu().numpy().reshape(-1), vc.flat)


@pytest.mark.parametrize("waves,depth", [("1", "5"), ("7", "3"), ("1024", "5"), ("65536", "3")])
def test_fp8_wave_counts_and_depths(waves, depth, monkeypatch):
    monkeypatch.setenv("PA_VERIFY_TOTAL_WAVES", waves)
    monkeypatch.setenv("PA_VERIFY_DEPTH", depth)
    for name in FP8_MINIS:
        check_parity(workloads.mini(name), pools=False)


def test_fp8_invariances():
    """Placement, stale bytes (0xff codes and scales vs zeros) and table padding change no output bit."""
    wl = workloads.mini("verify_fp8")
    base = _device_run(wl)
    ref_bits = base.host(base.out)
    alt = np.random.default_rng(97).permutation(wl.num_blocks).astype(np.int32)
    moved = _device_run(wl, free_order=alt)
    assert moved.tables != base.tables
    assert np.array_equal(moved.host(moved.out), ref_bits)
    zero = _device_run(wl, fill="zero")
    assert np.array_equal(zero.host(zero.out), ref_bits)
    wide = _device_run(wl, table_stride=max(len(t) for t in base.tables) + 7)
    assert np.array_equal(wide.host(wide.out), ref_bits)


def test_fp8_unsupported_shapes():
    """fp8 caches are built for head_dim 128 only: other shapes are refused before any launch."""
    pa = ensure_library()
    import ctypes
    desc64 = pa.CacheDesc(100, 8, 64, 16, pa.PA_FP8)
    assert pa.lib.pa_forward_workspace_size(4, 600, 32, 4096, 512, ctypes.byref(desc64)) == 0
    st = pa.lib.pa_forward(None, None, None, None, None, 1, None, None, None, 4, 600, 32, 4096, 512,
                           ctypes.byref(desc64), 0.1, 1, None, 0, None)
    assert st == pa.PA_ERR_UNSUPPORTED and "fp8" in pa.lib.pa_last_error().decode()
    st = pa.lib.pa_write_kv(None, None, None, None, None, 4, ctypes.byref(desc64), None)
    assert st == pa.PA_ERR_UNSUPPORTED
