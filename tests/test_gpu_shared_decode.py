"""pa_forward_shared: the shared-prefix decode against the oracle.

"Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
(slavadubrov.com), section "Gemeinsame Nutzung erfordert mehr als
Speicherzuweisung": forked requests point at the same blocks.  The library
reads each block a group of sequences shares once for the whole group; the
result must be the attention each sequence's query has over its own tokens --
the oracle's, within the stated tolerance -- whatever the sharing the caller
reports (the allocator's count, less than it, none), on every group size
(query heads per KV head 1, 2, 4, 8), on fork trees with copy-on-write, at
full size, with any number of waves, and bit for bit the same under another
physical placement.  Batches the shared decode does not take run pa_forward's
paths unchanged.  Check mode refuses an over-reported sharing.
"""

import numpy as np
import pytest

import workloads
from helpers import OracleRun, compare, ensure_library

pytestmark = pytest.mark.gpu

TREE = [(0, 300)] * 5 + [(1, 250), (0, 17), (0, 0), (0, 0), (8, 0), (0, 160), (0, 160)]


HEADS = {1: (4, 4), 2: (8, 4), 4: (32, 8), 8: (64, 8)}     # G -> (Hq, Hkv)


def _tree(G, seed, forks=TREE, root=304, suffix_max=40):
    Hq, Hkv = HEADS[G]
    return workloads.fork_tree(f"tree_g{G}", seed, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", root=root,
                               forks=forks, suffix_max=suffix_max)


def _run(wl, **kw):
    ensure_library()
    import torch
    from workloads.device import DeviceRun
    run = DeviceRun(wl, shared=True, **kw)
    run.step()
    torch.cuda.synchronize()
    return run


def _check(run, ref=None):
    wl = run.wl
    want = OracleRun(wl).out if ref is None else ref
    ok, max_abs, mean_abs = compare(run.out_f64(), want, wl.dtype)
    print(f"[parity] {wl.name} shared: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}", flush=True)
    assert ok, (wl.name, max_abs, mean_abs)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fork_tree_every_group_size(G, monkeypatch):
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    wl = _tree(G, 400 + G)
    run = _run(wl)
    assert run.shared_blocks.max() > 0 and run.cow
    _check(run)


def test_fan_out_minis(monkeypatch):
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    _check(_run(workloads.mini("shared_bf16")))
    # a long shared prefix, many members per group, ragged private suffixes
    wl = workloads.shared_prefix("fan_out_40", 411, Hq=32, Hkv=8, D=128, dtype="bf16", num_seqs=40,
                                 prefix=1008, suffix_max=300, num_blocks=3000)
    _check(_run(wl))


def test_under_reported_sharing(monkeypatch):
    """Fewer shared blocks than the allocator's count (half, none) share less and change nothing else."""
    import torch
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    wl = _tree(4, 421)
    ref = OracleRun(wl).out
    run = _run(wl)
    full = run.host(run.out).copy()
    for scale in (0.5, 0.0):
        run.shared_blocks_d.copy_(torch.from_numpy((run.shared_blocks * scale).astype(np.int32)))
        run.out.fill_(float("nan"))
        run.forward()
        torch.cuda.synchronize()
        _check(run, ref)
    run.shared_blocks_d.copy_(torch.from_numpy(run.shared_blocks))
    run.forward()
    torch.cuda.synchronize()
    assert np.array_equal(run.host(run.out), full)             # deterministic


@pytest.mark.parametrize("waves", ["1", "7", "64", "1024", "65536"])
def test_wave_counts(waves, monkeypatch):
    monkeypatch.setenv("PA_SHARED_TOTAL_WAVES", waves)
    _check(_run(_tree(4, 431)))
    _check(_run(_tree(8, 432)))


def test_placement_invariance(monkeypatch):
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    wl = _tree(4, 441)
    a = _run(wl)
    b = _run(wl, free_order=np.random.default_rng(5).permutation(wl.num_blocks).astype(np.int32))
    assert a.tables != b.tables
    assert np.array_equal(a.host(a.out), b.host(b.out))


@pytest.mark.timeout(900)
def test_shared_prefix_cow_full_size(monkeypatch):
    """256 sequences on one 2048-token prefix (refcount 256), one diverging inside the last shared block."""
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    wl = workloads.shared_prefix_cow()
    run = _run(wl)
    assert int(run.shared_blocks[1:].min()) >= 127
    _check(run)


def test_other_batches_take_pa_forward(monkeypatch):
    """A batch with chunks, an fp8 cache, fp32: pa_forward_shared gives pa_forward's bits."""
    import torch
    monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
    from workloads.device import DeviceRun
    ensure_library()
    for name in ("mixed_bf16", "decode_fp8", "decode_f32", "verify_bf16"):
        wl = workloads.mini(name)
        a = DeviceRun(wl)
        a.step()
        b = DeviceRun(wl, shared=True)
        b.step()
        torch.cuda.synchronize()
        assert np.array_equal(a.host(a.out), b.host(b.out)), name


def test_check_mode_refuses_over_reported_sharing(monkeypatch):
    import torch
    import paged_kv_cache_forward_amd as pa
    wl = _tree(4, 451)
    run = _run(wl)
    monkeypatch.setenv("PA_CHECK", "1")
    run.forward()                                    # the true counts pass
    torch.cuda.synchronize()
    bad = run.shared_blocks.copy()
    i = int(np.argmax(bad))
    bad[i] += 1
    run.shared_blocks_d.copy_(torch.from_numpy(bad))
    with pytest.raises(pa.PagedAttnError) as e:
        run.forward()
    assert e.value.status == pa.PA_ERR_RANGE
