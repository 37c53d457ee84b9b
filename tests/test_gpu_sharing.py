"""Shared blocks and copy-on-write on the GPU: bit identities.

"Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
(slavadubrov.com), section "Gemeinsame Nutzung erfordert mehr als
Speicherzuweisung": requests may share physical blocks, and sharing must not
change or corrupt what any of them reads.  "PagedAttention et vLLM"
(aiunderstanding.org), FAQ on sharing: a shared block is copied only when a
branch diverges.

  * A batch whose sequences share their prefix blocks gives, bit for bit, the
    output of the same batch built with private copies of every row (same
    lengths, same batch order, other physical blocks): the kernels gather a
    sequence's tokens through its own table, and nothing else about the
    placement reaches the arithmetic.
  * The step's copy-on-write (the diverging sequence's block copied, then its
    token written into the copy) leaves every other sequence's output bits,
    and the shared block's bytes, as they were before it.
"""

import numpy as np
import pytest

import workloads
from helpers import OracleRun, compare, ensure_library

pytestmark = pytest.mark.gpu

ROUTES = {
    "default": {},
    "partition": {"PA_DECODE": "partition"},
    "multi_token": {"PA_VERIFY": "all"},
}


def _device(wl):
    ensure_library()
    import torch
    from workloads.device import DeviceRun
    run = DeviceRun(wl)
    torch.cuda.synchronize()
    return run


def _set_route(monkeypatch, route):
    for k in ("PA_DECODE", "PA_VERIFY", "PA_DECODE_TOTAL_WAVES", "PA_DECODE_DEPTH"):
        monkeypatch.delenv(k, raising=False)
    for k, v in ROUTES[route].items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("route", list(ROUTES))
def test_shared_prefix_equals_private_copies_mini(route, monkeypatch):
    import torch
    _set_route(monkeypatch, route)
    wl = workloads.mini("shared_bf16")
    priv = workloads.unshared(wl)
    a, b = _device(wl), _device(priv)
    assert a.cow and not b.cow                       # only the shared batch copies a block
    a.step()
    b.step()
    torch.cuda.synchronize()
    assert set(sum(a.tables, [])) != set(sum(b.tables, []))
    assert np.array_equal(a.host(a.out), b.host(b.out))
    ok, max_abs, mean_abs = compare(a.out_f64(), OracleRun(wl).out, wl.dtype)
    assert ok, (max_abs, mean_abs)


@pytest.mark.timeout(900)
def test_shared_prefix_equals_private_copies_full_size(monkeypatch):
    """256 sequences on one 2048-token prefix (refcount 256) against 256 private copies."""
    import torch
    _set_route(monkeypatch, "default")
    wl = workloads.shared_prefix_cow()
    priv = workloads.unshared(wl)
    a = _device(wl)
    a.step()
    torch.cuda.synchronize()
    shared_bits = a.host(a.out).copy()
    del a
    torch.cuda.empty_cache()
    b = _device(priv)
    assert not b.cow
    b.step()
    torch.cuda.synchronize()
    assert np.array_equal(shared_bits, b.host(b.out))


def _cow_before_after(wl):
    """Output bits of every sequence but the diverging one, before and after the step's copy-on-write.

    Before: the other sequences' new tokens are written and the diverging
    sequence still reads the shared block through its pre-copy table (its own
    new token not written).  After: the step itself -- pa_copy_blocks, every
    new token written, attention with the post-copy tables.  Lengths and batch
    order are the same, so every other sequence's output must keep its bits.
    """
    import torch
    import paged_kv_cache_forward_amd as pa
    run = _device(wl)
    assert len(run.cow) == 1
    src, dst = run.cow[0]
    d = wl.num_seqs - 1                               # the diverging sequence (the builder's last)
    assert dst in run.tables[d] and src not in run.tables[d]
    assert all(src in t for t in run.tables[:d])
    assert list(wl.query_lens) == [1] * wl.num_seqs   # row i is sequence i's one query token
    slots = run.new_slots.copy()
    slots[d] = -1
    bt = run.block_tables.clone()
    row = bt[d]
    row[row == dst] = src
    shared_k = run.host(run.k_cache[src]).copy()
    shared_v = run.host(run.v_cache[src]).copy()
    pa.pa_write_kv(run.k_new, run.v_new, run.k_cache, run.v_cache, torch.from_numpy(slots).to(run.dev))
    pa.pa_forward(run.out, run.q, run.k_cache, run.v_cache, bt, run.seq_lens, run.qsl, run.cached_lens,
                  wl.max_seq_len, wl.max_query_len, wl.scale, wl.causal, workspace=run.workspace)
    torch.cuda.synchronize()
    before = run.host(run.out).copy()
    run.out.fill_(float("nan"))
    run.step()
    torch.cuda.synchronize()
    after = run.host(run.out)
    assert np.array_equal(run.host(run.k_cache[src]), shared_k)
    assert np.array_equal(run.host(run.v_cache[src]), shared_v)
    assert np.array_equal(before[:d], after[:d])
    assert not np.array_equal(before[d], after[d])    # the diverging sequence now reads its own token
    return run


@pytest.mark.parametrize("route", list(ROUTES))
def test_copy_on_write_keeps_other_outputs_mini(route, monkeypatch):
    _set_route(monkeypatch, route)
    wl = workloads.mini("shared_bf16")
    run = _cow_before_after(wl)
    ok, max_abs, mean_abs = compare(run.out_f64(), OracleRun(wl).out, wl.dtype)
    assert ok, (max_abs, mean_abs)


@pytest.mark.timeout(900)
def test_copy_on_write_keeps_other_outputs_full_size(monkeypatch):
    """The 255 sequences that do not diverge keep their output bits across the step's block copy."""
    _set_route(monkeypatch, "default")
    _cow_before_after(workloads.shared_prefix_cow())
