"""pa_write_kv_forward: the step's cache write fused into the decode.

"Was ändert PagedAttention an der KV-Speicherzuweisung für LLMs?"
(slavadubrov.com), lead paragraph, and "Внутреннее устройство vLLM"
(artificials.ru), forward-pass paragraph: a step stores its new tokens' keys
and values in their slots, then attends over the cache.  The fused call must
leave the same bytes in both pools and the same output bits as pa_write_kv
followed by pa_forward, on every decode route (balanced at every depth and
wave count, the partitioned vector kernel, and the routes that do not fuse),
on every dtype and head grouping, with the new token on the first, a middle
and the last row of its block, at full size, and the output must meet the
oracle.  pa_write_kv_forward_shared is held to the same bar against
pa_write_kv + pa_forward_shared.  Check mode refuses a slot that is not the
sequence's last position.
"""

import numpy as np
import pytest

import workloads
from helpers import OracleRun, compare, ensure_library

pytestmark = pytest.mark.gpu


def _pair(wl, **kw):
    """(fused run, separate run) after one step each."""
    ensure_library()
    import torch
    from workloads.device import DeviceRun
    a = DeviceRun(wl, fused=True, **kw)
    a.step()
    b = DeviceRun(wl, fused=False, **kw)
    b.step()
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    for x, y, part in ((a.out, b.out, "out"), (a.k_cache, b.k_cache, "k pool"), (a.v_cache, b.v_cache, "v pool")):
        hx, hy = a.host(x), b.host(y)
        assert np.array_equal(hx.view(np.uint8), hy.view(np.uint8)), f"{what}: {part} differs"


def _oracle(run):
    wl = run.wl
    ok, max_abs, mean_abs = compare(run.out_f64(), OracleRun(wl).out, wl.dtype)
    print(f"[parity] {wl.name} fused: max_abs={max_abs:.3e} mean_abs={mean_abs:.3e}", flush=True)
    assert ok, (wl.name, max_abs, mean_abs)


ROUTES = {
    "default": {},
    "valu": {"PA_DECODE": "valu"},
    "valu_split64": {"PA_DECODE": "valu", "PA_SPLIT": "64"},
    "partition": {"PA_DECODE": "partition"},
    "depth3": {"PA_DECODE_DEPTH": "3"},
    "depth4": {"PA_DECODE_DEPTH": "4"},
    "waves1": {"PA_DECODE_TOTAL_WAVES": "1"},
    "waves7": {"PA_DECODE_TOTAL_WAVES": "7"},
    "waves65536": {"PA_DECODE_TOTAL_WAVES": "65536"},
}
KNOBS = ["PA_DECODE", "PA_SPLIT", "PA_DECODE_DEPTH", "PA_DECODE_TOTAL_WAVES", "PA_VERIFY", "PA_CHECK"]


def _route(monkeypatch, route):
    for k in KNOBS:
        monkeypatch.delenv(k, raising=False)
    for k, v in ROUTES[route].items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("name", ["decode_bf16", "decode_gqa8", "decode_mha", "decode_f32", "decode_d64_bf16",
                                  "shared_bf16"])
def test_fused_equals_separate(name, route, monkeypatch):
    _route(monkeypatch, route)
    a, b = _pair(workloads.mini(name))
    _same(a, b, f"{name}/{route}")
    _oracle(a)


@pytest.mark.parametrize("name", ["mixed_bf16", "verify_bf16", "decode_fp8", "noncausal_bf16", "prefill_f32"])
def test_batches_that_do_not_fuse(name, monkeypatch):
    """Chunks, multi-token rows and an fp8 cache run the two calls: the same bits."""
    _route(monkeypatch, "default")
    a, b = _pair(workloads.mini(name))
    _same(a, b, name)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_new_token_on_every_row_of_its_block(G, monkeypatch):
    """Contexts putting the new token on row 0 (a fresh block), 1, 7, 14 and 15, and a one-token sequence."""
    Hq, Hkv = {1: (8, 8), 2: (8, 4), 4: (16, 4), 8: (32, 4)}[G]
    cached = [0, 16, 17, 23, 30, 31, 47, 64, 1000, 1023, 4095, 4096]
    wl = workloads.independent(f"rows_g{G}", 600 + G, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", cached=cached,
                               new=[1] * len(cached), pool_extra=2)
    for route in ("default", "valu", "waves7"):
        _route(monkeypatch, route)
        a, b = _pair(wl)
        _same(a, b, f"rows_g{G}/{route}")
        _oracle(a)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["batched_decode", "long_context_decode", "tiny_decode"])
def test_full_size(name, monkeypatch):
    _route(monkeypatch, "default")
    wl = workloads.named(name)
    a, b = _pair(wl)
    _same(a, b, name)
    if name != "long_context_decode":      # the long-context oracle is the parity suite's (minutes on the CPU)
        _oracle(a)


def test_check_mode_refuses_a_wrong_slot(monkeypatch):
    import torch
    import paged_kv_cache_forward_amd as pa
    _route(monkeypatch, "default")
    ensure_library()
    from workloads.device import DeviceRun
    wl = workloads.mini("decode_bf16")
    run = DeviceRun(wl)
    monkeypatch.setenv("PA_CHECK", "1")
    run.step()                                     # the true slots pass
    torch.cuda.synchronize()
    good = run.new_slots_d.clone()
    for bad in (good.flip(0), good + 1):
        if torch.equal(bad, good):
            continue
        run.new_slots_d.copy_(bad)
        with pytest.raises(pa.PagedAttnError) as e:
            run.step()
        assert e.value.status == pa.PA_ERR_RANGE
    run.new_slots_d.copy_(good)


HEADS = {1: (4, 4), 2: (8, 4), 4: (32, 8), 8: (64, 8)}     # G -> (Hq, Hkv)
TREE = [(0, 300)] * 5 + [(1, 250), (0, 17), (0, 0), (0, 0), (8, 0), (0, 160), (0, 160)]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_shared_fused_equals_separate(G, monkeypatch):
    """Fork trees (shared prefixes, copy-on-write) through the shared-prefix decode."""
    for key in ("PA_SHARED_TOTAL_WAVES", "PA_SHARED_CG", "PA_CHECK"):
        monkeypatch.delenv(key, raising=False)
    Hq, Hkv = HEADS[G]
    wl = workloads.fork_tree(f"tree_g{G}", 500 + G, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", root=304, forks=TREE,
                             suffix_max=40)
    for waves in (None, "7", "65536"):
        if waves is None:
            monkeypatch.delenv("PA_SHARED_TOTAL_WAVES", raising=False)
        else:
            monkeypatch.setenv("PA_SHARED_TOTAL_WAVES", waves)
        a, b = _pair(wl, shared=True)
        assert a.shared_blocks.max() > 0 and a.cow
        _same(a, b, f"tree_g{G}/{waves}")
        _oracle(a)


def test_shared_fused_minis_and_other_batches(monkeypatch):
    """The shared mini and CG = 4; batches the shared decode does not take run the two calls."""
    for key in ("PA_SHARED_TOTAL_WAVES", "PA_SHARED_CG", "PA_CHECK"):
        monkeypatch.delenv(key, raising=False)
    a, b = _pair(workloads.mini("shared_bf16"), shared=True)
    _same(a, b, "shared_bf16")
    _oracle(a)
    monkeypatch.setenv("PA_SHARED_CG", "4")
    a, b = _pair(workloads.mini("shared_bf16"), shared=True)
    _same(a, b, "shared_bf16/cg4")
    monkeypatch.delenv("PA_SHARED_CG")
    for name in ("mixed_bf16", "decode_fp8", "decode_f32", "verify_bf16"):
        a, b = _pair(workloads.mini(name), shared=True)
        _same(a, b, name)


@pytest.mark.timeout(900)
def test_shared_fused_full_size(monkeypatch):
    for key in ("PA_SHARED_TOTAL_WAVES", "PA_SHARED_CG", "PA_CHECK"):
        monkeypatch.delenv(key, raising=False)
    a, b = _pair(workloads.shared_prefix_cow(), shared=True)
    _same(a, b, "shared_prefix_cow")
    _oracle(a)


def test_shared_check_mode_refuses_a_wrong_slot(monkeypatch):
    import torch
    import paged_kv_cache_forward_amd as pa
    for key in ("PA_SHARED_TOTAL_WAVES", "PA_SHARED_CG"):
        monkeypatch.delenv(key, raising=False)
    ensure_library()
    from workloads.device import DeviceRun
    run = DeviceRun(workloads.mini("shared_bf16"), shared=True)
    monkeypatch.setenv("PA_CHECK", "1")
    run.step()                                     # the true slots pass
    torch.cuda.synchronize()
    good = run.new_slots_d.clone()
    run.new_slots_d.copy_(good.flip(0))
    with pytest.raises(pa.PagedAttnError) as e:
        run.step()
    assert e.value.status == pa.PA_ERR_RANGE
    run.new_slots_d.copy_(good)


@pytest.mark.parametrize("seed", range(6))
def test_random_batches(seed, monkeypatch):
    """Random single-token batches (lengths 1..3000, any group size, 1..80 sequences) on the default
    route and the vector kernel: the fused call gives the two calls' bits."""
    rng = np.random.default_rng(7000 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 81))
    cached = rng.integers(0, 3000, size=S).tolist()
    wl = workloads.independent(f"random_{seed}", 7100 + seed, Hq=G * Hkv, Hkv=Hkv, D=128, dtype="bf16",
                               cached=cached, new=[1] * S, pool_extra=3)
    for route in ("default", "valu", "waves7"):
        _route(monkeypatch, route)
        a, b = _pair(wl)
        _same(a, b, f"random_{seed}/G{G}/Hkv{Hkv}/S{S}/{route}")
    _oracle(a)
