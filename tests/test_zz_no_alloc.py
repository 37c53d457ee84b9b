"""pa_forward_noalloc: pa_forward without a workspace, for callers that cannot allocate.

Its scratch is the library's own per-GPU device array.  Through the C ABI, on
consecutive calls (each later one with a smaller batch, so stale contents of
the array from the previous call are present), its output must equal
pa_forward's with a caller workspace bit for bit -- the same kernels on the
same inputs -- and meet the oracle's tolerance.  A batch needing more scratch
than the array holds is refused before anything is enqueued.
"""

import numpy as np
import pytest

import workloads
from helpers import OracleRun, compare, ensure_library

pytestmark = pytest.mark.gpu


def _prepared(name):
    ensure_library()
    import torch
    from workloads.device import DeviceRun
    run = DeviceRun(workloads.mini(name))
    run.step_writes()
    torch.cuda.synchronize()
    return run


def _noalloc(run):
    import paged_kv_cache_forward_amd as pa
    wl = run.wl
    pa.pa_forward_noalloc(run.out, run.q, run.k_cache, run.v_cache, run.block_tables, run.seq_lens, run.qsl,
                          run.cached_lens, run.max_seq_len, wl.max_query_len, wl.scale, wl.causal)


@pytest.mark.parametrize("first,second", [("mixed_bf16", "decode_bf16"), ("mixed_fp8", "decode_fp8"),
                                          ("decode_gqa8", "decode_f32")])
def test_noalloc_matches_pa_forward(first, second, monkeypatch):
    import torch
    import paged_kv_cache_forward_amd as pa
    for k in ("PA_CHECK", "PA_DECODE", "PA_VERIFY"):
        monkeypatch.delenv(k, raising=False)
    runs = [_prepared(first), _prepared(second)]
    wss = [pa.pa_forward_workspace_size(r.wl.num_seqs, r.wl.num_tokens, r.wl.num_q_heads, r.max_seq_len,
                                        r.wl.max_query_len, r.k_cache) for r in runs]
    assert 0 < wss[1] < wss[0] <= pa.NOALLOC_MAX_SCRATCH
    for run in runs:                      # two calls in a row, the second with the smaller batch
        run.forward()                     # pa_forward with its own workspace
        torch.cuda.synchronize()
        want = run.host(run.out).copy()
        run.out.fill_(float("nan"))
        torch.cuda.synchronize()
        _noalloc(run)
        torch.cuda.synchronize()
        got = run.host(run.out)
        assert np.array_equal(got, want), f"{run.wl.name}: pa_forward_noalloc differs from pa_forward"
        ok, max_abs, mean_abs = compare(run.out_f64(), OracleRun(run.wl).out, run.wl.dtype)
        assert ok, (run.wl.name, max_abs, mean_abs)


def test_noalloc_refuses_batches_beyond_its_scratch():
    import torch
    import paged_kv_cache_forward_amd as pa
    run = _prepared("decode_bf16")
    wl = run.wl
    # 65536 single-token sequences of up to 8192 tokens: the partitioned decode's partials exceed the array.
    S, L = 65536, 8192
    need = pa.pa_forward_workspace_size(S, S, wl.num_q_heads, L, 1, run.k_cache)
    assert need > pa.NOALLOC_MAX_SCRATCH
    dev = run.dev
    bt = torch.zeros((S, 1), dtype=torch.int32, device=dev)
    lens = torch.ones(S, dtype=torch.int32, device=dev)
    qsl = torch.arange(S + 1, dtype=torch.int32, device=dev)
    q = torch.zeros((S, wl.num_q_heads, wl.head_dim), dtype=run.q.dtype, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pa_forward_noalloc(out, q, run.k_cache, run.v_cache, bt, lens, qsl, lens - 1, L, 1, wl.scale, True)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    # the library still works afterwards
    _noalloc(run)
    torch.cuda.synchronize()
    ok, max_abs, mean_abs = compare(run.out_f64(), OracleRun(wl).out, wl.dtype)
    assert ok, (max_abs, mean_abs)
