"""HIP-graph capture of a serving step (pa_copy_blocks + pa_write_kv_forward).

"Внутреннее устройство vLLM" (artificials.ru), forward-pass paragraph: the
step's kernels are captured once and replayed as a graph.  The step is
captured with torch.cuda.graph on a side stream and replayed several times,
with the program's own eager work and synchronisations between replays; every
replay must give the eager step's output bits and meet the oracle's tolerance.
A replay after the query rows are changed in place must give the eager result
for the new queries (the captured calls read device inputs at replay time).
A replay after every sequence has grown by one token -- new slots, new block
table entries, longer seq_lens, new K/V rows and queries, all written in place
within the captured sizes -- must give the eager result and the oracle's
attention over the grown sequences.  Check mode, which synchronises, must
refuse to run under capture.
"""

import numpy as np
import pytest

import workloads
from helpers import OracleRun, compare, ensure_library, logical_rows, oracle_from_rows

pytestmark = pytest.mark.gpu


def _run(name, **kw):
    ensure_library()
    from workloads.device import DeviceRun
    import torch
    run = DeviceRun(workloads.mini(name), **kw)
    torch.cuda.synchronize()
    return run


def _check_oracle(run, want, tag):
    ok, max_abs, mean_abs = compare(run.out_f64(), want, run.wl.dtype)
    assert ok, f"{tag}: max_abs={max_abs} mean_abs={mean_abs}"


@pytest.mark.parametrize("name", ["decode_bf16", "decode_gqa8", "mixed_bf16", "shared_bf16", "decode_f32",
                                  "verify_bf16", "decode_fp8", "verify_fp8"])
def test_graph_replay_matches_eager(name, monkeypatch):
    import torch
    monkeypatch.delenv("PA_CHECK", raising=False)
    run = _run(name)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.step()                       # eager step (also warms the library up)
    torch.cuda.synchronize()
    want = run.host(run.out).copy()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run.step()
    torch.cuda.synchronize()
    ref = OracleRun(run.wl).out
    for rep in range(3):
        run.out.fill_(float("nan"))      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.host(run.out)
        assert np.array_equal(got, want), f"{name}: replay {rep} differs from the eager step"
        _check_oracle(run, ref, f"{name} replay {rep}")

    # New query rows, same shapes: the replay reads them.
    perm = np.random.default_rng(5).permutation(run.q.shape[0])
    run.q.copy_(run.q[torch.from_numpy(perm).to(run.q.device)].clone())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        run.step()
    torch.cuda.synchronize()
    want2 = run.host(run.out).copy()
    assert not np.array_equal(want2, want)
    run.out.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(run.host(run.out), want2), f"{name}: replay with new queries differs"


@pytest.mark.parametrize("name", ["decode_bf16", "decode_gqa8", "decode_f32", "shared_bf16", "decode_fp8"])
def test_graph_replay_after_sequences_grow(name, monkeypatch):
    """Capture a decode step with room for one more token per sequence, then replay it for the next
    step: each sequence's next slot comes from the library's allocator, its new block (if any) goes
    into the device block table, lengths grow by one, new K/V rows and queries are copied in."""
    import torch
    monkeypatch.delenv("PA_CHECK", raising=False)
    wl = workloads.mini(name)
    assert list(wl.query_lens) == [1] * wl.num_seqs
    width = max(-(-(int(L) + 1) // wl.block_size) for L in wl.seq_lens)
    run = _run(name, table_stride=width, max_seq_len=wl.max_seq_len + 1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.step()
    torch.cuda.synchronize()
    _check_oracle(run, OracleRun(wl).out, f"{name} eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run.step()
    torch.cuda.synchronize()

    # The next step: one more token per sequence.
    rng = np.random.Generator(np.random.PCG64(wl.seed + 500))
    S, B = wl.num_seqs, wl.block_size
    k2 = workloads._normal(rng, wl.k_new.shape, wl.dtype)
    v2 = workloads._normal(rng, wl.v_new.shape, wl.dtype)
    q2 = workloads._normal(rng, wl.q.shape, wl.dtype)
    slots = np.empty(S, dtype=np.int64)
    bt = run.block_tables.cpu().numpy()
    for i, h in enumerate(wl.batch):
        sl, pairs = run.alloc.append(run.ids[h], 1)
        assert not pairs                 # every sequence writes into a block of its own
        slots[i] = sl[0]
        t = run.alloc.block_table(run.ids[h])
        assert len(t) <= width and t[:len(run.tables[i])] == run.tables[i]
        bt[i, :len(t)] = t
    run.pairs_d.fill_(-1)                # this step copies no block (pairs outside the pool are skipped)
    run.new_slots_d.copy_(torch.from_numpy(slots))
    run.block_tables.copy_(torch.from_numpy(bt))
    run.seq_lens.add_(1)
    run.cached_lens.add_(1)
    run.k_new.copy_(run.upload(k2))
    run.v_new.copy_(run.upload(v2))
    run.q.copy_(run.upload(q2))
    torch.cuda.synchronize()
    rows = [(np.concatenate([K, k2[i:i + 1]]), np.concatenate([V, v2[i:i + 1]]))
            for i, (K, V) in enumerate(logical_rows(wl))]
    want = oracle_from_rows(rows, q2, np.ones(S), wl)
    for rep in range(2):
        run.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check_oracle(run, want, f"{name} grown, replay {rep}")
        got = run.host(run.out).copy()
    run.out.fill_(float("nan"))
    with torch.cuda.stream(side):
        run.step()                       # the same grown step, eagerly
    torch.cuda.synchronize()
    assert np.array_equal(run.host(run.out), got), f"{name}: grown replay differs from the eager step"


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")   # nothing was launched: the point of the test
def test_check_mode_refused_under_capture(monkeypatch):
    import torch
    import paged_kv_cache_forward_amd as pa
    run = _run("decode_bf16")
    monkeypatch.setenv("PA_CHECK", "1")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    errors = []
    with torch.cuda.stream(side):
        graph.capture_begin()
        try:
            for call in (run.forward, run.step_writes):
                try:
                    call()
                except pa.PagedAttnError as e:   # returns before launching anything
                    errors.append(e.status)
        finally:
            graph.capture_end()
    torch.cuda.synchronize()
    assert errors and all(s == pa.PA_ERR_ARG for s in errors)
