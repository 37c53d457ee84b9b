"""HIP-graph capture of a serving step (pa_copy_blocks + pa_write_kv + pa_forward).

The step is captured once with torch.cuda.graph on a side stream and replayed
several times, with the program's own eager work and synchronisations between
replays; every replay must give the eager step's output bits.  A replay after
the query rows are changed in place must give the eager result for the new
queries (the captured calls read device inputs at replay time).  Check mode,
which synchronises, must refuse to run under capture.
"""

import numpy as np
import pytest

import workloads
from helpers import ensure_library

pytestmark = pytest.mark.gpu


def _run(name):
    ensure_library()
    from workloads.device import DeviceRun
    import torch
    run = DeviceRun(workloads.mini(name))
    torch.cuda.synchronize()
    return run


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
    for rep in range(3):
        run.out.fill_(float("nan"))      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = run.host(run.out)
        assert np.array_equal(got, want), f"{name}: replay {rep} differs from the eager step"

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
