"""Benchmark: one engine step of paged attention on one MI355X.

A step is the whole device-side hot path on one synthetic batch whose host
allocation has already produced its block tables and slot mapping: the
copy-on-write block copies (pa_copy_blocks, when the step has any), then the
cache write of the step's new tokens and attention in one call
(pa_write_kv_forward: a decode-only batch fuses the write into the decode;
otherwise pa_write_kv, then decode + split-KV merge, and chunked prefill when
the batch has chunks).
Inputs are resident in HBM before the timed region.  Steps rotate over enough
identical copies of the K/V pools that no step finds its K/V in the 256 MB
last-level cache, as successive layers of a model would not (at most 128
copies: a tiny batch's K/V stays cache-resident, as in a model of 128 layers).

Headline workloads: `batched_decode` (64 decode sequences with contexts
U[128, 4096], 32 query / 8 KV heads, head_dim 128, bf16, 16-token blocks
scattered over a 20000-block pool) gives `value`; `long_context_decode` (8
sequences of 32K-128K tokens, 64/8 heads, split-KV) is reported beside it in
`headline_configs`.  Prints one JSON line on stdout; progress goes to stderr.

Before any timing, untimed steps run until the GPU has been busy for a few
hundred milliseconds (`settle_ms`), so that the clocks have left their idle
state, as in a serving loop; then --warmup untimed steps, then timed regions
of --steps steps each: the first (HIP events around the K steps only) gives
`value` and `ms_per_step`; the second records an event after every step
(median, p10, p90 per step); the third repeats one pool copy every step (the
"hot" median: K/V partly served from the caches); the fourth runs with the
library's per-kernel HIP-event tracing on and gives the kernel durations behind
`roofline`.  After the first, a probe kernel reads the shader clock
(`pa_trace_clock`).  Side legs: the prefill chunks of the mixed super-batch
(MFMA utilisation), a speculative-decoding step (64 sequences verifying 2..8
tokens each) through the multi-token decode kernel and, for comparison,
through the chunked-prefill kernel, the default decode step on a quantised fp8
cache (`fp8_decode`), every other configuration as a whole step (`configs`,
with its allocator accounting), a step launched call by call vs replayed from
a HIP graph (`graph`), the host allocator's replay rate, and the CPU oracle
(`cpu_baseline`, every configuration, in a child process that never touches
the GPU: a process pool over (sequence, KV head) items, one BLAS thread each).
`--copy-probe` instead runs only the known-size copy used to calibrate
rocprofv3's HBM byte counters.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read GB/s (% HBM peak) + tokens/s; prefill MFMA util"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, datasheet
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, datasheet
PROFILES = os.path.join(ROOT, "profiles")
CONTEXT = {"tiny_decode": "{35,16,1,50}", "batched_decode": "U[128,4096]",
           "long_context_decode": "U[32768,131072]",
           "mixed_superbatch": "16 decode U[256,4096] + 4x512 chunks on 0/1024/4096/8192 cached",
           "shared_prefix_cow": "2048 shared + U[0,512] private",
           "spec_verify": "U[128,4096], U{2..8} query tokens each",
           "batched_decode_fp8": "U[128,4096], fp8 cache"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def elem_bytes(wl):
    return 4 if wl.dtype == "f32" else 2


def decode_rows(wl):
    return [i for i in range(wl.num_seqs) if wl.query_lens[i] == 1]


def kv_row_bytes(wl):
    """Stored bytes of one token's K (or V) row for one KV head: head_dim elements, or for an
    fp8 cache head_dim E4M3 codes + one scale byte."""
    return wl.head_dim + 1 if wl.cache == "fp8" else wl.head_dim * elem_bytes(wl)


def kv_bytes(wl, seqs=None):
    """K and V bytes of the visible context, read once per KV head (paging leaves bytes per token unchanged)."""
    seqs = range(wl.num_seqs) if seqs is None else seqs
    return sum(int(wl.seq_lens[i]) for i in seqs) * 2 * wl.num_kv_heads * kv_row_bytes(wl)


def unique_kv_bytes(wl, tables):
    """K and V bytes of the distinct physical blocks the batch reads (a shared block counted once,
    with the most tokens any sequence reads from it)."""
    used = {}
    for i, t in enumerate(tables):
        L = int(wl.seq_lens[i])
        for p, b in enumerate(t):
            n = min(wl.block_size, L - p * wl.block_size)
            if n > 0:
                used[b] = max(used.get(b, 0), n)
    return sum(used.values()) * 2 * wl.num_kv_heads * kv_row_bytes(wl)


def decode_algorithmic_bytes(wl):
    """Decode rows: K/V + q read + out written + block-table entries."""
    seqs = decode_rows(wl)
    e = elem_bytes(wl)
    table = sum((int(wl.seq_lens[i]) + 15) // 16 for i in seqs) * 4
    return kv_bytes(wl, seqs) + 2 * len(seqs) * wl.num_q_heads * wl.head_dim * e + table


def multi_token_algorithmic_bytes(wl):
    """Sequences with 2..16 query rows: K/V once per KV head + their q read + out written + table entries."""
    seqs = [i for i in range(wl.num_seqs) if 2 <= wl.query_lens[i] <= 16]
    e = elem_bytes(wl)
    rows = sum(int(wl.query_lens[i]) for i in seqs)
    table = sum((int(wl.seq_lens[i]) + 15) // 16 for i in seqs) * 4
    return kv_bytes(wl, seqs) + 2 * rows * wl.num_q_heads * wl.head_dim * e + table


def write_algorithmic_bytes(wl):
    """pa_write_kv of the step's new tokens: K and V read and written, plus the slots."""
    return wl.num_tokens * (2 * 2 * wl.num_kv_heads * wl.head_dim * elem_bytes(wl) + 8)


def prefill_flops(wl):
    """Causal visible (query, key) pairs x 4 * Hq * D, for sequences with more than one query."""
    f = 0
    for c, n in zip(wl.cached_lens.astype(np.int64), wl.query_lens.astype(np.int64)):
        if n > 1:
            f += 4 * wl.num_q_heads * wl.head_dim * int(c * n + n * (n + 1) // 2)
    return int(f)


def run_steps(run, steps, stream, with_writes=True, rotate=True, events=None):
    """Enqueue `steps` steps, rotating pool copies (or always the first with rotate=False); with
    `events` (steps + 1 of them) one is recorded before the first step and after each step."""
    if events is not None:
        events[0].record(stream)
    for k in range(steps):
        run.use(k if rotate else 0)
        if with_writes:
            run.step(stream)
        else:
            run.forward(stream)
        if events is not None:
            events[k + 1].record(stream)


MAX_POOL_COPIES = 128


def pool_copies(kvb):
    """Identical K/V pool copies that timed steps rotate over: enough for >= 1 GiB of K/V read
    across the rotation (so a step's K/V is not served from the 256 MB last-level cache), at
    least 2 and at most MAX_POOL_COPIES (a model's layer count: a tiny batch then stays
    cache-resident, as it would in a model)."""
    return min(MAX_POOL_COPIES, max(2, -(-(1 << 30) // max(int(kvb), 1))))


SETTLE_MS = 300.0


def _settle_set(ms):
    global SETTLE_MS
    SETTLE_MS = float(ms)


def settle(run, stream, with_writes=True, min_ms=None):
    """Untimed steps until the GPU has been busy for at least `min_ms` (default SETTLE_MS; wall
    clock, synchronised every few steps): the clocks leave their idle state before anything is
    timed."""
    import torch
    min_ms = SETTLE_MS if min_ms is None else min_ms
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        run_steps(run, 8, stream, with_writes)
        torch.cuda.synchronize()
        n += 8
    return n


def step_distribution(run, steps, stream, with_writes=True, rotate=True):
    """Per-step times (us) from events recorded after every step: median, p10, p90."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    run_steps(run, steps, stream, with_writes, rotate, events=evs)
    torch.cuda.synchronize()
    us = np.array([evs[k].elapsed_time(evs[k + 1]) * 1e3 for k in range(steps)])
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"median": round(float(p50), 2), "p10": round(float(p10), 2), "p90": round(float(p90), 2)}


def read_mclk_mhz():
    """Current memory clock from the driver's DPM table in sysfs (the level marked '*'), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_mclk")):
        try:
            with open(path) as f:
                for line in f:
                    if line.strip().endswith("*"):
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            continue
    return None


def clocks(pa, stream):
    """Shader clock the GPU runs at right now (probe kernel) and the memory clock (sysfs)."""
    try:
        sclk = round(pa.pa_trace_clock(stream), 1)
    except Exception as e:                     # instrumentation only: never fail the bench on it
        log(f"clock probe failed: {e}")
        sclk = None
    return {"sclk_mhz": sclk, "mclk_mhz": read_mclk_mhz()}


def alloc_accounting(wl, run):
    """The host allocator's view of the batch after the step's allocations ("Was ändert
    PagedAttention an der KV-Speicherzuweisung für LLMs?", sections "Ungenutzten Platz in Blöcken
    berechnen" and "Gemeinsame Nutzung ..."): blocks, slots, tokens and the unused share of the
    allocated slots, per sequence (logical) and per physical block (a shared block counted once)."""
    st = run.alloc.stats()
    filled = {}
    for i, t in enumerate(run.tables):
        L = int(wl.seq_lens[i])
        for p, b in enumerate(t):
            n = min(wl.block_size, L - p * wl.block_size)
            if n > 0:
                filled[b] = max(filled.get(b, 0), n)
    tokens_physical = int(sum(filled.values()))
    out = {k: int(v) for k, v in st.items()}
    out["tokens_physical"] = tokens_physical
    out["unused_frac_logical"] = round(1.0 - st["tokens_logical"] / max(st["slots_logical"], 1), 5)
    out["unused_frac_physical"] = round(1.0 - tokens_physical / max(st["slots_physical"], 1), 5)
    out["sharing_factor"] = round(st["tokens_logical"] / max(tokens_physical, 1), 3)
    return out


def timed_region(run, steps, stream, with_writes=True):
    """Events + wall clock around exactly `steps` steps, synchronised on both sides."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    run_steps(run, steps, stream, with_writes)
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return start.elapsed_time(end) / steps, wall_ms


def unfused_step(run, steps, stream):
    """The same step as two calls (pa_write_kv, then pa_forward): its median per-step time in us,
    for a single-token batch (where pa_write_kv_forward fuses the write), else None."""
    if run.wl.max_query_len != 1 or run.shared:
        return None
    run.fused = False
    try:
        return step_distribution(run, steps, stream)
    finally:
        run.fused = True


def traced_region(pa, run, steps, stream, with_writes=True):
    """The same steps with per-kernel tracing on; returns {kernel: [ms, ...]}."""
    import torch
    torch.cuda.synchronize()
    pa.pa_trace_read()                       # drop stale records
    pa.pa_trace_enable(True)
    try:
        run_steps(run, steps, stream, with_writes)
        torch.cuda.synchronize()
    finally:
        pa.pa_trace_enable(False)
    per = {}
    for name, ms in pa.pa_trace_read():
        per.setdefault(name, []).append(ms)
    return per


def strip_comments(text):
    """C/C++ source without // and /* */ comments, trailing blanks or blank lines (string literals kept)."""
    out, i, n, quote = [], 0, len(text), None
    while i < n:
        c = text[i]
        if quote:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(text[i + 1])
                i += 2
                continue
            if c == quote:
                quote = None
            i += 1
        elif c in "\"'":
            quote = c
            out.append(c)
            i += 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = [l.rstrip() for l in "".join(out).split("\n")]
    return "\n".join(l for l in lines if l)


def source_digest(*names):
    """sha256 of the kernels' code (comments and blank lines stripped): a comment edit keeps it."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_forward_amd", "csrc", n), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()


KERNEL_SOURCES = {
    "decode_mfma": ("decode_mfma.hip", "device.h"),
    "decode_valu": ("decode.hip", "device.h"),
    "prefill": ("prefill.hip", "device.h"),
    "write_kv": ("cache_ops.hip", "device.h"),
    "decode_verify": ("decode_verify.hip", "device.h"),
    "decode_shared": ("decode_shared.hip", "device.h"),
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the kernel is unchanged since.

    The summary (profiles/<kernel>-<workload>-hbm_counters.txt) holds key=value
    lines: the bytes one dispatch read and wrote past the L2, from the TCC
    request counters by size (TCC_EA0_RDREQ_32B/64B/128B: requests of 32, 64
    and 128 bytes; TCC_EA0_WRREQ, TCC_EA0_WRREQ_64B: write requests of 32 and 64
    bytes), and the sha256 of the kernel's sources when the counters were taken.
    Returns None when there is no summary or the sources have changed.
    """
    path = os.path.join(PROFILES, f"{kernel}-{workload}-hbm_counters.txt")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(*KERNEL_SOURCES[kernel]):
        return None
    return int(round(float(kv["read_bytes_per_dispatch"]) + float(kv["write_bytes_per_dispatch"])))


# -- CPU oracle baseline -----------------------------------------------------------
#
# Runs in a child process started with subprocess (never an exec of this
# process) that imports neither torch nor the library and never opens the GPU,
# with one BLAS thread per process.  It generates each configuration from its
# seed, builds the oracle's pools (not timed), then times whole passes of the
# oracle over the batch with a fork-started pool of N = len(sched_getaffinity)
# worker processes over (sequence, KV head) items, longest first.

_CPU = {}


def _cpu_noop(_):
    return os.getpid()


def _cpu_item(item):
    """The oracle on sequence i's query rows of KV head g's query heads, that head's pool slice."""
    import oracle
    i, g = item
    wl, ref = _CPU["wl"], _CPU["ref"]
    qsl = wl.query_start_loc
    r0, r1 = int(qsl[i]), int(qsl[i + 1])
    G = wl.num_q_heads // wl.num_kv_heads
    out = oracle.ref_paged_attention(wl.q[r0:r1, g * G:(g + 1) * G], ref.k_cache[:, g:g + 1], ref.v_cache[:, g:g + 1],
                                     [ref.tables[i]], wl.seq_lens[i:i + 1], np.array([0, r1 - r0]),
                                     wl.cached_lens[i:i + 1], wl.scale, wl.causal, wl.block_size, wl.dtype)
    return float(np.abs(out).sum())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_child_main(spec):
    """--cpu-baseline-child: time the oracle on each named configuration; one JSON line on stdout."""
    import multiprocessing as mp
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads
    from helpers import OracleRun
    n_proc = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas = None
    res = {"cores": n_proc, "cpu_model": cpu_model(), "blas_threads_per_process": blas, "configs": {}}
    for name in spec["names"]:
        log(f"cpu baseline: {name}: generating it and building the oracle's pools (not timed)")
        wl = workloads.named(name)
        if wl.cache == "fp8":
            continue
        ref = OracleRun(wl, compute_out=False)
        _CPU.update(wl=wl, ref=ref)
        items = [(i, g) for i in range(wl.num_seqs) if wl.query_lens[i] > 0 for g in range(wl.num_kv_heads)]
        items.sort(key=lambda ig: -int(wl.seq_lens[ig[0]]) * int(wl.query_lens[ig[0]]))
        small = name in ("tiny_decode", "batched_decode")
        want_runs = 3 if small else 1
        min_s = spec.get("min_s", 0.0) if name == spec.get("headline") else 0.0
        runs = []
        with mp.get_context("fork").Pool(n_proc) as pool:
            pool.map(_cpu_noop, range(4 * n_proc))        # workers started before timing
            log(f"cpu baseline: {name}: {len(items)} (sequence, KV head) items on {n_proc} processes")
            t_all = time.perf_counter()
            while True:
                t0 = time.perf_counter()
                pool.map(_cpu_item, items, chunksize=1)
                runs.append(time.perf_counter() - t0)
                elapsed = time.perf_counter() - t_all
                if (len(runs) >= want_runs and elapsed >= min_s) or elapsed > spec.get("max_s", 60.0):
                    break
        best = min(runs)
        kvb = kv_bytes(wl)
        entry = {"seconds_best": round(best, 4), "seconds_runs": [round(x, 4) for x in runs],
                 "query_tokens": wl.num_tokens, "tokens_per_s": round(wl.num_tokens / best, 2),
                 "kv_bytes": int(kvb), "kv_GBs": round(kvb / best / 1e9, 4), "items": len(items)}
        pf = prefill_flops(wl)
        if pf:
            entry["prefill_GFLOPs"] = round(pf / best / 1e9, 3)
        res["configs"][name] = entry
        log(f"cpu baseline: {name}: best pass {best:.3f} s ({entry['kv_GBs']} GB/s of K/V)")
        _CPU.clear()
        del ref, wl
    print(json.dumps(res), flush=True)


def cpu_baselines(names, headline, min_s=5.0, max_s=60.0, timeout=900):
    """Run cpu_child_main in a child process (BLAS threads fixed at 1) and return its JSON, or an error."""
    import subprocess
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS",
              "NUMEXPR_NUM_THREADS"):
        env[k] = "1"
    spec = {"names": list(names), "headline": headline, "min_s": min_s, "max_s": max_s}
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", json.dumps(spec)],
                           env=env, stdout=subprocess.PIPE, stderr=None, text=True, timeout=timeout)
    except subprocess.TimeoutExpired:
        return {"error": f"cpu baseline child timed out after {timeout} s"}
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    if r.returncode != 0 or not lines:
        return {"error": f"cpu baseline child exited with {r.returncode}"}
    return json.loads(lines[-1])


def allocator_rate(pa, wl, reps=3):
    """Host block allocator: replay the workload's allocation trace through the C ABI (ctypes included)."""
    from workloads import drive as _drive
    best = None
    for _ in range(reps):
        alloc = pa.BlockAllocator(wl.num_blocks, wl.block_size, wl.free_order)
        t0 = time.perf_counter()
        _drive(wl, alloc)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
    tokens = int(wl.seq_lens.sum() - sum(int(op[3]) for op in wl.trace if op[0] == "fork"))
    return {"calls": len(wl.trace), "tokens_appended": tokens, "s": round(best, 6),
            "calls_per_s": round(len(wl.trace) / best, 1), "tokens_per_s": round(tokens / best, 1)}


def copy_probe(pa, torch, stream, steps):
    """pa_copy_blocks over 16384 pairs of 32 KiB blocks (K and V): 1 GiB read and 1 GiB written per launch."""
    nb, hkv, d = 32768, 8, 128
    kc = torch.zeros((nb, hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    half = nb // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], dim=1).to(torch.int32).cuda()
    per_launch = 2 * half * hkv * 16 * d * 2
    for _ in range(2):
        pa.pa_copy_blocks(kc, vc, pairs, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        pa.pa_copy_blocks(kc, vc, pairs, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"probe": "pa_copy_blocks", "bytes_read_per_launch": per_launch,
                      "bytes_written_per_launch": per_launch, "ms": round(ms, 5),
                      "copy_gbs": round(2 * per_launch / (ms * 1e-3) / 1e9, 1)}), flush=True)


def mean(xs):
    return float(np.mean(xs)) if xs else None


GRAPH_LAYERS = 8


def graph_leg(pa, torch, workloads, DeviceRun, name, steps):
    """Serving steps (pa_copy_blocks + pa_write_kv_forward) issued one call at a time vs replayed
    from HIP graphs.

    Three ways, timed back to back on a side stream with HIP events: eager
    steps; a graph of one step, replayed; a graph of GRAPH_LAYERS steps over as
    many pool copies (a model's layers, each with its own cache), replayed --
    per step.  Every replay's output bits must equal the eager step's.
    """
    wl = workloads.named(name)
    run = DeviceRun(wl, fill="zero", copies=GRAPH_LAYERS)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            run.step()
    torch.cuda.synchronize()
    want = run.host(run.out).copy()

    def layers():
        for k in range(GRAPH_LAYERS):
            run.use(k)
            run.step()
        run.use(0)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run.step()
    graph_l = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_l, stream=side):
        layers()
    torch.cuda.synchronize()
    for g in (graph, graph_l):
        run.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not np.array_equal(run.host(run.out), want):
            raise RuntimeError(f"graph replay of {name} differs from the eager step")

    def timed(fn, per=1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            for _ in range(5):
                fn()
            a.record(side)
            for _ in range(steps):
                fn()
            b.record(side)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (steps * per)

    eager_us = timed(run.step)
    graph_us = timed(graph.replay)
    eager_l_us = timed(layers, GRAPH_LAYERS)
    graph_l_us = timed(graph_l.replay, GRAPH_LAYERS)
    del graph, graph_l, run
    torch.cuda.empty_cache()
    return {"workload": name, "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "speedup": round(eager_us / graph_us, 3),
            "layers_per_graph": GRAPH_LAYERS, "eager_layers_us_per_step": round(eager_l_us, 2),
            "graph_layers_us_per_step": round(graph_l_us, 2),
            "speedup_layers": round(eager_l_us / graph_l_us, 3)}


def shared_leg(pa, torch, DeviceRun, wl, steps, stream, uniq):
    """The same step through pa_forward_shared (shared blocks read once per group of sequences, the
    allocator's shared-block counts passed in), its decode kernel against HBM on the distinct bytes."""
    log(f"config leg: {wl.name} through pa_forward_shared")
    run = DeviceRun(wl, fill="zero", copies=pool_copies(kv_bytes(wl)), shared=True)
    settle(run, stream)
    run_steps(run, 3, stream)
    ms_step, _ = timed_region(run, steps, stream)
    dist = step_distribution(run, steps, stream)
    per = traced_region(pa, run, steps, stream)
    out = {"ms_per_step": round(ms_step, 5), "step_us": dist,
           "tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
           "kv_GBs_step_unique": round(uniq / (ms_step * 1e-3) / 1e9, 2),
           "kernel_ms": {k: round(mean(v), 5) for k, v in per.items()},
           "kernel_us_median": {k: round(float(np.median(v)) * 1e3, 2) for k, v in per.items()},
           "groups_shared_blocks_max": int(run.shared_blocks.max())}
    if "decode_shared" in per:
        algo = decode_algorithmic_bytes(wl) - kv_bytes(wl, decode_rows(wl)) + uniq
        dms = mean(per["decode_shared"])
        ach = algo / (dms * 1e-3) / 1e9
        out["decode_roofline"] = {"kernel": "decode_shared", "bound": "hbm", "achieved": round(ach, 2),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes_per_launch": int(algo), "launch_ms": round(dms, 5),
                                  "traffic": measured_traffic("decode_shared", wl.name)}
    del run
    torch.cuda.empty_cache()
    return out


def config_leg(pa, torch, workloads, DeviceRun, name, steps, stream):
    """One workload's whole step (copies, writes, forward) and its decode kernel against the HBM roofline.

    Pools rotate over copies as in the headline run (pool_copies); after the settle
    phase, the step time comes from events around untraced steps, its spread
    from events after every step, per-kernel times from the library's own
    events on the launch stream."""
    log(f"config leg: {name}")
    wl = workloads.named(name)
    kvb = kv_bytes(wl)
    run = DeviceRun(wl, fill="zero", copies=pool_copies(kvb))
    settle(run, stream)
    run_steps(run, 3, stream)
    ms_step, _ = timed_region(run, steps, stream)
    clk = clocks(pa, stream)
    dist = step_distribution(run, steps, stream)
    hot = step_distribution(run, steps, stream, rotate=False)
    unfused = unfused_step(run, steps, stream)
    per = traced_region(pa, run, steps, stream)
    out = {"seqs": wl.num_seqs, "query_tokens": wl.num_tokens, "sum_context_tokens": int(wl.seq_lens.sum()),
           "dtype": wl.dtype, "ms_per_step": round(ms_step, 5), "step_us": dist, "step_us_hot": hot,
           "tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
           "kv_GBs_step": round(kvb / (ms_step * 1e-3) / 1e9, 2),
           "step_frac": round(kvb / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "kernel_ms": {k: round(mean(v), 5) for k, v in per.items()},
           "kernel_us_median": {k: round(float(np.median(v)) * 1e3, 2) for k, v in per.items()},
           "clocks": clk, "allocator": alloc_accounting(wl, run)}
    if unfused is not None:
        out["step_us_unfused"] = unfused
    dec = next((k for k in ("decode_mfma", "decode_valu", "decode_verify") if k in per), None)
    if dec is not None and decode_rows(wl):
        algo = decode_algorithmic_bytes(wl)
        logical = algo
        if name == "shared_prefix_cow":
            # HBM has to deliver each shared block once: price the kernel on the distinct blocks
            algo = algo - kv_bytes(wl, decode_rows(wl)) + unique_kv_bytes(wl, run.tables)
        dms = mean(per[dec])
        ach = algo / (dms * 1e-3) / 1e9
        out["decode_roofline"] = {"kernel": dec, "bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                  "algorithmic_bytes_per_launch": int(algo), "launch_ms": round(dms, 5),
                                  "traffic": measured_traffic(dec, wl.name)}
        if logical != algo:
            out["decode_roofline"]["logical_bytes_per_launch"] = int(logical)
            out["decode_roofline"]["logical_GBs"] = round(logical / (dms * 1e-3) / 1e9, 2)
    if "prefill" in per:
        pms = mean(per["prefill"])
        tf = prefill_flops(wl) / (pms * 1e-3) / 1e12
        out["prefill"] = {"ms": round(pms, 5), "tflops": round(tf, 2),
                          "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    if name == "shared_prefix_cow":
        # the shared prefix is read by all 256 sequences; count its blocks once
        uniq = unique_kv_bytes(wl, run.tables)
        out["kv_unique_bytes"] = int(uniq)
        out["kv_GBs_step_unique"] = round(uniq / (ms_step * 1e-3) / 1e9, 2)
        out["shared_decode"] = shared_leg(pa, torch, DeviceRun, wl, steps, stream, uniq)
    if name == "long_context_decode":
        # bulk cache write: the first 262144 context tokens stored again (same slots, same bytes)
        n = min(len(wl.ctx_k), 1 << 18)
        k = run.upload(wl.ctx_k[:n])
        v = run.upload(wl.ctx_v[:n])
        sl = torch.from_numpy(run.ctx_slots[:n]).to(run.dev)
        torch.cuda.synchronize()
        pa.pa_trace_read()
        pa.pa_trace_enable(True)
        try:
            for _ in range(5):
                pa.pa_write_kv(k, v, run.k_cache, run.v_cache, sl, stream=stream)
            torch.cuda.synchronize()
        finally:
            pa.pa_trace_enable(False)
        wms = mean([ms for kname, ms in pa.pa_trace_read() if kname == "write_kv"])
        moved = n * (2 * 2 * wl.num_kv_heads * wl.head_dim * elem_bytes(wl) + 8)
        out["bulk_write_kv"] = {"tokens": n, "bytes_moved": int(moved), "ms": round(wms, 5),
                                "GBs": round(moved / (wms * 1e-3) / 1e9, 2),
                                "frac": round(moved / (wms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del k, v, sl
    del run
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batched_decode")
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate (0: pool_copies, >= 1 GiB of K/V, at most 128)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill MFMA-utilisation leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph step-replay leg")
    ap.add_argument("--no-verify", action="store_true", help="skip the multi-token decode leg")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache decode leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration leg (tiny, long-context, mixed and shared-prefix steps)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run pa_copy_blocks over 1 GiB (read) + 1 GiB (write): the known-size copy "
                         "that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed busy time before timing (0 for a counter-collection run, where every "
                         "dispatch is serialised)")
    ap.add_argument("--config-leg", default=None, metavar="WORKLOAD",
                    help="run only this workload's configuration leg (as in `configs`) and print it")
    ap.add_argument("--cpu-baseline-child", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child is not None:    # the GPU-free child of cpu_baselines()
        cpu_child_main(json.loads(args.cpu_baseline_child))
        return
    _settle_set(args.settle_ms)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported: the library is the "
              "single-GPU hot path and this benchmark measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import paged_kv_cache_forward_amd as pa
    from workloads.device import DeviceRun

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        copy_probe(pa, torch, stream, args.steps)
        return
    if args.config_leg:
        # one configuration's leg alone (for a profiler run): its JSON object on stdout
        print(json.dumps({args.config_leg: config_leg(pa, torch, workloads, DeviceRun, args.config_leg,
                                                      args.steps, stream)}), flush=True)
        return

    log(f"generating workload {args.workload}")
    wl = workloads.named(args.workload)
    kvb = kv_bytes(wl)
    copies = args.copies or pool_copies(kvb)
    log(f"placing it on the GPU ({copies} pool copies)")
    run = DeviceRun(wl, fill="zero", copies=copies)
    log(f"settle ({SETTLE_MS:.0f} ms of untimed steps), warm-up {args.warmup} steps, then timed regions of "
        f"{args.steps} steps")
    settled = settle(run, stream)
    run_steps(run, args.warmup, stream)
    ms_step, wall_ms = timed_region(run, args.steps, stream)
    clk = clocks(pa, stream)
    dist = step_distribution(run, args.steps, stream)
    hot = step_distribution(run, args.steps, stream, rotate=False)
    unfused = unfused_step(run, args.steps, stream)
    per = traced_region(pa, run, args.steps, stream)
    kern_ms = {k: round(mean(v), 5) for k, v in per.items()}
    dominant = max(per, key=lambda k: sum(per[k]))
    dec_kernel = next(k for k in ("decode_mfma", "decode_verify", "decode_valu") if k in per)

    algo = decode_algorithmic_bytes(wl)
    dom_ms = mean(per[dec_kernel])
    achieved = algo / (dom_ms * 1e-3) / 1e9
    traffic = measured_traffic(dec_kernel, wl.name)
    value = kvb / (ms_step * 1e-3) / 1e9
    plan_ws = pa.pa_forward_workspace_size(wl.num_seqs, wl.num_tokens, wl.num_q_heads, wl.max_seq_len,
                                           wl.max_query_len, run.k_cache)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "seqs": wl.num_seqs,
            "context": CONTEXT.get(wl.name, "custom"),
            "sum_context_tokens": int(wl.seq_lens.sum()),
            "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "pool_blocks": wl.num_blocks, "pool_copies": copies,
            "step": "pa_copy_blocks (if any) + pa_write_kv_forward(new tokens, attention)",
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
        "wall_ms_per_step": round(wall_ms, 5),
        "step_us": dist,
        "step_us_hot": hot,
        "step_us_unfused": unfused,
        "settle_steps": settled,
        "clocks": clk,
        "kernel_ms": kern_ms,
        "dominant_kernel": dominant,
        "workspace_bytes": int(plan_ws),
        "roofline": {
            "kernel": dec_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(algo),
            "launch_ms": round(dom_ms, 5),
        },
    }
    if "write_kv" in per:
        wb = write_algorithmic_bytes(wl)
        res["write_kv"] = {"tokens": wl.num_tokens, "ms": kern_ms["write_kv"],
                           "GBs": round(wb / (kern_ms["write_kv"] * 1e-3) / 1e9, 2)}
    res["allocator"] = allocator_rate(pa, wl)
    res["allocator"]["accounting"] = alloc_accounting(wl, run)
    del run
    torch.cuda.empty_cache()

    if not args.no_prefill:
        log("prefill leg: the four 512-token chunks of the mixed super-batch (forward only)")
        mix = workloads.mixed_superbatch()
        sel = [i for i in range(mix.num_seqs) if mix.query_lens[i] > 1]
        pre = workloads.independent("mixed_prefill_chunks", 4, Hq=32, Hkv=8, D=128, dtype="bf16",
                                    cached=mix.cached_lens[sel], new=mix.query_lens[sel], pool_factor=1.25)
        prun = DeviceRun(pre, fill="zero", copies=2)
        psteps = max(5, args.steps // 5)
        settle(prun, stream, with_writes=False, min_ms=100)
        run_steps(prun, 3, stream, with_writes=False)
        pper = traced_region(pa, prun, psteps, stream, with_writes=False)
        pms = mean(pper["prefill"])
        fl = prefill_flops(pre)
        tf = fl / (pms * 1e-3) / 1e12
        res["prefill"] = {"workload": "4 chunks x 512 tokens on 0/1024/4096/8192 cached, 32/8 heads, D128, bf16",
                          "kernel": "prefill", "ms": round(pms, 5), "tflops": round(tf, 2),
                          "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl,
                          "kernel_ms": {k: round(mean(v), 5) for k, v in pper.items()}}
        del prun
        torch.cuda.empty_cache()

    if not args.no_verify:
        log("multi-token decode leg: 64 sequences verifying 2..8 tokens (forward only), two routes")
        vwl = workloads.spec_verify()
        vrun = DeviceRun(vwl, fill="zero", copies=pool_copies(kv_bytes(vwl)))
        vsteps = max(10, args.steps // 2)
        legs = {}
        for route in ("verify", "prefill"):
            if route == "prefill":
                os.environ["PA_VERIFY"] = "prefill"
                vrun.ensure_workspace()   # the workspace size follows the route
            try:
                settle(vrun, stream, with_writes=False, min_ms=100)
                run_steps(vrun, 3, stream, with_writes=False)
                vms, _ = timed_region(vrun, vsteps, stream, with_writes=False)
                legs[route] = (vms, traced_region(pa, vrun, vsteps, stream, with_writes=False))
            finally:
                os.environ.pop("PA_VERIFY", None)
        vms, vper = legs["verify"]
        vkern = mean(vper["decode_verify"])
        valgo = multi_token_algorithmic_bytes(vwl)
        vach = valgo / (vkern * 1e-3) / 1e9
        res["multi_token_decode"] = {
            "workload": "spec_verify: " + CONTEXT["spec_verify"] + ", 32/8 heads, D128, bf16, causal",
            "ms_per_forward": round(vms, 5),
            "kv_GBs": round(kv_bytes(vwl) / (vms * 1e-3) / 1e9, 2),
            "query_tokens_per_s": round(vwl.num_tokens / (vms * 1e-3), 1),
            "kernel_ms": {k: round(mean(v), 5) for k, v in vper.items()},
            "roofline": {"kernel": "decode_verify", "bound": "hbm", "achieved": round(vach, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(vach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_verify", vwl.name),
                         "algorithmic_bytes_per_launch": int(valgo), "launch_ms": round(vkern, 5)},
            "prefill_route": {"ms_per_forward": round(legs["prefill"][0], 5),
                              "kernel_ms": {k: round(mean(v), 5) for k, v in legs["prefill"][1].items()}},
        }
        del vrun
        torch.cuda.empty_cache()

    if not args.no_fp8:
        log("fp8 leg: the default batched decode on a quantised (E4M3 + row scales) cache, whole steps")
        fwl = workloads.batched_decode_fp8()
        frun = DeviceRun(fwl, fill="zero", copies=pool_copies(kv_bytes(fwl)))
        fsteps = max(10, args.steps // 2)
        settle(frun, stream, min_ms=100)
        run_steps(frun, 3, stream)
        fms, _ = timed_region(frun, fsteps, stream)
        fper = traced_region(pa, frun, fsteps, stream)
        fkern = mean(fper["decode_verify"])
        falgo = decode_algorithmic_bytes(fwl)
        fach = falgo / (fkern * 1e-3) / 1e9
        res["fp8_decode"] = {
            "workload": "batched_decode_fp8: 64 seqs, context U[128,4096], 32/8 heads, D128, fp8 (E4M3, one "
                        "power-of-two scale per token and KV head) cache, bf16 q/out",
            "ms_per_step": round(fms, 5),
            "kv_GBs": round(kv_bytes(fwl) / (fms * 1e-3) / 1e9, 2),
            "tokens_per_s": round(fwl.num_tokens / (fms * 1e-3), 1),
            "kernel_ms": {k: round(mean(v), 5) for k, v in fper.items()},
            "roofline": {"kernel": "decode_verify", "bound": "hbm", "achieved": round(fach, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_verify", fwl.name),
                         "algorithmic_bytes_per_launch": int(falgo), "launch_ms": round(fkern, 5)},
        }
        del frun
        torch.cuda.empty_cache()
        # the four 512-token chunks of the mixed batch on an fp8 cache (forward only)
        mix = workloads.mixed_superbatch()
        sel = [i for i in range(mix.num_seqs) if mix.query_lens[i] > 1]
        fpre = workloads.independent("mixed_prefill_chunks_fp8", 4, Hq=32, Hkv=8, D=128, dtype="bf16",
                                     cached=mix.cached_lens[sel], new=mix.query_lens[sel], pool_factor=1.25,
                                     cache_dtype="fp8")
        fprun = DeviceRun(fpre, fill="zero", copies=2)
        settle(fprun, stream, with_writes=False, min_ms=100)
        run_steps(fprun, 3, stream, with_writes=False)
        fpper = traced_region(pa, fprun, max(5, args.steps // 5), stream, with_writes=False)
        fpms = mean(fpper["prefill"])
        ftf = prefill_flops(fpre) / (fpms * 1e-3) / 1e12
        res["fp8_decode"]["prefill"] = {"workload": "4 chunks x 512 tokens on 0/1024/4096/8192 cached, fp8 cache",
                                        "kernel": "prefill", "ms": round(fpms, 5), "tflops": round(ftf, 2),
                                        "mfma_util": round(ftf / MFMA_BF16_PEAK_TFLOPS, 4),
                                        "kernel_ms": {k: round(mean(v), 5) for k, v in fpper.items()}}
        del fprun
        torch.cuda.empty_cache()

    if not args.no_configs:
        res["configs"] = {n: config_leg(pa, torch, workloads, DeviceRun, n, max(10, args.steps // 2), stream)
                          for n in ("tiny_decode", "long_context_decode", "mixed_superbatch", "shared_prefix_cow")}
        # Both decode configurations lead: the batch `value` is quoted on, and the longest contexts.
        lc = res["configs"]["long_context_decode"]
        res["headline_configs"] = {
            wl.name: {"kv_GBs_step": res["value"], "step_frac": res["hbm_frac"],
                      "decode_kernel_frac": res["roofline"]["frac"], "step_us": dist},
            "long_context_decode": {"kv_GBs_step": lc["kv_GBs_step"], "step_frac": lc["step_frac"],
                                    "decode_kernel_frac": lc.get("decode_roofline", {}).get("frac"),
                                    "step_us": lc["step_us"]},
        }

    if not args.no_graph:
        log("graph leg: one step per launch vs replayed from a HIP graph (tiny and batched decode)")
        res["graph"] = [graph_leg(pa, torch, workloads, DeviceRun, n, max(20, args.steps))
                        for n in ("tiny_decode", "batched_decode")]

    if not args.no_cpu_baseline:
        names = [wl.name] + ([n for n in ("tiny_decode", "long_context_decode", "mixed_superbatch",
                                          "shared_prefix_cow") if n != wl.name] if not args.no_configs else [])
        log(f"cpu baseline (oracle, child process): {', '.join(names)}")
        cb = cpu_baselines(names, wl.name)
        head = cb.get("configs", {}).get(wl.name)
        if head is None:
            res["cpu_baseline"] = {"value": None, "unit": "GB/s", "cores": cb.get("cores"), "kind": "oracle",
                                   "sample": "not measured", "error": cb.get("error")}
        else:
            res["cpu_baseline"] = {
                "value": head["kv_GBs"], "unit": "GB/s", "cores": cb["cores"], "kind": "oracle",
                "sample": f"the whole {wl.name} batch ({wl.num_seqs} sequences, {wl.num_tokens} query tokens, "
                          f"{head['kv_bytes'] / 1e9:.3f} GB of K/V), best of {len(head['seconds_runs'])} passes: "
                          f"ref_paged_attention (NumPy float64) over {head['items']} (sequence, KV head) items on a "
                          f"pool of {cb['cores']} processes, one BLAS thread each",
                "tokens_per_s": head["tokens_per_s"], "seconds_best": head["seconds_best"],
                "cpu_model": cb.get("cpu_model"), "blas_threads_per_process": cb.get("blas_threads_per_process"),
            }
            for n, e in cb["configs"].items():
                if n in res.get("configs", {}):
                    res["configs"][n]["cpu_baseline"] = e
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
