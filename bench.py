"""Benchmark: one engine step of paged attention on one MI355X.

A step is the whole hot path on one synthetic batch whose host-side
allocation has already produced its slot mapping: copy-on-write block copies
(pa_copy_blocks, when the step has any), the cache write of the step's new
tokens (pa_write_kv), then attention (pa_forward: split-KV decode + merge,
and chunked prefill when the batch has chunks).  Inputs are resident in HBM
before the timed region.

Default workload: 64 decode sequences with contexts U[128, 4096], 32 query /
8 KV heads, head_dim 128, bf16, 16-token blocks scattered over a 20000-block
pool.  Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode KV-read GB/s (% HBM peak) + tokens/s; prefill MFMA util"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_bytes(wl):
    e = 4 if wl.dtype == "f32" else 2
    return int(wl.seq_lens.astype(np.int64).sum()) * 2 * wl.num_kv_heads * wl.head_dim * e


def decode_algorithmic_bytes(wl):
    """KV read once per KV head + q read + out written + block-table entries."""
    e = 4 if wl.dtype == "f32" else 2
    tables = int(sum((int(L) + 15) // 16 for L in wl.seq_lens)) * 4
    return kv_bytes(wl) + 2 * wl.num_tokens * wl.num_q_heads * wl.head_dim * e + tables


def prefill_flops(wl):
    """Causal visible (query, key) pairs x 4 * Hq * D, for sequences with more than one query."""
    f = 0
    for c, n in zip(wl.cached_lens.astype(np.int64), wl.query_lens.astype(np.int64)):
        if n > 1:
            f += 4 * wl.num_q_heads * wl.head_dim * int(c * n + n * (n + 1) // 2)
    return int(f)


def time_steps(run, steps, warmup, stream, with_writes=True):
    """Returns (wall ms per step, event ms per forward call, list of per-forward ms)."""
    import torch
    for _ in range(warmup):
        if with_writes:
            run.step_writes(stream)
        run.forward(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for k in range(steps):
        if with_writes:
            run.step_writes(stream)
        ev[k][0].record(stream)
        run.forward(stream)
        ev[k][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per_fwd = [a.elapsed_time(b) for a, b in ev]
    return start.elapsed_time(end) / steps, wall, per_fwd


def cpu_baseline(wl, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same workload (first sequences, in order)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from helpers import OracleRun
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    log("cpu baseline: building the oracle's pools")
    ref = OracleRun(wl, compute_out=False)
    qsl = wl.query_start_loc
    e = 4 if wl.dtype == "f32" else 2
    done_bytes, done_seqs, done_tokens = 0, 0, 0
    t0 = time.perf_counter()
    for i in range(wl.num_seqs):
        r0, r1 = int(qsl[i]), int(qsl[i + 1])
        oracle.ref_paged_attention(wl.q[r0:r1], ref.k_cache, ref.v_cache, [ref.tables[i]],
                                   wl.seq_lens[i:i + 1], np.array([0, r1 - r0]), wl.cached_lens[i:i + 1],
                                   wl.scale, wl.causal, wl.block_size, wl.dtype)
        done_seqs += 1
        done_tokens += r1 - r0
        done_bytes += int(wl.seq_lens[i]) * 2 * wl.num_kv_heads * wl.head_dim * e
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"pa_forward oracle (NumPy float64) on the first {done_seqs} of {wl.num_seqs} sequences "
                  f"({done_tokens} query tokens, {done_bytes / 1e6:.1f} MB of K/V) in {dt:.1f} s",
        "tokens_per_s": round(done_tokens / dt, 3),
    }


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batched_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill MFMA-utilisation leg")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run pa_copy_blocks over 1 GiB (read) + 1 GiB (write): the known-size copy "
                         "that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path is single-GPU; see DESIGN.md for how it would shard).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import paged_kv_cache_forward_amd as pa
    from paged_kv_cache_forward_amd.replay import DeviceRun

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    stream = torch.cuda.current_stream()

    if args.copy_probe:
        copy_probe(pa, torch, stream, args.steps)
        return

    log(f"generating workload {args.workload}")
    wl = workloads.named(args.workload)
    log("placing it on the GPU")
    run = DeviceRun(wl, fill="zero")
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    ms_step, wall_ms, per_fwd = time_steps(run, args.steps, args.warmup, stream)
    fwd_ms = float(np.mean(per_fwd))

    kvb = kv_bytes(wl)
    algo = decode_algorithmic_bytes(wl)
    value = kvb / (ms_step * 1e-3) / 1e9
    achieved = algo / (fwd_ms * 1e-3) / 1e9
    wl_cfg = {
        "workload": wl.name,
        "seqs": wl.num_seqs,
        "context": {"tiny_decode": "{35,16,1,50}", "batched_decode": "U[128,4096]",
                    "long_context_decode": "U[32768,131072]", "mixed_superbatch": "16 decode U[256,4096] + 4x512 chunks",
                    "shared_prefix_cow": "2048 shared + U[0,512]"}.get(wl.name, "custom"),
        "sum_context_tokens": int(wl.seq_lens.sum()),
        "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
        "block_size": wl.block_size, "pool_blocks": wl.num_blocks,
        "step": "pa_copy_blocks (if any) + pa_write_kv(new tokens) + pa_forward",
    }
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
        "config": wl_cfg,
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(wl.num_tokens / (ms_step * 1e-3), 1),
        "wall_ms_per_step": round(wall_ms, 5),
        "forward_ms": round(fwd_ms, 5),
        "roofline": {
            "kernel": "pa_forward (decode_kernel + merge_kernel)" if plan_ws else "pa_forward (decode_kernel)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": algo,
        },
    }
    del run
    torch.cuda.empty_cache()

    if not args.no_prefill:
        log("prefill leg: the four 512-token chunks of the mixed super-batch")
        mix = workloads.mixed_superbatch()
        sel = [i for i in range(mix.num_seqs) if mix.query_lens[i] > 1]
        pre = workloads.independent("mixed_prefill_chunks", 4, Hq=32, Hkv=8, D=128, dtype="bf16",
                                    cached=mix.cached_lens[sel], new=mix.query_lens[sel], pool_factor=1.25)
        prun = DeviceRun(pre, fill="zero")
        _, _, pf = time_steps(prun, max(5, args.steps // 5), 3, stream, with_writes=False)
        pms = float(np.mean(pf))
        fl = prefill_flops(pre)
        tf = fl / (pms * 1e-3) / 1e12
        res["prefill"] = {"workload": "4 chunks x 512 tokens on 0/1024/4096/8192 cached, 32/8 heads, D128, bf16",
                          "ms": round(pms, 5), "tflops": round(tf, 2),
                          "mfma_util": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": fl}
        del prun
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
