"""Benchmark of the splice hot path on one MI355X.

Workload (default): a DeepSeek-V2-Lite shaped MLA cache, 27 layers, one
sequence of 32768 tokens, rows c_kv 512 + k_pe 64 bf16 ~ N(0,1), page size 16,
pages randomly permuted in a pool of 4096 pages; one AMORTIZE splice drops
three 2048-token tool turns [8192, 14336) for a 24-row stub (Delta = -6120),
moving and rotating every downstream row ("Leyline: KV Cache Directives for
Agentic Inference", sections 2.1-2.3).

A step is one whole splice call through the C ABI (host plan, one upload, one
kernel launch that moves rows, rotates k_pe and rewrites the page table),
preceded by restoring the sequence's original page table (the splice never
writes the old pages, so the pristine state comes back by table alone).
`value` is the row bytes the splice must move per step divided by the wall
time per step.  The roofline object times the row kernel alone with HIP
events recorded on the stream it runs on.  The CPU baseline runs the oracle
on the same workload on the host and checks the GPU result against it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "downstream KV GB/s moved+rotated (% HBM peak); splice latency @32k ctx"
HBM_PEAK_GBS = 8000.0
LAYERS, TOKENS, PAGE, POOL_PAGES = 27, 32768, 16, 4096
S_START, S_END, STUB = 8192, 14336, 24
ROW = 576


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--latency-runs", type=int, default=25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the splice path runs per GPU with no cross-GPU exchange "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import permuted_pages, random_rows_torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    data = random_rows_torch(0, (LAYERS, POOL_PAGES, PAGE, ROW), dev)
    stub = random_rows_torch(1, (LAYERS, STUB, ROW), dev)
    table = torch.full((1, TOKENS // PAGE + 8), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    T = permuted_pages(0, TOKENS // PAGE)
    directive = [L.Directive(0, S_START, S_END, stub)]

    def restore():
        pool.seq_set_pages(0, T, TOKENS)

    # snapshot for the CPU baseline / parity check, taken before any splice
    host_before = None
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        host_before = data.view(torch.int16).cpu().numpy().view(np.uint16)

    restore()
    pool.splice(directive)
    torch.cuda.synchronize()
    stats = pool.last_stats()
    alg_bytes = stats.alg_bytes
    _, _, new_table = pool.seq_get(0)
    gpu_after = None
    if host_before is not None:
        j = np.arange(TOKENS + STUB - (S_END - S_START))
        phys = torch.from_numpy(new_table.astype(np.int64)[j // PAGE] * PAGE + j % PAGE).to(dev)
        gpu_after = data.view(LAYERS, -1, ROW)[:, phys].view(torch.int16).cpu().numpy().view(np.uint16)

    # ---- throughput: K whole steps, bracketed by synchronize
    for _ in range(args.warmup):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    pool.profile_read(0)
    pool.set_profiling(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pool.set_profiling(False)
    launches, kernel_ms, kernel_bytes = pool.profile_read(0)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    k_avg_ms = kernel_ms / max(1, launches)
    achieved = (kernel_bytes / max(1, launches)) / (k_avg_ms * 1e-3) / 1e9

    # ---- latency: API call to stream completion, MALL flushed before each
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    lat = []
    for _ in range(args.latency_runs):
        restore()
        flush.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        pool.splice(directive)
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - a) * 1e6)
    del flush

    # ---- plain device copy of the same byte count, for context
    n_copy = alg_bytes // 2
    src = torch.empty(n_copy, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n_copy * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "splice_32k_27layer",
            "layers": LAYERS, "tokens": TOKENS, "page_size": PAGE, "pool_pages": POOL_PAGES,
            "span": [S_START, S_END], "stub_rows": STUB, "delta": STUB - (S_END - S_START),
            "storage": "bf16 rows c_kv 512 + k_pe 64, rotation in f32",
            "alg_bytes_per_step": alg_bytes,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "splice_latency_us": {"median": round(statistics.median(lat), 1), "min": round(min(lat), 1),
                              "max": round(max(lat), 1), "runs": len(lat)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "splice_kernel",
            "kernel_avg_us": round(k_avg_ms * 1e3, 2),
            "bytes_per_launch": kernel_bytes // max(1, launches),
        },
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "cpu_baseline": None,
    }

    if host_before is not None:
        out["cpu_baseline"] = cpu_baseline(host_before, gpu_after, T, alg_bytes, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    pool.close()


def cpu_baseline(host_before, gpu_after, T, alg_bytes, seconds):
    """The oracle, as it stands, on the same splice on the host: repeated
    until `seconds` have passed; also checks the GPU result against it."""
    from oracle import leyline_oracle as O
    from synth import random_rows_torch  # noqa: F401  (same generator as the device pool)
    import torch

    st = O.CacheState.empty(0, POOL_PAGES, PAGE, TOKENS // PAGE + 8, with_rows=False)
    st.layers = [host_before[i] for i in range(LAYERS)]
    st.set_pages(0, T, TOKENS)
    stub_host = random_rows_torch(1, (LAYERS, STUB, ROW), "cuda:0").view(torch.int16).cpu().numpy().view(np.uint16)
    d = [O.Directive(0, S_START, S_END, STUB, stub_host)]
    runs, t = 0, 0.0
    new = None
    while t < seconds or runs == 0:
        a = time.perf_counter()
        new, _ = O.splice(st, d)
        t += time.perf_counter() - a
        runs += 1
    # parity of the timed GPU workload against the oracle
    for layer in range(LAYERS):
        exp = new.logical_rows(0, layer)
        got = gpu_after[layer]
        if not np.array_equal(exp[:, :512], got[:, :512]) or not np.array_equal(exp[:, 512:], got[:, 512:]):
            raise SystemExit(f"GPU splice differs from the oracle on layer {layer}")
    return {
        "value": round(alg_bytes * runs / t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the full 27-layer splice, run {runs} times ({t:.1f} s) by the numpy oracle on one core "
                  f"({len(os.sched_getaffinity(0))} available); GPU result matched it bit-exactly",
    }


if __name__ == "__main__":
    main()
