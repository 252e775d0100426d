"""Benchmark of the splice / evict hot path on one MI355X.

Default workload (the headline): a DeepSeek-V2-Lite shaped MLA cache, 27
layers, one sequence of 32768 tokens, rows c_kv 512 + k_pe 64 bf16 ~ N(0,1),
page size 16, the sequence on a random permutation of its own 2048 pages; one
AMORTIZE splice drops three 2048-token tool turns [8192, 14336) for a 24-row stub
(Delta = -6120), moving and rotating every downstream row ("Leyline: KV Cache
Directives for Agentic Inference", sections 2.1-2.3).

A step is one whole splice call through the C ABI (host plan, the plan's
expansion into page tasks on the device, one kernel launch that moves rows,
rotates k_pe and rewrites the page table) on a sequence of its own: the pool
holds one such sequence per timed step (up to 64; beyond that one sequence
has its page table restored before every splice, which also serves as the
context figure `step_with_table_restore_ms`).  `value` is the row bytes the
splice must move per step divided by the wall time per step; no launch in the
timed loop is stamped.  The roofline object times the row kernel alone, in a
separate pass, with HIP events recorded on the stream it runs on (percentiles
in `kernel_us`); its `traffic` is the HBM traffic per launch
from the rocprofv3 counter summary in profiles/, used only while that summary
was taken on the current kernel source.  The CPU baseline runs the oracle on
the same workload on the host and checks the GPU result against it; a second
leg deals the layers out over the host's cores.  Every other workload carries
the oracle timed on a bounded sample of its own shape.

Other workloads (one JSON line each, not the headline):
  --workload splice_4k_1layer        the small case: 1 layer, 4096 tokens,
                                     [1000, 3000) -> 16 rows on an identity
                                     table; launch-latency bound
  --workload splice_16x32k_27layer   16 sequences x 32768 tokens, one random
                                     directive each, one batched call
  --workload evict_256x16k_27layer_p16 / _p1
                                     KV-streams eviction of 256 rollouts x
                                     16384 tokens under random turn drops
  --workload kvs_mask_64x32k         KV-streams trainer mask for 64 rollouts x
                                     32768 tokens: death times from the
                                     eviction logs, 128 x 128 block mask and the
                                     dense bit mask (8.6 GB written)
  --workload splice_32k_27layer_inplace
                                     the headline shape with no stub: Delta =
                                     -6144 is a whole number of pages, so every
                                     downstream row only has its k_pe band
                                     turned in place (127 MB)
  --workload drift_128k_60layer      131072 tokens x 60 layers, ten successive
                                     seeded splices; per-splice GB/s and the
                                     k_pe drift per number of rotations
  --workload rope_rows_32k_27layer   per-row-angle rotation: all 32768 rows of
                                     the 27-layer MLA cache gathered with k_pe
                                     turned back by its position (2.04 GB)
  --workload rope_rows_32k_27layer_inplace
                                     the same rows' bands turned in place
  --workload evict_32x16k_llama8b_p16
                                     KV-streams eviction of 32 rollouts x
                                     16384 tokens on a Llama-3-8B shaped GQA
                                     cache (K and V planes), turn drops
  --workload splice_32k_llama8b      the headline splice on a GQA cache of
                                     Llama-3-8B shape (32 layers, K and V of 8
                                     heads x 128, RoPE on all 128, half-split,
                                     base 500000)

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "downstream KV GB/s moved+rotated (% HBM peak); splice latency @32k ctx"
HBM_PEAK_GBS = 8000.0
ROW = 576
# Measured ceiling of the in-place band pattern on MI355X: read and write the
# 128-byte k_pe line of every 1152-byte row, lines of 8 rows per load
# instruction, over 0.9 GB of band lines cycled so that no repeat hits the
# memory-side cache (best of the probe's variants; a contiguous copy of the
# same bytes runs at 6.2 TB/s).
INPLACE_CEILING_GBS = 4385.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--latency-runs", type=int, default=25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", default="splice_32k_27layer",
                    choices=["splice_32k_27layer", "splice_32k_27layer_inplace", "splice_16x32k_27layer",
                             "evict_256x16k_27layer_p16", "evict_256x16k_27layer_p1", "splice_32k_llama8b",
                             "kvs_mask_64x32k", "rope_rows_32k_27layer", "rope_rows_32k_27layer_inplace",
                             "splice_4k_1layer", "evict_32x16k_llama8b_p16", "drift_128k_60layer",
                             "compact_128x16k_27layer_p16"])
    return ap.parse_args()


# The source file of each measured kernel; its hash also covers the shared
# device helpers and the launch structures.
KERNEL_SOURCE = {"splice_kernel": "kernels.hip", "splice_inplace_kernel": "kernels.hip",
                 "evict_move_kernel": "kernels.hip", "unit_page_kernel": "kernels.hip",
                 "gqa_splice_kernel": "kernels_gqa.hip", "plane_evict_kernel": "kernels_gqa.hip",
                 "kvs_dense_ev_kernel": "kernels_kvs.hip", "rope_rows_kernel": "kernels_rows.hip",
                 "rope_gather_mla_kernel": "kernels_rows.hip", "rope_inplace_mla_kernel": "kernels_rows.hip"}


def kernel_source_sha(kernel: str) -> str:
    csrc = os.path.join(ROOT, "mla_paged_cache_amd", "csrc")
    src = KERNEL_SOURCE[kernel]
    headers = {"kernels_kvs.hip": ("device_common.h", "leyline_internal.h", "kvs_internal.h"),
               "kernels_rows.hip": ("device_common.h", "leyline_internal.h", "rows_internal.h")}.get(
        src, ("device_common.h", "leyline_internal.h"))
    h = hashlib.sha256()
    for name in (*headers, src):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing or was taken on other kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    h = re.search(r"kernel_source_sha256_16: ([0-9a-f]+)", text)
    if not m or not h or kernel_source_sha(kernel) != h.group(1):
        return None
    return int(m.group(1))


def quiet_gc():
    """Keep Python's cyclic collector off until the timed region ends: its
    pauses (tens of ms with torch loaded) would otherwise land inside the timed
    host loop and starve the GPU.  No collection is forced here: a full
    collection right before a loop walks every Python object and leaves the
    host caches cold, and the loop's first call then took 123 us on the host
    instead of 48-59 us (the GPU idles meanwhile)."""
    gc.disable()


def kernel_pass(torch, pool, kernel, run, n, prepare=None):
    """The kernel-timing pass, apart from the timed loop (which stamps no
    launch): n calls of run(i) with every launch of `kernel` stamped by HIP
    events on the stream it runs on.  Returns (launches, total_ms,
    total_bytes, per-launch ms)."""
    if prepare is not None:
        prepare()
    pool.profile_read(kernel)
    torch.cuda.synchronize()
    pool.set_profiling(True, 1)
    quiet_gc()
    for i in range(n):
        run(i)
    torch.cuda.synchronize()
    gc.enable()
    pool.set_profiling(False)
    return pool.profile_read(kernel, samples=n + 8)


def pct(samples, q):
    """q-th percentile (0..100) by linear interpolation."""
    if not samples:
        return None
    return float(np.percentile(np.asarray(samples, dtype=np.float64), q))


def torch_copy_rate(torch, dev, n_bytes):
    """torch's own device copy (`dst.copy_(src)`, rocclr's copy kernel) of
    n_bytes read + written, GB/s, for context -- not a ceiling: hand-written
    copies run faster.  At least 1 GiB, so that repeats do not run out of the
    memory-side cache.  The counter runs also use this copy to calibrate
    FETCH_SIZE and WRITE_SIZE."""
    n_bytes = max(n_bytes, 1 << 30)
    src = torch.empty(n_bytes, dtype=torch.uint8, device=dev)
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
    return 2 * n_bytes * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9


def roofline(kernel, workload, launches, kernel_ms, kernel_bytes, samples=None):
    k_avg_ms = kernel_ms / max(1, launches)
    per = kernel_bytes // max(1, launches)
    achieved = per / (k_avg_ms * 1e-3) / 1e9 if k_avg_ms > 0 else 0.0
    out = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": profiled_traffic(kernel, workload),
        "kernel": kernel,
        "kernel_avg_us": round(k_avg_ms * 1e3, 2),
        "timed_launches": launches,
        "bytes_per_launch": per,
    }
    if samples:
        out["kernel_us"] = {"median": round(pct(samples, 50) * 1e3, 2), "p10": round(pct(samples, 10) * 1e3, 2),
                            "p90": round(pct(samples, 90) * 1e3, 2), "samples": len(samples)}
    return out


def base_line(args, workload, value, ms_per_step, config):
    return {
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
        "config": {"workload": workload, **config},
    }


# ------------------------------------------------------------------ splice --

def bench_drift(args):
    """Long context: one sequence of 131072 tokens, 60 layers, page size 16,
    randomly permuted pages in a pool of 16384, takes 10 successive seeded
    AMORTIZE splices (span U[1024, 16384], stub U[8, 64], start
    U[1024, len - span]) with the rotation in float32 on bf16 storage
    ("Leyline", section 4.3: the error stays small and grows sub-linearly
    with fp32 rotation).  A step is one splice; the ten are the workload, so
    --steps is not used.  Three passes over the same ten directives from the
    same initial table: the first untimed (its tables are checked against the
    oracle's page plan, and two layers whose k_pe was stored as
    bf16(RoPE(i) k) give the drift per number of rotations a row went
    through); the second times the ten calls back to back (value); the third
    stamps every launch (roofline, per splice)."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from oracle import leyline_oracle as O
    from synth import draw_span, np_rng, permuted_pages, random_normal_np, random_rows_np, random_rows_torch

    LAYERS, TOKENS, PAGE, POOL_PAGES, SPLICES = 60, 131072, 16, 16384, 10
    TRACKED = (0, 59)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data = random_rows_torch(5, (LAYERS, POOL_PAGES, PAGE, ROW), dev)
    table = torch.full((1, POOL_PAGES), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    T = permuted_pages(5, TOKENS // PAGE)
    j = np.arange(TOKENS)
    phys = np.asarray(T, np.int64)[j // PAGE] * PAGE + j % PAGE
    phys_dev = torch.from_numpy(phys).to(dev)

    def roped(seed, positions):
        n = len(positions)
        rows = random_rows_np(seed, (n, ROW))
        k = random_normal_np(seed, (n, O.ROPE_DIM))
        rows[:, O.KV_LORA_RANK:] = O.f32_to_bf16(O.rotate_f64(k, positions).astype(np.float32))
        return rows, k

    k_raw = {}
    for layer in TRACKED:
        rows, k_raw[layer] = roped(100 + layer, j)
        data[layer].view(-1, ROW)[phys_dev] = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to(dev)
    rng = np_rng(5, 7)
    plan = O.CacheState.empty(0, POOL_PAGES, PAGE, POOL_PAGES, with_rows=False)
    plan.set_pages(0, T, TOKENS)
    dirs, stubs, spans, expected = [], [], [], []
    origin = np.arange(TOKENS)
    turns = np.zeros(TOKENS, np.int64)
    for k in range(SPLICES):
        n = plan.lengths[0]
        d = draw_span(rng, n, 1024, 16384, 8, 64)
        delta = d.r_len - (d.s_end - d.s_start)
        stub = random_rows_torch(2000 + k, (LAYERS, d.r_len, ROW), dev)
        for layer in TRACKED:
            rows, _ = roped(1000 * k + layer, np.arange(d.s_start, d.s_start + d.r_len))
            stub[layer] = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16).to(dev)
        stubs.append(stub)
        dirs.append([L.Directive(0, d.s_start, d.s_end, stub)])
        spans.append((d.s_start, d.s_end, d.r_len))
        kind, index, down = O.splice_sources(n, d.s_start, d.s_end, d.r_len)
        origin = np.where(kind == 0, origin[np.where(kind == 0, index, 0)], -1)
        turns = np.where(kind == 0, turns[np.where(kind == 0, index, 0)] + (down & (delta != 0)), 0)
        # the oracle's page plan only (no rows on the host): the stub is a placeholder
        plan, _ = O.splice(plan, [O.Directive(0, d.s_start, d.s_end, d.r_len, ())])
        expected.append((plan.lengths[0], plan.next_pos[0], list(plan.tables[0])))

    def restore():
        pool.seq_set_pages(0, T, TOKENS)
        torch.cuda.synchronize()

    # pass 1: untimed; tables against the oracle's plan, drift of two layers
    restore()
    per_bytes = []
    for k in range(SPLICES):
        pool.splice(dirs[k])
        n2, pos, pages = pool.seq_get(0)
        if (n2, pos, list(pages)) != expected[k]:
            raise SystemExit(f"splice {k}: the GPU page plan differs from the oracle's")
        per_bytes.append(pool.last_stats().alg_bytes)
    torch.cuda.synchronize()
    n = plan.lengths[0]
    jj = np.arange(n)
    pages = np.asarray(plan.tables[0], np.int64)
    ph = torch.from_numpy(pages[jj // PAGE] * PAGE + jj % PAGE).to(dev)
    keep = origin >= 0
    drift, glob = {}, {}
    for layer in TRACKED:
        got = data[layer].view(-1, ROW)[ph].view(torch.int16).cpu().numpy().view(np.uint16)
        kpe = O.bf16_to_f32(got[keep, O.KV_LORA_RANK:]).astype(np.float64)
        fresh = O.rotate_f64(k_raw[layer][origin[keep]], jj[keep])
        t = turns[keep]
        glob[layer] = float(np.linalg.norm(kpe - fresh) / np.linalg.norm(fresh))
        for kk in np.unique(t):
            m = t == kk
            err = float(np.linalg.norm(kpe[m] - fresh[m]) / np.linalg.norm(fresh[m]))
            cur = drift.setdefault(int(kk), {"rows": int(m.sum()), "rel_l2": 0.0})
            cur["rel_l2"] = max(cur["rel_l2"], err)

    # pass 2: the ten calls back to back, nothing stamped
    for _ in range(max(1, args.warmup // 5)):
        restore()
        for k in range(SPLICES):
            pool.splice(dirs[k])
    restore()
    quiet_gc()
    t0 = time.perf_counter()
    for k in range(SPLICES):
        pool.splice(dirs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_per_splice = (t1 - t0) * 1e3 / SPLICES
    total = sum(per_bytes)
    # pass 3: every launch stamped
    restore()
    launches, kernel_ms, kernel_bytes, samples = kernel_pass(torch, pool, 0, lambda k: pool.splice(dirs[k]), SPLICES)
    out = base_line(args, "drift_128k_60layer", total / (ms_per_splice * 1e-3 * SPLICES) / 1e9, ms_per_splice, {
        "layers": LAYERS, "tokens": TOKENS, "page_size": PAGE, "pool_pages": POOL_PAGES, "splices": SPLICES,
        "directives": [list(x) for x in spans], "alg_bytes_per_splice": per_bytes,
        "draws": "span U[1024,16384], stub U[8,64], start U[1024,len-span], seeded",
        "storage": "bf16 rows c_kv 512 + k_pe 64, rotation in f32"})
    out["steps"] = SPLICES
    out["roofline"] = roofline("splice_kernel", "drift_128k_60layer", launches, kernel_ms, kernel_bytes)
    out["roofline"]["per_splice_gbs"] = [round(b / (ms * 1e-3) / 1e9, 1) for b, ms in zip(per_bytes, samples)]
    out["drift"] = {"protocol": "k_pe stored as bf16(RoPE_f64(i) k), k ~ N(0,1), layers 0 and 59; relative L2 "
                                "to float64 RoPE at the final position, the worse layer, per number of rotations",
                    "by_rotations": {str(k): v for k, v in sorted(drift.items())},
                    "all_rows": round(max(glob.values()), 6),
                    "sqrt_law": "1.66e-3 * sqrt(k + 1)"}
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_drift(T, spans[0], per_bytes[0], LAYERS,
                                                                               TOKENS, PAGE, POOL_PAGES)
    pool.close()
    return out


def cpu_baseline_drift(T, span, alg_bytes, LAYERS, TOKENS, PAGE, POOL_PAGES):
    """The oracle's first splice of the drift workload, in full: all 60
    layers of the 131072-token sequence, the whole 16384-page pool held on the
    host (18 GB), run once."""
    from oracle import leyline_oracle as O
    st = O.CacheState.empty(0, POOL_PAGES, PAGE, POOL_PAGES, with_rows=False)
    st.layers = host_pool(LAYERS, POOL_PAGES, PAGE, ROW)
    st.set_pages(0, T, TOKENS)
    s0, s1, r = span
    d = [O.Directive(0, s0, s1, r, [np.full((r, ROW), 0x3F80, np.uint16)] * LAYERS)]
    a = time.perf_counter()
    O.splice(st, d)
    t = time.perf_counter() - a
    return oracle_line(alg_bytes, 1, t, f"the first of the ten splices in full ({LAYERS} layers, {TOKENS} tokens, "
                                        f"{POOL_PAGES}-page pool on the host)")


MAX_DISTINCT_SEQS = 64


def bench_splice_32k(args, STUB=24, workload="splice_32k_27layer", kernel="splice_kernel"):
    """The headline.  Every timed step splices its own 32k x 27 sequence: up to
    64 identically shaped sequences, each a random permutation of its own 2048
    pages, sit above a spare region that holds every step's fresh pages, so
    each step's fresh pages are one run of consecutive ids (as in a pool that
    holds the one sequence) and no table restore runs between steps.  The
    JSON also gives, for context, the step that restores one sequence's table
    before each splice, and the step with the host-staged page plan.

    With STUB = 0 (splice_32k_27layer_inplace) Delta = -6144 is a whole
    number of pages: no page is fresh, and every downstream row only has its
    k_pe band turned in place (splice_inplace_kernel).  Each step's sequence is
    its own, so the bands it turns are read from HBM, not from the last step's
    caches."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import permuted_pages, random_rows_torch

    LAYERS, TOKENS, PAGE = 27, 32768, 16
    S_START, S_END = 8192, 14336
    NP = TOKENS // PAGE
    # Delta = -6120 is not a multiple of the page size, so every new page from
    # the one holding s_start on is fresh; Delta = -6144 is, and s_start is on
    # a page boundary, so then no page is fresh
    new_pages = -(-(TOKENS + STUB - (S_END - S_START)) // PAGE)
    FRESH = 0 if (STUB - (S_END - S_START)) % PAGE == 0 else new_pages - S_START // PAGE
    distinct = args.steps <= MAX_DISTINCT_SEQS
    NSEQ = args.steps if distinct else 1
    SPARE = max(NSEQ, 2) * FRESH
    POOL_PAGES = SPARE + NSEQ * NP
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data = torch.empty((LAYERS, POOL_PAGES, PAGE, ROW), dtype=torch.bfloat16, device=dev)
    data[:, :SPARE].zero_()
    for s in range(NSEQ):
        data[:, SPARE + s * NP:SPARE + (s + 1) * NP] = random_rows_torch(s, (LAYERS, NP, PAGE, ROW), dev)
    stub = random_rows_torch(1000, (LAYERS, STUB, ROW), dev) if STUB else None
    table = torch.full((NSEQ, NP + 8), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    T0 = permuted_pages(0, NP)                       # sequence 0: the oracle's table
    tables = [T0 + SPARE] + [permuted_pages(s, NP, start=SPARE + s * NP) for s in range(1, NSEQ)]
    directive = [L.Directive(0, S_START, S_END, stub)]

    def restore():
        pool.seq_set_pages(0, tables[0], TOKENS)

    def set_all():
        for s in range(1, NSEQ):
            if s in live:
                pool.seq_free(s)
        restore()
        for s in range(1, NSEQ):
            pool.seq_set_pages(s, tables[s], TOKENS)
            live.add(s)
        torch.cuda.synchronize()

    live = set()
    host_before = None
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        host_before = data[:, SPARE:SPARE + NP].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    restore()
    pool.splice(directive)
    torch.cuda.synchronize()
    st = pool.last_stats()
    alg_bytes = st.alg_bytes
    assert st.fresh_pages == FRESH and st.planned_on_device == 1, st
    _, _, new_table = pool.seq_get(0)
    gpu_after = None
    if host_before is not None:
        j = np.arange(TOKENS + STUB - (S_END - S_START))
        phys = torch.from_numpy(new_table.astype(np.int64)[j // PAGE] * PAGE + j % PAGE).to(dev)
        gpu_after = data.view(LAYERS, -1, ROW)[:, phys].view(torch.int16).cpu().numpy().view(np.uint16)

    def timed(run, n):
        """Host milliseconds per call of n calls, bracketed by synchronize."""
        torch.cuda.synchronize()
        quiet_gc()
        t0 = time.perf_counter()
        for i in range(n):
            run(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        return (t1 - t0) * 1e3 / n

    def device_timed(run, n):
        """Device milliseconds per call of the same loop: one event pair
        around all n calls (the pair itself costs stream time, so the host
        loop above runs without it)."""
        torch.cuda.synchronize()
        quiet_gc()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e1.record()  # creates the event outside the timed region (torch creates it at its first record)
        e0.record()
        for i in range(n):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        gc.enable()
        return e0.elapsed_time(e1) / n

    def restore_step(_):
        restore()
        pool.splice(directive)

    dirs = [[L.Directive(s, S_START, S_END, stub)] for s in range(NSEQ)]

    def distinct_step(i):
        pool.splice(dirs[i])

    for _ in range(args.warmup):
        restore_step(0)
    # context: one sequence, its table restored before every splice
    ms_restore = timed(restore_step, args.steps)
    # throughput: K whole splices, bracketed by synchronize; no launch in
    # this loop is stamped and no event recorded
    step = distinct_step if distinct else restore_step
    if distinct:
        # warm-up pass of the timed step itself: every sequence spliced once,
        # then all tables set back.  In serving, a sequence's pages are read
        # by attention at every decode step before it is spliced; pages left
        # idle behind other traffic since they were filled made the first
        # splice's kernel about 2% slower (183.2 against 179.7 us under the
        # tracer) and the 20-step loop 4-6 us per step slower.
        set_all()
        for s in range(NSEQ):
            distinct_step(s)
        set_all()
    ms_per_step = timed(step, args.steps)
    if distinct:
        set_all()
    step_device_ms = device_timed(step, args.steps)
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    # the row kernel's own time: a separate pass with every launch stamped
    launches, kernel_ms, kernel_bytes, samples = kernel_pass(torch, pool, 0, step, args.steps,
                                                             set_all if distinct else None)
    ms_host_plan = None
    if distinct:
        set_all()
        pool.set_splice_planner(L.SPLICE_PLAN_HOST)
        ms_host_plan = timed(distinct_step, args.steps)
        pool.set_splice_planner(L.SPLICE_PLAN_AUTO)

    # latency: API call to stream completion, MALL flushed before each run
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    lat, host = [], []
    quiet_gc()
    for _ in range(args.latency_runs):
        restore()
        flush.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        pool.splice(directive)
        b = time.perf_counter()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - a) * 1e6)
        host.append((b - a) * 1e6)
    gc.enable()
    del flush

    out = base_line(args, workload, value, ms_per_step, {
        "layers": LAYERS, "tokens": TOKENS, "page_size": PAGE, "span": [S_START, S_END], "stub_rows": STUB,
        "delta": STUB - (S_END - S_START), "storage": "bf16 rows c_kv 512 + k_pe 64, rotation in f32",
        "alg_bytes_per_step": alg_bytes, "fresh_pages": st.fresh_pages,
        "rows_turned_in_place_per_layer": st.rows_rotated_inplace,
        "sequences": f"{NSEQ} of this shape, one spliced per step, each on its own randomly permuted pages"
                     if distinct else "one, its page table restored before every splice (more steps than "
                                      f"{MAX_DISTINCT_SEQS} distinct sequences)",
        "pool_pages": POOL_PAGES})
    out["pct_hbm_peak"] = round(100.0 * value / HBM_PEAK_GBS, 2)
    # the same loop on the device's clock: one event pair around all the calls
    # (the events sit on the pool's stream; the first call's host time is
    # inside the span)
    out["step_device_us"] = round(step_device_ms * 1e3, 2)
    out["step_with_table_restore_ms"] = round(ms_restore, 5)
    if ms_host_plan is not None:
        out["step_host_staged_plan_ms"] = round(ms_host_plan, 5)
    out["splice_latency_us"] = {"median": round(statistics.median(lat), 1), "min": round(min(lat), 1),
                                "max": round(max(lat), 1), "runs": len(lat),
                                "host_call_median": round(statistics.median(host), 1)}
    out["roofline"] = roofline(kernel, workload, launches, kernel_ms, kernel_bytes, samples)
    out["torch_copy_gbs"] = round(torch_copy_rate(torch, dev, alg_bytes // 2), 1)
    out["cpu_baseline"] = None
    if host_before is not None:
        out["cpu_baseline"] = cpu_baseline_splice(host_before, gpu_after, T0, alg_bytes, args.cpu_seconds,
                                                  LAYERS, TOKENS, PAGE, 2 * NP, S_START, S_END, STUB)
        del host_before, gpu_after
        out["cpu_baseline_layer_parallel"] = cpu_baseline_layer_parallel(
            T0, alg_bytes, args.cpu_seconds / 2, LAYERS, TOKENS, PAGE, 2 * NP, S_START, S_END, STUB)
    pool.close()
    return out


def cpu_baseline_splice(host_before, gpu_after, T, alg_bytes, seconds, LAYERS, TOKENS, PAGE, POOL_PAGES,
                        S_START, S_END, STUB, stub_seed=1000):
    """The oracle, as it stands, on the same splice on the host: repeated
    until `seconds` have passed; also checks the GPU result against it.
    host_before holds the sequence's pages (T is a permutation of them); the
    oracle's pool adds free pages after them up to POOL_PAGES."""
    import torch
    from oracle import leyline_oracle as O
    from synth import random_rows_torch

    st = O.CacheState.empty(0, POOL_PAGES, PAGE, TOKENS // PAGE + 8, with_rows=False)
    pad = np.zeros((POOL_PAGES - host_before.shape[1], PAGE, ROW), np.uint16)
    st.layers = [np.concatenate([host_before[i], pad]) for i in range(LAYERS)]
    st.set_pages(0, T, TOKENS)
    stub_host = random_rows_torch(stub_seed, (LAYERS, STUB, ROW), "cuda:0").view(torch.int16).cpu().numpy().view(
        np.uint16) if STUB else None
    d = [O.Directive(0, S_START, S_END, STUB, stub_host)]
    runs, t = 0, 0.0
    new = None
    while t < seconds or runs == 0:
        a = time.perf_counter()
        new, _ = O.splice(st, d)
        t += time.perf_counter() - a
        runs += 1
    for layer in range(LAYERS):
        if not np.array_equal(new.logical_rows(0, layer), gpu_after[layer]):
            raise SystemExit(f"GPU splice differs from the oracle on layer {layer}")
    return {
        "value": round(alg_bytes * runs / t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"the full {LAYERS}-layer splice, run {runs} times ({t:.1f} s) by the numpy oracle on one core "
                  f"({len(os.sched_getaffinity(0))} available, {cpu_model()}); GPU result matched it bit-exactly",
    }


def bench_splice_4k(args):
    """The small case: one layer, 4096 tokens, page size 16, identity page
    table (pages 0..255) in a pool of 512 pages; [1000, 3000) spliced for a
    16-row stub (Delta = -1984, a whole number of pages: 68 downstream pages
    are reused and turned in place, 2 pages are fresh).  Launch-latency bound;
    the figure that matters is the call's latency.  Restoring the table does
    not undo the in-place turn, so each step turns those rows again (the same
    work every step)."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import random_rows_torch

    TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB = 4096, 16, 512, 1000, 3000, 16
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data = random_rows_torch(0, (1, POOL_PAGES, PAGE, ROW), dev)
    stub = random_rows_torch(1, (1, STUB, ROW), dev)
    table = torch.full((1, TOKENS // PAGE + 8), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    T = np.arange(TOKENS // PAGE, dtype=np.int32)
    directive = [L.Directive(0, S_START, S_END, stub)]

    def restore():
        pool.seq_set_pages(0, T, TOKENS)

    restore()
    pool.splice(directive)
    torch.cuda.synchronize()
    st = pool.last_stats()
    alg_bytes = st.alg_bytes
    for _ in range(args.warmup):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    quiet_gc()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    def step(_):
        restore()
        pool.splice(directive)

    launches, kernel_ms, kernel_bytes, samples = kernel_pass(torch, pool, 0, step, args.steps)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    lat, call = [], []
    quiet_gc()
    for _ in range(args.latency_runs):
        restore()
        flush.zero_()
        torch.cuda.synchronize()
        a = time.perf_counter()
        pool.splice(directive)
        b = time.perf_counter()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - a) * 1e6)
        call.append((b - a) * 1e6)
    gc.enable()
    del flush
    out = base_line(args, "splice_4k_1layer", alg_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": 1, "tokens": TOKENS, "page_size": PAGE, "pool_pages": POOL_PAGES, "table": "identity",
        "span": [S_START, S_END], "stub_rows": STUB, "delta": STUB - (S_END - S_START),
        "reused_pages_turned_in_place": st.rows_rotated_inplace // PAGE, "fresh_pages": st.fresh_pages,
        "alg_bytes_per_step": alg_bytes})
    out["splice_latency_us"] = {"median": round(statistics.median(lat), 1), "min": round(min(lat), 1),
                                "max": round(max(lat), 1), "runs": len(lat),
                                "host_call_median": round(statistics.median(call), 1)}
    out["roofline"] = roofline("splice_kernel", "splice_4k_1layer", launches, kernel_ms, kernel_bytes, samples)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_small(
        args.cpu_seconds / 4, alg_bytes, TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB)
    pool.close()
    return out


# ------------------------------------------------- oracle baselines --
# Each workload's oracle leg: the oracle as it stands, on one host core, on
# seeded host rows of the workload's shape (the values do not change the work
# it does; parity of the GPU against the oracle is the tests' job), timed
# around the oracle's own call only.

def timed_oracle(run, seconds):
    """Repeat `run` until `seconds` of its own time have passed; returns
    (runs, seconds spent, the first run's result)."""
    runs, t, first = 0, 0.0, None
    while t < seconds or runs == 0:
        a = time.perf_counter()
        res = run()
        t += time.perf_counter() - a
        if runs == 0:
            first = res
        runs += 1
    return runs, t, first


def oracle_line(bytes_per_run, runs, t, sample, **extra):
    out = {"value": round(bytes_per_run * runs / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{sample}; {runs} run(s) in {t:.1f} s on one core "
                     f"({len(os.sched_getaffinity(0))} available, {cpu_model()})"}
    out.update(extra)
    return out


def host_pool(n_arrays, pool_pages, page, width):
    """Host layer arrays of bf16 1.0 (the oracle copies and turns bits; the
    values do not change its work)."""
    return [np.full((pool_pages, page, width), 0x3F80, np.uint16) for _ in range(n_arrays)]


def cpu_baseline_evict(masks, page, seconds, LAYERS, TOKENS, ROLL, reuse=True):
    """The oracle's eviction on 8 of the rollouts (all layers, the same masks,
    the same pool shape per rollout; reuse False: page reuse off)."""
    from oracle import leyline_oracle as O
    from synth import permuted_pages
    k = 8
    per = TOKENS // page
    pool_pages = k * per + (k * per if not reuse else (k * per // 2 if page > 1 else 0))
    st = O.CacheState.empty(0, pool_pages, page, per, with_rows=False)
    st.layers = host_pool(LAYERS, pool_pages, page, ROW)
    perm = permuted_pages(0, k * per)
    for r in range(k):
        st.set_pages(r, perm[r * per:(r + 1) * per], TOKENS)
    ms = [masks[r * TOKENS:(r + 1) * TOKENS] for r in range(k)]
    runs, t, (_, plans) = timed_oracle(lambda: O.evict(st, list(range(k)), ms, reuse_pages=reuse), seconds)
    nb = sum(O.algorithmic_bytes(pl, int(m.sum()), page, np.zeros(int(m.sum()), np.int64),
                                 np.zeros(int(m.sum()), bool), 0, LAYERS, rotate=False) for pl, m in zip(plans, ms))
    return oracle_line(nb, runs, t, f"{k} of the {ROLL} rollouts, all {LAYERS} layers, the same masks",
                       ms_per_call_all_rollouts=round(t / runs * 1e3 * ROLL / k, 1))


def cpu_baseline_batched(dir_spans, seconds, LAYERS, TOKENS, PAGE):
    """The oracle's batched splice on 4 of the 16 sequences (their own
    directives, all layers), pool pages twice theirs (as on the GPU)."""
    from oracle import leyline_oracle as O
    from synth import permuted_pages
    k = 4
    per = TOKENS // PAGE
    pool_pages = 2 * k * per
    st = O.CacheState.empty(0, pool_pages, PAGE, per + 8, with_rows=False)
    st.layers = host_pool(LAYERS, pool_pages, PAGE, ROW)
    perm = permuted_pages(0, k * per)
    dirs, nb = [], 0
    for s in range(k):
        st.set_pages(s, perm[s * per:(s + 1) * per], TOKENS)
        s0, s1, r = dir_spans[s]
        dirs.append(O.Directive(s, s0, s1, r, [np.full((r, ROW), 0x3F80, np.uint16)] * LAYERS if r else None))
    runs, t, (_, plans) = timed_oracle(lambda: O.splice(st, dirs), seconds)
    for (s0, s1, r), pl in zip(dir_spans[:k], plans):
        kind, index, down = O.splice_sources(TOKENS, s0, s1, r)
        nb += O.algorithmic_bytes(pl, len(kind), PAGE, kind, down, r - (s1 - s0), LAYERS)
    return oracle_line(nb, runs, t, f"{k} of the 16 sequences with their own directives, all {LAYERS} layers")


def cpu_baseline_gqa(seconds, HEADS, HEAD_DIM, TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB, layers=8):
    """The oracle's GQA splice (half-split pairs, base 500000) on `layers` of
    the 32 layers (K and V arrays)."""
    from oracle import leyline_oracle as O
    from synth import permuted_pages
    specs = []
    for _ in range(layers):
        specs += [O.gqa_k_row(HEADS, HEAD_DIM, HEAD_DIM), O.plain_row(HEADS * HEAD_DIM)]
    st = O.CacheState.empty(len(specs), POOL_PAGES, PAGE, TOKENS // PAGE + 8, with_rows=False, specs=specs)
    st.layers = host_pool(len(specs), POOL_PAGES, PAGE, HEADS * HEAD_DIM)
    st.set_pages(0, permuted_pages(0, TOKENS // PAGE), TOKENS)
    stub = [np.full((STUB, HEADS * HEAD_DIM), 0x3F80, np.uint16)] * len(specs)
    d = [O.Directive(0, S_START, S_END, STUB, stub)]
    runs, t, (_, plans) = timed_oracle(lambda: O.splice(st, d, pairing="half", base=500000.0), seconds)
    kind, index, down = O.splice_sources(TOKENS, S_START, S_END, STUB)
    nb = O.algorithmic_bytes(plans[0], len(kind), PAGE, kind, down, STUB - (S_END - S_START), layers, specs=specs)
    return oracle_line(nb, runs, t, f"{layers} of the 32 layers (K and V), the same splice")


def cpu_baseline_kvs(rolls, seconds, TOKENS):
    """The mask oracle (death times, 128 x 128 block lists, dense bits) for
    one rollout of the batch."""
    from oracle import kvs_mask_oracle as K
    n, events = rolls[0]

    def run():
        d = K.death_times(TOKENS, n, events)
        vis = K.visibility(d)
        K.block_mask(vis, 128, 128)
        K.dense_bits(vis)

    runs, t, _ = timed_oracle(run, seconds)
    return oracle_line(TOKENS * TOKENS // 8, runs, t, f"rollout 0 of {len(rolls)}: death times, block lists, "
                       "dense bits (dense bytes counted, as on the GPU line)")


def cpu_baseline_rope(seconds, LAYERS, TOKENS, PAGE, POOL_PAGES, in_place=False):
    """The oracle's per-row rotation (angle -p for row p) of the whole
    sequence, all layers, gathered or in place."""
    from oracle import leyline_oracle as O
    from synth import permuted_pages
    st = O.CacheState.empty(0, POOL_PAGES, PAGE, TOKENS // PAGE + 8, with_rows=False)
    st.layers = host_pool(LAYERS, POOL_PAGES, PAGE, ROW)
    st.set_pages(0, permuted_pages(0, TOKENS // PAGE), TOKENS)
    angles = -np.arange(TOKENS, dtype=np.int64)
    if in_place:
        runs, t, _ = timed_oracle(lambda: O.rope_rows(st, 0, 0, angles, in_place=True), seconds)
        return oracle_line(LAYERS * TOKENS * 2 * 128, runs, t, f"all {TOKENS} rows, all {LAYERS} layers, in place")
    runs, t, _ = timed_oracle(lambda: O.rope_rows(st, 0, 0, angles), seconds)
    return oracle_line(LAYERS * TOKENS * 2 * ROW * 2, runs, t, f"all {TOKENS} rows, all {LAYERS} layers, gathered")


def cpu_baseline_small(seconds, alg_bytes, TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB):
    """The oracle's splice of the one-layer 4k case."""
    from oracle import leyline_oracle as O
    st = O.CacheState.empty(0, POOL_PAGES, PAGE, TOKENS // PAGE + 8, with_rows=False)
    st.layers = host_pool(1, POOL_PAGES, PAGE, ROW)
    st.set_pages(0, np.arange(TOKENS // PAGE), TOKENS)
    d = [O.Directive(0, S_START, S_END, STUB, [np.full((STUB, ROW), 0x3F80, np.uint16)])]
    runs, t, _ = timed_oracle(lambda: O.splice(st, d), seconds)
    return oracle_line(alg_bytes, runs, t, "the same one-layer splice", ms_per_call=round(t / runs * 1e3, 3))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_layer_barrier = None


def _set_layer_barrier(b):
    global _layer_barrier
    _layer_barrier = b


def _oracle_layers_worker(task):
    """One process of the layer-parallel oracle leg: seeded N(0,1) bf16 rows
    for its own layers of the same pool shape, then, once every process is
    ready, the oracle's splice on them until `seconds` have passed."""
    seed, n_layers, pool_pages, page, tokens, T, s_start, s_end, stub, seconds = task
    from oracle import leyline_oracle as O
    rng = np.random.default_rng(seed)
    st = O.CacheState.empty(0, pool_pages, page, tokens // page + 8, with_rows=False)
    st.layers = [O.f32_to_bf16(rng.standard_normal((pool_pages, page, ROW), dtype=np.float32))
                 for _ in range(n_layers)]
    st.set_pages(0, T, tokens)
    stub_rows = O.f32_to_bf16(rng.standard_normal((n_layers, stub, ROW), dtype=np.float32)) if stub else None
    d = [O.Directive(0, s_start, s_end, stub, stub_rows)]
    _layer_barrier.wait(timeout=300)
    runs, t = 0, 0.0
    while t < seconds or runs == 0:
        a = time.perf_counter()
        O.splice(st, d)
        t += time.perf_counter() - a
        runs += 1
    return runs, t


def cpu_baseline_layer_parallel(T, alg_bytes, seconds, LAYERS, TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB):
    """The same oracle on all host cores (at most 16 processes), the layers
    dealt out among them: each process splices its own layers (same pool
    shape, same directive, its own seeded rows).  Throughput is the sum over
    processes of their layers' bytes per second of splice time."""
    import multiprocessing as mp
    n = max(1, min(16, len(os.sched_getaffinity(0)), LAYERS))
    counts = [LAYERS // n + (1 if i < LAYERS % n else 0) for i in range(n)]
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(n)
    tasks = [(1000 + i, c, POOL_PAGES, PAGE, TOKENS, T, S_START, S_END, STUB, seconds) for i, c in enumerate(counts)]
    with ctx.Pool(n, initializer=_set_layer_barrier, initargs=(barrier,)) as pool:
        res = pool.map(_oracle_layers_worker, tasks, chunksize=1)
    per_layer = alg_bytes / LAYERS
    value = sum(c * per_layer * runs / t for c, (runs, t) in zip(counts, res))
    return {
        "value": round(value / 1e9, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle, layer-parallel",
        "sample": f"the 27-layer splice, layers dealt over {n} processes ({counts[0]} or {counts[-1]} layers each, "
                  f"same pool shape and directive, own seeded rows), each repeating its share for {seconds:.0f} s; "
                  f"host {cpu_model()}",
    }


def bench_splice_batched(args):
    """16 sequences x 32768 tokens x 27 layers in one pool, one random
    directive each (span U[256,8192], stub U[8,64], start U[1024,len-span]),
    applied in one call.  As in the headline, every timed step splices
    sequences of its own: the pool holds SETS sets of 16 such sequences, each
    sequence on a random permutation of its own 2048 pages, above a spare
    region that holds every step's fresh pages.  The tables are restored only
    after every SETS steps, outside the timed region (which adds up exactly
    `steps` calls)."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import draw_span, np_rng, permuted_pages, random_rows_torch

    LAYERS, TOKENS, PAGE, SEQS = 27, 32768, 16, 16
    per = TOKENS // PAGE
    rng = np_rng(0, 4)
    draws = [draw_span(rng, TOKENS, 256, 8192, 8, 64) for _ in range(SEQS)]
    # fresh pages of one set, at most: every new page from the one holding s_start
    fresh_bound = sum(-(-(TOKENS + d.r_len - (d.s_end - d.s_start)) // PAGE) - d.s_start // PAGE for d in draws)
    page_bytes = LAYERS * PAGE * ROW * 2
    SETS = max(1, min(args.steps, 6, int(160e9 // ((SEQS * per + fresh_bound) * page_bytes))))
    SPARE = SETS * fresh_bound
    POOL_PAGES = SPARE + SETS * SEQS * per
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data = torch.empty((LAYERS, POOL_PAGES, PAGE, ROW), dtype=torch.bfloat16, device=dev)
    data[:, :SPARE].zero_()
    for k in range(SETS):
        lo = SPARE + k * SEQS * per
        data[:, lo:lo + SEQS * per] = random_rows_torch(k, (LAYERS, SEQS * per, PAGE, ROW), dev)
    table = torch.full((SETS * SEQS, per + 8), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    tables = [permuted_pages(i, per, start=SPARE + i * per) for i in range(SETS * SEQS)]
    stubs = [random_rows_torch(100 + s, (LAYERS, d.r_len, ROW), dev) for s, d in enumerate(draws)]
    dirs = [[L.Directive(k * SEQS + s, d.s_start, d.s_end, stubs[s]) for s, d in enumerate(draws)]
            for k in range(SETS)]
    spans = [(d.s_start, d.s_end, d.r_len) for d in draws]

    def restore():
        for i in range(SETS * SEQS):
            pool.seq_set_pages(i, tables[i], TOKENS)
        torch.cuda.synchronize()

    restore()
    pool.splice(dirs[0])
    torch.cuda.synchronize()
    st = pool.last_stats()
    alg_bytes = st.alg_bytes
    assert st.planned_on_device == 1 and st.fresh_pages <= fresh_bound, st

    def chunks(n, run, after=None):
        """n calls, SETS at a time after a restore; returns the seconds spent
        inside the chunks (restores excluded)."""
        spent, done = 0.0, 0
        while done < n:
            m = min(SETS, n - done)
            restore()
            quiet_gc()
            t0 = time.perf_counter()
            for k in range(m):
                run(k)
            torch.cuda.synchronize()
            spent += time.perf_counter() - t0
            gc.enable()
            if after is not None:
                after()
            done += m
        return spent

    def step(k):
        pool.splice(dirs[k])

    chunks(args.warmup, step)
    spent = chunks(args.steps, step)
    # kernel pass: every launch of the row kernel stamped, same chunks
    pool.profile_read(0)
    torch.cuda.synchronize()
    pool.set_profiling(True, 1)
    chunks(args.steps, step)
    pool.set_profiling(False)
    launches, kernel_ms, kernel_bytes, samples = pool.profile_read(0, samples=args.steps + 8)
    ms_per_step = spent * 1e3 / args.steps
    out = base_line(args, "splice_16x32k_27layer", alg_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": LAYERS, "tokens": TOKENS, "sequences": SEQS, "page_size": PAGE, "pool_pages": POOL_PAGES,
        "sets": SETS, "alg_bytes_per_step": alg_bytes,
        "layout": "each sequence on a random permutation of its own 2048 pages; fresh pages from a spare region",
        "step": f"one 16-directive splice call on a set of its own; tables restored after every {SETS} calls, "
                f"outside the timed region"})
    out["roofline"] = roofline("splice_kernel", "splice_16x32k_27layer", launches, kernel_ms, kernel_bytes, samples)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_batched(
        spans, args.cpu_seconds, LAYERS, TOKENS, PAGE)
    pool.close()
    return out


def bench_splice_gqa(args):
    """The headline splice ([8192, 14336) -> 24 stub rows on one 32768-token
    sequence, page size 16, permuted pages) on a GQA cache of Llama-3-8B
    shape: 32 layers, K and V planes of 8 KV heads x 128, RoPE on all 128
    dims of each K head (half-split pairs, base 500000)."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import permuted_pages, random_rows_torch

    LAYERS, HEADS, HEAD_DIM, TOKENS, PAGE, POOL_PAGES = 32, 8, 128, 32768, 16, 4096
    S_START, S_END, STUB = 8192, 14336, 24
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = random_rows_torch(0, (LAYERS, POOL_PAGES, PAGE, HEADS, HEAD_DIM), dev)
    v = random_rows_torch(1, (LAYERS, POOL_PAGES, PAGE, HEADS, HEAD_DIM), dev)
    k_stub = random_rows_torch(2, (LAYERS, STUB, HEADS, HEAD_DIM), dev)
    v_stub = random_rows_torch(3, (LAYERS, STUB, HEADS, HEAD_DIM), dev)
    table = torch.full((1, TOKENS // PAGE + 8), -1, dtype=torch.int32, device=dev)
    pool = L.GqaPool(k, v, table, rotary_dim=HEAD_DIM, rope_base=500000.0, pairing=L.ROPE_HALF)
    T = permuted_pages(0, TOKENS // PAGE)
    directive = [L.Directive(0, S_START, S_END, k_stub, stub_v=v_stub)]

    def restore():
        pool.seq_set_pages(0, T, TOKENS)

    restore()
    pool.splice(directive)
    torch.cuda.synchronize()
    alg_bytes = pool.last_stats().alg_bytes
    for _ in range(args.warmup):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    quiet_gc()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        restore()
        pool.splice(directive)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()

    def step(_):
        restore()
        pool.splice(directive)

    launches, kernel_ms, kernel_bytes, samples = kernel_pass(torch, pool, 0, step, args.steps)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    out = base_line(args, "splice_32k_llama8b", alg_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": LAYERS, "kv_heads": HEADS, "head_dim": HEAD_DIM, "rotary_dim": HEAD_DIM, "tokens": TOKENS,
        "page_size": PAGE, "pool_pages": POOL_PAGES, "span": [S_START, S_END], "stub_rows": STUB,
        "delta": STUB - (S_END - S_START), "storage": "bf16 K and V planes, rotation in f32",
        "alg_bytes_per_step": alg_bytes})
    out["pct_hbm_peak"] = round(100.0 * out["value"] / HBM_PEAK_GBS, 2)
    out["roofline"] = roofline("gqa_splice_kernel", "splice_32k_llama8b", launches, kernel_ms, kernel_bytes, samples)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_gqa(
        args.cpu_seconds, HEADS, HEAD_DIM, TOKENS, PAGE, POOL_PAGES, S_START, S_END, STUB)
    pool.close()
    return out


# ------------------------------------------------------ per-row rotation --

def bench_rope_rows(args, in_place=False):
    """Per-row-angle rotation of MLA rows (page size 16, permuted pages), as
    VECTOR does before reconstructing V from K: every row's k_pe turned back by
    its position (angle -p).  rope_rows_32k_27layer gathers all 32768 rows of a
    27-layer sequence into a dense [27][32768][576] buffer (per-row table
    kernel + row kernel); rope_rows_32k_27layer_inplace turns the same rows in
    place (one kernel: 128-byte k_pe lines 1152 bytes apart, read and
    written).  A step is one ll_rope_rows call.  The pool holds 8 such
    sequences, 8.2 GB, and step i works on sequence i mod 8, so a step's rows
    (0.9 GB of band lines in place, 1 GB of rows gathered) never sit in the
    chip's 256 MB memory-side cache from an earlier step."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import permuted_pages, random_rows_torch

    LAYERS, TOKENS, PAGE, NSEQ = 27, 32768, 16, 8
    NP = TOKENS // PAGE
    POOL_PAGES = NSEQ * NP
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    data = torch.empty((LAYERS, POOL_PAGES, PAGE, ROW), dtype=torch.bfloat16, device=dev)
    for q in range(NSEQ):
        data[:, q * NP:(q + 1) * NP] = random_rows_torch(q, (LAYERS, NP, PAGE, ROW), dev)
    table = torch.full((NSEQ, NP + 8), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    perm = permuted_pages(0, POOL_PAGES)
    for q in range(NSEQ):
        pool.seq_set_pages(q, perm[q * NP:(q + 1) * NP], TOKENS)
    angles = -torch.arange(TOKENS, dtype=torch.int64, device=dev)
    out = None if in_place else torch.empty((LAYERS, TOKENS, ROW), dtype=torch.bfloat16, device=dev)
    pool.rope_rows(0, 0, angles, out=out)
    torch.cuda.synchronize()
    alg = pool.last_stats().alg_bytes

    def step(i):
        pool.rope_rows(i % NSEQ, 0, angles, out=out)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    quiet_gc()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launches, kernel_ms, kernel_bytes, samples = kernel_pass(torch, pool, 2, step, args.steps)
    name = "rope_rows_32k_27layer_inplace" if in_place else "rope_rows_32k_27layer"
    out_line = base_line(args, name, alg / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": LAYERS, "tokens": TOKENS, "page_size": PAGE, "angles": "-position of each row",
        "mode": "in place (k_pe bands only)" if in_place else "gather to a dense buffer",
        "sequences": f"{NSEQ}, step i on sequence i mod {NSEQ}", "pool_pages": POOL_PAGES,
        "alg_bytes_per_step": alg})
    out_line["metric"] = "per-row-angle RoPE rotation: row bytes GB/s"
    # MLA rows at page size 16: gathered by rope_gather_mla_kernel (the timed
    # launch also holds the per-row table kernel), turned in place by
    # rope_inplace_mla_kernel alone
    kernel = "rope_inplace_mla_kernel" if in_place else "rope_gather_mla_kernel"
    out_line["roofline"] = roofline(kernel, name, launches, kernel_ms, kernel_bytes, samples)
    if in_place:
        out_line["access_pattern_ceiling_gbs"] = INPLACE_CEILING_GBS
    out_line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_rope(
        args.cpu_seconds, LAYERS, TOKENS, PAGE, NP * 2, in_place)
    pool.close()
    return out_line


# --------------------------------------------------------- trainer mask --

def bench_kvs_mask(args):
    """KV-streams trainer-side mask for a batch of 64 rollouts of 32768 tokens
    (turns U[64, 512], compaction after every 10 turns, budget 8192 tokens,
    strategies window / half / pick in turn).  A step is one death-time call
    (log replay; the logs' keep masks already on the device, their one-off
    upload reported apart), one 128 x 128 block mask and one dense bit
    mask."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import compaction_log, np_rng

    ROLL, TOKENS = 64, 32768
    strategies = ("window", "half", "pick")
    rolls = [(TOKENS, compaction_log(np_rng(0, 10 + i), TOKENS, strategies[i % 3], 8192, 64, 512, 10))
             for i in range(ROLL)]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ctx = L.KvsMask(0)
    t_up = time.perf_counter()
    logs = ctx.upload_logs(rolls)
    torch.cuda.synchronize()
    upload_ms = (time.perf_counter() - t_up) * 1e3
    death, status = ctx.death_times(logs, TOKENS)
    bits = ctx.dense_mask(death)
    blocks = ctx.block_mask(death, 128, 128)
    torch.cuda.synchronize()
    if status.any().item():
        raise SystemExit("a synthetic eviction log did not match its own cache")
    dense_bytes = bits.numel() * 4
    ev = {k: [] for k in ("death", "block", "dense")}

    def step(record):
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            marks[0].record()
        ctx.death_times(logs, TOKENS, out=(death, status))
        if record:
            marks[1].record()
        ctx.block_mask(death, 128, 128, out=blocks)
        if record:
            marks[2].record()
        ctx.dense_mask(death, out=bits)
        if record:
            marks[3].record()
            for key, a, b in (("death", 0, 1), ("block", 1, 2), ("dense", 2, 3)):
                ev[key].append((marks[a], marks[b]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    quiet_gc()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(False)                       # no event in the timed loop
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gc.enable()
    for _ in range(args.steps):           # the phases' own times, apart
        step(True)
    torch.cuda.synchronize()
    ms = {k: statistics.mean(a.elapsed_time(b) for a, b in v) for k, v in ev.items()}
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    out = base_line(args, "kvs_mask_64x32k", dense_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "rollouts": ROLL, "tokens": TOKENS, "events_per_rollout": round(statistics.mean(len(r[1]) for r in rolls), 1),
        "turns": "U[64,512], compaction every 10 turns, budget 8192", "block": [128, 128],
        "dense_bytes": dense_bytes, "keep_mask_bytes": int(logs.keep.numel()),
        "step": "death times (logs resident) + block mask + dense mask"})
    out["metric"] = "KV-streams trainer mask: dense mask bytes written GB/s per step"
    out["dtype"] = "int32"
    # the timed launch spans the per-rollout pre-pass (kvs_events_kernel: the
    # distinct death times and the key codes, about 1/300 of the bytes) and
    # the row kernel
    out["roofline"] = roofline("kvs_dense_ev_kernel", "kvs_mask_64x32k", args.steps, ms["dense"] * args.steps,
                               dense_bytes * args.steps)
    out["kernel_ms"] = {k: round(v, 4) for k, v in ms.items()}
    out["log_upload_ms"] = round(upload_ms, 3)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_kvs(rolls, args.cpu_seconds, TOKENS)
    ctx.close()
    return out


# ------------------------------------------------------------------- evict --

def bench_evict(args, page, compact=False):
    """256 rollouts x 16384 tokens x 27 layers; per-rollout keep masks from
    random turn drops (turns U[200,2000], each dropped with p = 0.5); one
    eviction call for all rollouts.  Restoring the tables between steps is
    outside the timed call.

    compact=True (compact_128x16k_27layer_p16): page reuse off and every row
    kept, so the call compacts the rollouts into the lowest free pages and
    every row moves; 128 rollouts, pool pages twice theirs (every new page is
    fresh)."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import np_rng, permuted_pages, turn_drop_mask

    LAYERS, ROLL, TOKENS = 27, (128 if compact else 256), 16384
    per = TOKENS // page
    extra = ROLL * per if compact else (ROLL * per // 2 if page > 1 else 0)
    POOL_PAGES = ROLL * per + extra
    dev = torch.device("cuda:0")
    data = torch.empty((LAYERS, POOL_PAGES, page, ROW), dtype=torch.int16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    flat = data.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        k = min(step, flat.numel() - i)
        flat[i:i + k] = torch.randint(-32768, 32767, (k,), generator=g, device=dev, dtype=torch.int16)
    data = data.view(torch.bfloat16)
    table = torch.full((ROLL, per), -1, dtype=torch.int32, device=dev)
    pool = L.Pool(data, table)
    perm = permuted_pages(0, ROLL * per)
    rng = np_rng(0, 6)
    if compact:
        pool.set_page_reuse(False)
        masks = np.ones(ROLL * TOKENS, np.uint8)
    else:
        masks = np.concatenate([turn_drop_mask(rng, TOKENS) for _ in range(ROLL)])
    keep = torch.from_numpy(masks).to(dev)
    offsets = np.arange(ROLL, dtype=np.int64) * TOKENS
    seqs = list(range(ROLL))

    def restore():
        for s in range(ROLL):
            pool.seq_set_pages(s, perm[s * per:(s + 1) * per], TOKENS)

    restore()
    pool.evict(seqs, keep, offsets)
    torch.cuda.synchronize()
    stats = pool.last_stats()
    alg_bytes = stats.alg_bytes
    times, call_times = [], []
    seq_arr = np.asarray(seqs, dtype=np.int32)

    def evict_steps(n, timed):
        quiet_gc()
        for i in range(n):
            restore()
            torch.cuda.synchronize()
            a = time.perf_counter()
            pool.evict(seq_arr, keep, offsets)
            b = time.perf_counter()
            torch.cuda.synchronize()
            pool.free_pages()  # settles the host bookkeeping of a device-planned call
            if timed:
                times.append(time.perf_counter() - a)
                call_times.append(b - a)
        gc.enable()

    evict_steps(args.warmup, False)
    # timed: no launch stamped
    evict_steps(args.steps, True)
    # kernel pass: every launch of the row moves (page size 1: the table
    # kernel) and of the keep scan stamped
    pool.profile_read(0)
    pool.profile_read(1)
    pool.set_profiling(True, 1)
    evict_steps(min(args.steps, 10), False)
    pool.set_profiling(False)
    launches, kernel_ms, kernel_bytes, samples = pool.profile_read(0, samples=16)
    s_launches, scan_ms, _ = pool.profile_read(1)
    ms_per_step = 1e3 * statistics.median(times)
    name = "compact_128x16k_27layer_p16" if compact else f"evict_256x16k_27layer_p{page}"
    out = base_line(args, name, alg_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": LAYERS, "rollouts": ROLL, "tokens": TOKENS, "page_size": page, "pool_pages": POOL_PAGES,
        "mask": "every row kept, page reuse off (a compaction)" if compact else "turn drops U[200,2000], p=0.5",
        "rows_kept": int(masks.sum()),
        "rows_moved_per_layer": stats.rows_moved, "fresh_pages": stats.fresh_pages,
        "alg_bytes_per_step": alg_bytes,
        "page_plan": "device",
        "step": "one kv_evict_compact call until its device work and host bookkeeping are done, median"})
    out["metric"] = "KV-streams eviction: row bytes moved GB/s; call latency"
    # nothing moves at page size 1: the timed kernel writes the new tables and
    # packs the freed-page bitmap
    out["roofline"] = roofline("evict_move_kernel" if page > 1 else "unit_page_kernel", name, launches,
                               kernel_ms, kernel_bytes, samples)
    out["step_us"] = {"median": round(1e6 * statistics.median(times), 1), "p10": round(1e6 * pct(times, 10), 1),
                      "p90": round(1e6 * pct(times, 90), 1)}
    out["keep_scan_us"] = round(scan_ms * 1e3 / max(1, s_launches), 2)
    out["call_return_us"] = round(1e6 * statistics.median(call_times), 1)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_evict(
        masks, page, args.cpu_seconds, LAYERS, TOKENS, ROLL, reuse=not compact)
    pool.close()
    return out


def bench_evict_gqa(args):
    """KV-streams eviction on a GQA cache of Llama-3-8B shape: 32 rollouts x
    16384 tokens x 32 layers of K and V planes (8 KV heads x 128), page size
    16, random turn drops (turns U[200,2000], p = 0.5); pool pages 1.5 x the
    rollouts' (fewer than if every new page were fresh: the device's verdict
    decides before the rows move).  Restoring the tables between steps is outside the
    timed call."""
    import torch
    from mla_paged_cache_amd import leyline as L
    from synth import np_rng, permuted_pages, turn_drop_mask

    LAYERS, HEADS, HEAD_DIM, ROLL, TOKENS, PAGE = 32, 8, 128, 32, 16384, 16
    per = TOKENS // PAGE
    POOL_PAGES = ROLL * per * 3 // 2
    dev = torch.device("cuda:0")
    planes = []
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    for _ in range(2):
        t = torch.empty((LAYERS, POOL_PAGES, PAGE, HEADS, HEAD_DIM), dtype=torch.int16, device=dev)
        flat = t.view(-1)
        step = 1 << 28
        for i in range(0, flat.numel(), step):
            k = min(step, flat.numel() - i)
            flat[i:i + k] = torch.randint(-32768, 32767, (k,), generator=g, device=dev, dtype=torch.int16)
        planes.append(t.view(torch.bfloat16))
    table = torch.full((ROLL, per), -1, dtype=torch.int32, device=dev)
    pool = L.GqaPool(planes[0], planes[1], table, rotary_dim=HEAD_DIM, rope_base=500000.0, pairing=L.ROPE_HALF)
    perm = permuted_pages(0, ROLL * per)
    rng = np_rng(0, 7)
    masks = np.concatenate([turn_drop_mask(rng, TOKENS) for _ in range(ROLL)])
    keep = torch.from_numpy(masks).to(dev)
    offsets = np.arange(ROLL, dtype=np.int64) * TOKENS
    seqs = list(range(ROLL))

    def restore():
        for s in range(ROLL):
            pool.seq_set_pages(s, perm[s * per:(s + 1) * per], TOKENS)

    restore()
    pool.evict(seqs, keep, offsets)
    torch.cuda.synchronize()
    stats = pool.last_stats()
    alg_bytes = stats.alg_bytes
    times = []
    seq_arr = np.asarray(seqs, dtype=np.int32)

    def evict_steps(n, timed):
        quiet_gc()
        for i in range(n):
            restore()
            torch.cuda.synchronize()
            a = time.perf_counter()
            pool.evict(seq_arr, keep, offsets)
            torch.cuda.synchronize()
            pool.free_pages()
            if timed:
                times.append(time.perf_counter() - a)
        gc.enable()

    evict_steps(args.warmup, False)
    evict_steps(args.steps, True)          # no launch stamped
    pool.profile_read(0)
    pool.set_profiling(True, 1)
    evict_steps(min(args.steps, 10), False)
    pool.set_profiling(False)
    launches, kernel_ms, kernel_bytes, samples = pool.profile_read(0, samples=16)
    ms_per_step = 1e3 * statistics.median(times)
    name = "evict_32x16k_llama8b_p16"
    out = base_line(args, name, alg_bytes / (ms_per_step * 1e-3) / 1e9, ms_per_step, {
        "layers": LAYERS, "kv_heads": HEADS, "head_dim": HEAD_DIM, "rollouts": ROLL, "tokens": TOKENS,
        "page_size": PAGE, "pool_pages": POOL_PAGES, "mask": "turn drops U[200,2000], p=0.5",
        "rows_kept": int(masks.sum()), "rows_moved_per_plane": stats.rows_moved, "fresh_pages": stats.fresh_pages,
        "alg_bytes_per_step": alg_bytes, "page_plan": "device",
        "step": "one kv_evict_compact call until its device work and host bookkeeping are done, median"})
    out["metric"] = "KV-streams eviction: row bytes moved GB/s; call latency"
    out["roofline"] = roofline("plane_evict_kernel", name, launches, kernel_ms, kernel_bytes, samples)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_evict_gqa(
        masks, args.cpu_seconds, LAYERS, HEADS, HEAD_DIM, TOKENS, PAGE, ROLL)
    pool.close()
    return out


def cpu_baseline_evict_gqa(masks, seconds, LAYERS, HEADS, HEAD_DIM, TOKENS, PAGE, ROLL, k=2, layers=8):
    """The oracle's GQA eviction on `k` of the rollouts and `layers` of the
    layers (K and V arrays), the same masks and pool shape per rollout."""
    from oracle import leyline_oracle as O
    from synth import permuted_pages
    per = TOKENS // PAGE
    pool_pages = k * per * 3 // 2
    specs = []
    for _ in range(layers):
        specs += [O.gqa_k_row(HEADS, HEAD_DIM, HEAD_DIM), O.plain_row(HEADS * HEAD_DIM)]
    st = O.CacheState.empty(len(specs), pool_pages, PAGE, per, with_rows=False, specs=specs)
    st.layers = host_pool(len(specs), pool_pages, PAGE, HEADS * HEAD_DIM)
    perm = permuted_pages(0, k * per)
    for r in range(k):
        st.set_pages(r, perm[r * per:(r + 1) * per], TOKENS)
    ms = [masks[r * TOKENS:(r + 1) * TOKENS] for r in range(k)]
    runs, t, (_, plans) = timed_oracle(lambda: O.evict(st, list(range(k)), ms, reuse_pages=reuse), seconds)
    nb = sum(O.algorithmic_bytes(pl, int(m.sum()), PAGE, np.zeros(int(m.sum()), np.int64),
                                 np.zeros(int(m.sum()), bool), 0, layers, rotate=False, specs=specs)
             for pl, m in zip(plans, ms))
    return oracle_line(nb, runs, t, f"{k} of the {ROLL} rollouts, {layers} of the {LAYERS} layers (K and V), "
                                    "the same masks")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the splice path runs per GPU with no cross-GPU exchange "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)
    if args.workload == "splice_32k_27layer":
        out = bench_splice_32k(args)
    elif args.workload == "splice_32k_27layer_inplace":
        out = bench_splice_32k(args, STUB=0, workload="splice_32k_27layer_inplace", kernel="splice_inplace_kernel")
        out["access_pattern_ceiling_gbs"] = INPLACE_CEILING_GBS
    elif args.workload == "drift_128k_60layer":
        out = bench_drift(args)
    elif args.workload == "rope_rows_32k_27layer_inplace":
        out = bench_rope_rows(args, in_place=True)
    elif args.workload == "splice_4k_1layer":
        out = bench_splice_4k(args)
    elif args.workload == "splice_16x32k_27layer":
        out = bench_splice_batched(args)
    elif args.workload == "splice_32k_llama8b":
        out = bench_splice_gqa(args)
    elif args.workload == "evict_32x16k_llama8b_p16":
        out = bench_evict_gqa(args)
    elif args.workload == "kvs_mask_64x32k":
        out = bench_kvs_mask(args)
    elif args.workload == "rope_rows_32k_27layer":
        out = bench_rope_rows(args)
    elif args.workload == "compact_128x16k_27layer_p16":
        out = bench_evict(args, 16, compact=True)
    else:
        out = bench_evict(args, 16 if args.workload.endswith("p16") else 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
