"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and builds input shapes only: random bf16
rows, page permutations, directive spans, keep masks and turn-level
compaction logs.  It holds none of the splice, eviction or visibility
arithmetic (no shift, no rotation, no page plan, no death times), so both
the CPU oracle and the HIP library can be fed from it without sharing code.

Workload shapes stand in for the workloads the pages describe: tool-turn stubs
that replace older tool outputs (Leyline, sections 2.1 and 4.2), concurrent
requests (Leyline, section 4.1, C up to 16), and the KV-streams compaction
strategies with 16k/32k token budgets (KV-streams, "how it works" and "how it
differs").  No item of any public benchmark is used.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROW = 576          # c_kv 512 + k_pe 64, bf16


def np_rng(seed: int, *stream: int) -> np.random.Generator:
    """A numpy generator for (seed, stream...) built from SeedSequence."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *stream])))


def permuted_pages(seed: int, n_pages: int, start: int = 0) -> np.ndarray:
    """A random permutation of the physical pages start .. start+n_pages-1."""
    return (np_rng(seed, 1).permutation(n_pages) + start).astype(np.int32)


def random_rows_np(seed: int, shape) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) draws, made on the host.

    The float32 draws are rounded to bf16 by torch's own conversion."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_rows_torch(seed: int, shape, device):
    """bf16 N(0,1) rows generated directly on `device` (a torch tensor of dtype
    bfloat16); used for pools too large to stage from the host."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        k = min(step, flat.numel() - i)
        flat[i:i + k] = torch.randn(k, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)
    return out


def random_normal_np(seed: int, shape) -> np.ndarray:
    """float64 N(0,1) draws (numpy), for position-free keys k_raw and queries."""
    return np_rng(seed, 2).standard_normal(shape)


# ---------------------------------------------------------------------------
# Directive and mask draws
# ---------------------------------------------------------------------------

@dataclass
class SpanDraw:
    s_start: int
    s_end: int
    r_len: int


def draw_span(rng: np.random.Generator, length: int, span_lo: int, span_hi: int,
              stub_lo: int, stub_hi: int, start_lo: int = 1024) -> SpanDraw:
    """span ~ U[span_lo, span_hi], stub ~ U[stub_lo, stub_hi], start ~
    U[start_lo, length - span], all integer and inclusive."""
    span = int(rng.integers(span_lo, span_hi + 1))
    stub = int(rng.integers(stub_lo, stub_hi + 1))
    start = int(rng.integers(start_lo, length - span + 1))
    return SpanDraw(start, start + span, stub)


def sliding_window_mask(n: int, drop: int) -> np.ndarray:
    """Keep mask (uint8) that drops the oldest `drop` tokens."""
    m = np.ones(n, np.uint8)
    m[:drop] = 0
    return m


def turn_drop_mask(rng: np.random.Generator, n: int, turn_lo: int = 200, turn_hi: int = 2000,
                   p_drop: float = 0.5) -> np.ndarray:
    """Keep mask (uint8): the sequence is cut into turns of U[turn_lo, turn_hi]
    tokens and each turn is dropped independently with probability p_drop."""
    m = np.ones(n, np.uint8)
    i = 0
    while i < n:
        t = int(rng.integers(turn_lo, turn_hi + 1))
        if rng.random() < p_drop:
            m[i:i + t] = 0
        i += t
    return m


@dataclass(frozen=True)
class EvictionEvent:
    """One compaction of a rollout: `time` tokens had been generated when it
    ran; `keep` is the keep mask (uint8) over the rows the cache held then, in
    order -- the mask the inference engine hands to its eviction call."""
    time: int
    keep: np.ndarray


def compaction_log(rng: np.random.Generator, n_tokens: int, strategy: str, budget: int,
                   turn_lo: int = 64, turn_hi: int = 512, every_turns: int = 10) -> list:
    """Eviction log of one synthetic rollout of `n_tokens` tokens, cut into
    turns of U[turn_lo, turn_hi] tokens, compacted after every `every_turns`
    completed turns while tokens remain (the KV-streams strategies, at turn
    granularity; the newest turn is always kept):

      * "window": keep the newest turns that fit in `budget` tokens
        (Sliding Window, o close to B);
      * "half": keep the newest turns that fit in budget // 2 (Markovian
        Thinker, o = B/2, s = 0);
      * "pick": drop each older turn with probability 1/2 (a random stand-in
        for Markovian Pick, where the model chooses).

    The generator tracks the cache as a list of (turn, length) segments; it
    never looks at individual token indices."""
    turns = []
    i = 0
    while i < n_tokens:
        t = min(int(rng.integers(turn_lo, turn_hi + 1)), n_tokens - i)
        turns.append(t)
        i += t
    held = []          # lengths of the turns the cache holds, oldest first
    log = []
    done = 0
    for k, t in enumerate(turns):
        held.append(t)
        done += t
        if (k + 1) % every_turns or done >= n_tokens:
            continue
        keep_turn = np.ones(len(held), bool)
        if strategy in ("window", "half"):
            cap = budget if strategy == "window" else budget // 2
            total = 0
            for h in range(len(held) - 1, -1, -1):
                if h < len(held) - 1 and total + held[h] > cap:
                    keep_turn[:h + 1] = False
                    break
                total += held[h]
        elif strategy == "pick":
            keep_turn[:-1] = rng.random(len(held) - 1) >= 0.5
        else:
            raise ValueError(strategy)
        mask = np.concatenate([np.full(h, 1 if kt else 0, np.uint8) for h, kt in zip(held, keep_turn)])
        log.append(EvictionEvent(done, mask))
        held = [h for h, kt in zip(held, keep_turn) if kt]
    return log


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    seqs: int
    tokens: int
    page_size: int
    num_pages: int


# A one-layer, 4096-token cache with an identity page table; splice
# [1000, 3000) for 16 stub rows.
SPLICE_4K_1L = Workload("splice_4k_1layer", 1, 1, 4096, 16, 512)
# A 27-layer (DeepSeek-V2-Lite shaped) 32768-token cache, randomly permuted
# pages; splice three 2048-token tool turns [8192, 14336) for 24 stub rows.
SPLICE_32K_27L = Workload("splice_32k_27layer", 27, 1, 32768, 16, 4096)
# 16 concurrent 32768-token sequences in one pool, one random directive each.
SPLICE_16x32K_27L = Workload("splice_16x32k_27layer", 27, 16, 32768, 16, 65536)
# 256 rollouts of 16384 tokens, eviction under keep masks.
EVICT_256x16K_27L = Workload("evict_256x16k_27layer", 27, 256, 16384, 16, 0)
# One 131072-token, 60-layer sequence; ten successive splices.
DRIFT_128K_60L = Workload("drift_128k_60layer", 60, 1, 131072, 16, 16384)
