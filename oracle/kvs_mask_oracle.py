"""Plain CPU oracle for the KV-streams trainer-side attention mask.

TEST INFRASTRUCTURE. Like leyline_oracle, this module is the checker, not the
product: only the tests, the package smoke check and the CPU-baseline leg of
the benchmark may import it, and it shares no code with the HIP library.

What it follows: "KV-streams" (onedev.kr summary, paper 273), "how it works":
the inference engine evicts dropped KV entries inside the engine and keeps one
continuous stream, kept entries keep their original (k_i, v_i) and positions,
and the trainer reproduces the same eviction pattern with a custom attention
mask so that one forward pass over the whole rollout sees what each token saw
when it was generated.

Readings taken where the page is silent:
  * a rollout is T tokens in generation order; the forward pass of token q
    attends to the tokens the cache held right after q was appended;
  * an eviction event (time t, keep) runs after t tokens have been generated
    and before token t: `keep` is the keep mask over the rows the cache held
    then, in order (exactly what the engine passed to its eviction call);
  * hence key k is visible to query q iff k <= q and no event with time <= q
    dropped k.  With d_k the time of the event that dropped k (T if none),
    visible(q, k) = k <= q < d_k;
  * in a batch padded to T_pad tokens, keys at or beyond a rollout's length
    are never visible (d_k = k); queries beyond it follow the same rule;
  * block mask: the T x T mask cut into block_q x block_k tiles; a tile is
    full when every entry is visible, empty when none is, partial otherwise;
    each query block lists its partial and its full key blocks in increasing
    order;
  * dense bit mask: row q is ceil(T/32) little-endian uint32 words, bit b of
    word w is key 32 w + b.
"""

from __future__ import annotations

import numpy as np


class InvalidLog(Exception):
    """An event's keep mask does not match the rows held at its time, or the
    event times are not increasing inside (0, T]."""


def replay_visibility(n_tokens: int, events) -> np.ndarray:
    """Brute-force replay of the engine, one token at a time: the cache is a
    Python list of token ids; before token q is appended, every event whose
    time is q filters the list by its keep mask.  Row q of the result is the
    list right after q was appended.  bool [n_tokens, n_tokens]."""
    cache: list[int] = []
    vis = np.zeros((n_tokens, n_tokens), bool)
    ev = sorted(events, key=lambda e: e.time)
    at = 0
    for q in range(n_tokens):
        while at < len(ev) and ev[at].time == q:
            keep = np.asarray(ev[at].keep)
            if len(keep) != len(cache):
                raise InvalidLog(f"event at {q}: mask of {len(keep)} rows, cache holds {len(cache)}")
            cache = [tok for tok, kp in zip(cache, keep) if kp]
            at += 1
        cache.append(q)
        vis[q, cache] = True
    return vis


def death_times(n_pad: int, n_tokens: int, events) -> np.ndarray:
    """d_k for k < n_pad: the time of the event that dropped token k, n_pad
    for tokens never dropped, k for padding keys (k >= n_tokens).  int64."""
    d = np.full(n_pad, n_pad, np.int64)
    d[n_tokens:] = np.arange(n_tokens, n_pad)
    prev = 0
    for e in events:
        t = int(e.time)
        if not (prev < t <= n_tokens):
            raise InvalidLog("event times must increase inside (0, n_tokens]")
        prev = t
        held = np.flatnonzero(d[:t] == n_pad)             # rows the cache holds at time t
        keep = np.asarray(e.keep)
        if len(keep) != len(held):
            raise InvalidLog(f"event at {t}: mask of {len(keep)} rows, cache holds {len(held)}")
        d[held[keep == 0]] = t
    return d


def visibility(death: np.ndarray) -> np.ndarray:
    """The T x T mask of the definition: visible(q, k) = k <= q < d_k."""
    T = len(death)
    q = np.arange(T)[:, None]
    k = np.arange(T)[None, :]
    return (k <= q) & (q < np.asarray(death)[None, :])


def visibility_rows(death: np.ndarray, rows) -> np.ndarray:
    """Rows `rows` of the mask of the definition (for masks too large to
    build whole)."""
    d = np.asarray(death)
    q = np.asarray(rows)[:, None]
    k = np.arange(len(d))[None, :]
    return (k <= q) & (q < d[None, :])


def tile_class(death: np.ndarray, q0: int, q1: int, k0: int, k1: int) -> str:
    """'full', 'partial' or 'empty' for the tile [q0, q1) x [k0, k1) of the
    mask of the definition."""
    d = np.asarray(death)[k0:k1]
    q = np.arange(q0, q1)[:, None]
    k = np.arange(k0, k1)[None, :]
    tile = (k <= q) & (q < d[None, :])
    return "full" if tile.all() else ("partial" if tile.any() else "empty")


def block_mask(vis: np.ndarray, block_q: int, block_k: int):
    """Tile classification of a dense mask.  Returns (partial, full): for each
    query block, the list of key blocks whose tile is partial, and the list of
    those whose tile is full, both increasing."""
    T = vis.shape[0]
    nq = -(-T // block_q)
    nk = -(-vis.shape[1] // block_k)
    partial, full = [], []
    for i in range(nq):
        p, f = [], []
        for j in range(nk):
            tile = vis[i * block_q:(i + 1) * block_q, j * block_k:(j + 1) * block_k]
            if tile.all():
                f.append(j)
            elif tile.any():
                p.append(j)
        partial.append(p)
        full.append(f)
    return partial, full


def dense_bits(vis: np.ndarray) -> np.ndarray:
    """Pack a bool mask into little-endian uint32 words per row."""
    T, K = vis.shape
    W = -(-K // 32)
    padded = np.zeros((T, W * 32), bool)
    padded[:, :K] = vis
    out = np.zeros((T, W), np.uint32)
    for b in range(32):
        out |= padded[:, b::32].astype(np.uint32) << np.uint32(b)
    return out
