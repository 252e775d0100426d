"""Plain CPU oracle for the Leyline AMORTIZE splice and KV-streams eviction on an
MLA paged KV cache.

TEST INFRASTRUCTURE. This module is the checker, not the product. Only the test
suite, the package smoke check and the CPU-baseline leg of the benchmark may
import or call it. The HIP library never routes through it, and the two share
no code: the only thing they have in common is the seeded input generators in
`synth/`, which hold none of the arithmetic below.

What it follows (pages as published):
  * "Leyline: KV Cache Directives for Agentic Inference" (gist.science summary,
    paper 2606.01065):
      - section 2.1, the directive D = (s_start, s_end, R, m) and the AMORTIZE /
        FORGET modes: R goes in place of the span, downstream slots are
        re-indexed, and their K_nope and V stay exactly as they were;
      - section 2.2, the shift Delta = |R| - |S| and the closed-form correction
        K_pe_new[i] = R(Delta) K_pe[i], correct because R(a)R(b) = R(a+b);
      - section 2.3, serving integration: the prefix [0, s_start) is left as
        is, R is prefilled into new slots, and the rotation step rotates the
        K_pe band of every downstream slot and re-indexes it;
      - section 4.3, the rotation is computed in fp32 on bf16 storage.
  * "KV-streams" (onedev.kr summary, paper 273), "how it works": dropped
    entries are evicted inside the engine, kept entries keep their original
    (k_i, v_i) and positions are not reset; "assumptions and limits": 16-token
    blocks in vLLM, block size 1 in the SGLang fork.

Readings taken where the pages are silent:
  * span bounds are half-open and 0-based, [s_start, s_end);
  * RoPE frequencies theta_j = base^(-2j/d), base 10000, d = 64; pairs are
    interleaved (2j, 2j+1) by default, or half-split (j, j + d/2);
  * R(a) rotates each pair by angle +a*theta_j, i.e.
        x' = x cos - y sin,   y' = x sin + y cos;
  * cos/sin are evaluated in float64 on the float64 angle Delta*theta_j and
    rounded to float32; the rotation is then
        x' = bf16(f32(f32(x*c) - f32(y*s))),  y' = bf16(f32(f32(x*s) + f32(y*c)))
    with x, y the bf16 inputs widened to f32, no fused multiply-add, and
    bf16 rounding to nearest-even;
  * stub rows R are copied bit-exactly (they are prefilled at their final
    positions) and are never rotated;
  * page plan: new logical page q reuses old physical page T[p] iff every live
    row of q comes from old logical page p at the same in-page offset; every
    other new page is fresh and takes the lowest-numbered free page, in order of
    (position of the request in the batch, q ascending), from the free set as it
    stood when the call began; old pages that are not reused are freed after
    the call;
  * next_position moves by Delta on a splice, is unchanged by an eviction, and
    a FORGET trims the sequence at s_start;
  * eviction never rotates (positions are not renumbered).

Row layout (from the MLA cache split of section 2.2): one token of one layer is
576 bf16 values, c_kv (the position-free latent, 512 values) followed by k_pe
(the RoPE band, 64 values): 1152 bytes.  A layer's pool is an array
[num_pages][page_size][576] of uint16 bit patterns; one page table per sequence
is shared by all layers.

GQA / MHA caches (Leyline section 5: the directive carries over to GQA/MHA,
only the rotation step differs) are described by the same machinery with other
row layouts (`RowSpec`): a K array row holds H heads of D values and the first
rotary_dim values of every head are a RoPE band; a V array row has no band.
Every band turns by R(Delta) exactly as k_pe does, with theta_j computed over
the band's own width.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KV_LORA_RANK = 512
ROPE_DIM = 64
ROW = KV_LORA_RANK + ROPE_DIM


@dataclass(frozen=True)
class RowSpec:
    """One token's row in one layer array: `width` bf16 values, of which each
    (offset, dim) band is RoPE-rotated (pairs inside the band)."""
    width: int
    bands: tuple = ()


MLA_ROW = RowSpec(ROW, ((KV_LORA_RANK, ROPE_DIM),))


def gqa_k_row(heads: int, head_dim: int, rotary_dim: int) -> RowSpec:
    """K row of a GQA/MHA cache: H heads of head_dim values, the first
    rotary_dim values of each head rotated."""
    return RowSpec(heads * head_dim, tuple((h * head_dim, rotary_dim) for h in range(heads)))


def plain_row(width: int) -> RowSpec:
    """A row with no RoPE band (a V row)."""
    return RowSpec(width, ())

AMORTIZE = 0
FORGET = 1
PIN = 2
DECAY = 3
SCRATCH = 4


class OracleError(Exception):
    """Base class: the request is rejected and the state is left unchanged."""


class InvalidRequest(OracleError):
    pass


class OutOfRange(OracleError):
    pass


class OutOfPages(OracleError):
    pass


class Unsupported(OracleError):
    pass


# ---------------------------------------------------------------------------
# bf16 storage (Leyline section 4.3: KV stored in bf16, rotation in fp32)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32: the bf16 bits are the high
    half of the float32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, to nearest, ties to even.  NaN stays
    a (quiet) NaN of the same sign."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    is_nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    return np.where(is_nan, quiet, rounded).astype(np.uint16)


# ---------------------------------------------------------------------------
# RoPE and the delta-rotation (Leyline section 2.2)
# ---------------------------------------------------------------------------

def rope_theta(rope_dim: int = ROPE_DIM, base: float = 10000.0) -> list[float]:
    """theta_j = base^(-2j/d) for j = 0 .. d/2-1, in float64."""
    return [base ** (-2.0 * j / rope_dim) for j in range(rope_dim // 2)]


def pair_index(rope_dim: int = ROPE_DIM, pairing: str = "interleaved"):
    """Dimension indices (x_j, y_j) of rotation pair j."""
    half = rope_dim // 2
    j = np.arange(half)
    if pairing == "interleaved":
        return 2 * j, 2 * j + 1
    if pairing == "half":
        return j, j + half
    raise ValueError(f"unknown pairing {pairing!r}")


def delta_cos_sin(delta: int, rope_dim: int = ROPE_DIM, base: float = 10000.0):
    """Per-pair (cos, sin) of the angle delta*theta_j: the angle and the cos/sin
    in float64 (libm through `math`), each then rounded to float32."""
    th = rope_theta(rope_dim, base)
    c = np.array([math.cos(float(delta) * t) for t in th], dtype=np.float64)
    s = np.array([math.sin(float(delta) * t) for t in th], dtype=np.float64)
    return c.astype(np.float32), s.astype(np.float32)


def rotate_kpe_bf16(kpe_bits: np.ndarray, delta: int, rope_dim: int = ROPE_DIM,
                    base: float = 10000.0, pairing: str = "interleaved") -> np.ndarray:
    """K_pe_new = R(delta) K_pe on bf16 storage, arithmetic in float32.

    kpe_bits: uint16 [..., rope_dim].  Returns uint16 of the same shape."""
    kpe_bits = np.asarray(kpe_bits, dtype=np.uint16)
    ix, iy = pair_index(rope_dim, pairing)
    c, s = delta_cos_sin(delta, rope_dim, base)
    x = bf16_to_f32(kpe_bits[..., ix])
    y = bf16_to_f32(kpe_bits[..., iy])
    xc = np.multiply(x, c, dtype=np.float32)
    ys = np.multiply(y, s, dtype=np.float32)
    xs = np.multiply(x, s, dtype=np.float32)
    yc = np.multiply(y, c, dtype=np.float32)
    x_new = np.subtract(xc, ys, dtype=np.float32)
    y_new = np.add(xs, yc, dtype=np.float32)
    out = np.empty_like(kpe_bits)
    out[..., ix] = f32_to_bf16(x_new)
    out[..., iy] = f32_to_bf16(y_new)
    return out


def rotate_f64(k: np.ndarray, angle_steps, rope_dim: int = ROPE_DIM,
               base: float = 10000.0, pairing: str = "interleaved") -> np.ndarray:
    """Exact (float64) rotation of every pair j by angle_steps*theta_j.
    angle_steps broadcasts against k's leading dimensions.  Used for fresh
    RoPE at a position (angle_steps = position) and for the float64 mode of
    the delta-rotation (angle_steps = delta)."""
    k = np.asarray(k, dtype=np.float64)
    ix, iy = pair_index(rope_dim, pairing)
    th = np.array(rope_theta(rope_dim, base), dtype=np.float64)
    a = np.asarray(angle_steps, dtype=np.float64)[..., None] * th
    c, s = np.cos(a), np.sin(a)
    x, y = k[..., ix], k[..., iy]
    out = np.empty_like(k)
    out[..., ix] = x * c - y * s
    out[..., iy] = x * s + y * c
    return out


def row_cos_sin(angles, rope_dim: int = ROPE_DIM, base: float = 10000.0):
    """Per-row tables for rows turned by their own angle steps a_i: the float64
    angle a_i * theta_j, its float64 cos and sin (libm through `math`), each
    rounded to float32.  Returns (cos, sin), float32 [n, rope_dim/2]."""
    th = rope_theta(rope_dim, base)
    a = [float(x) for x in np.asarray(angles, dtype=np.int64)]
    c = np.array([[math.cos(x * t) for t in th] for x in a], dtype=np.float64).reshape(len(a), len(th))
    s = np.array([[math.sin(x * t) for t in th] for x in a], dtype=np.float64).reshape(len(a), len(th))
    return c.astype(np.float32), s.astype(np.float32)


def rotate_rows_bf16(bits: np.ndarray, angles, rope_dim: int = ROPE_DIM, base: float = 10000.0,
                     pairing: str = "interleaved") -> np.ndarray:
    """Row i of `bits` (uint16 [n, rope_dim]) turned by R(angles[i]): the same
    float32 arithmetic as rotate_kpe_bf16, with the row's own cos/sin."""
    bits = np.asarray(bits, dtype=np.uint16)
    ix, iy = pair_index(rope_dim, pairing)
    c, s = row_cos_sin(angles, rope_dim, base)
    x = bf16_to_f32(bits[:, ix])
    y = bf16_to_f32(bits[:, iy])
    x_new = np.subtract(np.multiply(x, c, dtype=np.float32), np.multiply(y, s, dtype=np.float32), dtype=np.float32)
    y_new = np.add(np.multiply(x, s, dtype=np.float32), np.multiply(y, c, dtype=np.float32), dtype=np.float32)
    out = np.empty_like(bits)
    out[:, ix] = f32_to_bf16(x_new)
    out[:, iy] = f32_to_bf16(y_new)
    return out


# ---------------------------------------------------------------------------
# Paged cache state
# ---------------------------------------------------------------------------

@dataclass
class CacheState:
    """A paged MLA cache: per-layer pools and the bookkeeping shared by all
    layers.  Pools may be None when only the page plan is wanted."""
    page_size: int
    num_pages: int
    max_pages_per_seq: int
    layers: list | None
    specs: list | None = None                       # RowSpec per layer array (None: MLA rows)
    tables: dict = field(default_factory=dict)      # seq -> list of physical pages
    lengths: dict = field(default_factory=dict)     # seq -> tokens
    next_pos: dict = field(default_factory=dict)    # seq -> next RoPE position
    free: set = field(default_factory=set)

    @staticmethod
    def empty(num_layers: int, num_pages: int, page_size: int, max_pages_per_seq: int,
              with_rows: bool = True, specs=None) -> "CacheState":
        specs = list(specs) if specs is not None else None   # None: every array holds MLA rows
        widths = [sp.width for sp in specs] if specs is not None else [ROW] * num_layers
        layers = ([np.zeros((num_pages, page_size, w), np.uint16) for w in widths]
                  if with_rows else None)
        return CacheState(page_size, num_pages, max_pages_per_seq, layers, specs,
                          free=set(range(num_pages)))

    def spec(self, layer: int) -> RowSpec:
        return self.specs[layer] if self.specs is not None else MLA_ROW

    def copy(self) -> "CacheState":
        return CacheState(self.page_size, self.num_pages, self.max_pages_per_seq,
                          None if self.layers is None else [a.copy() for a in self.layers],
                          None if self.specs is None else list(self.specs),
                          {k: list(v) for k, v in self.tables.items()},
                          dict(self.lengths), dict(self.next_pos), set(self.free))

    def set_pages(self, seq: int, pages, n_tokens: int) -> None:
        """Give sequence `seq` an explicit page table (fixtures: e.g. a random
        permutation of physical pages); next_position = n_tokens."""
        pages = [int(p) for p in pages]
        own = set(self.tables.get(seq, []))
        need = -(-n_tokens // self.page_size)
        if len(pages) != need or len(pages) > self.max_pages_per_seq:
            raise InvalidRequest("page count does not match the length")
        if len(set(pages)) != len(pages) or any(p not in self.free and p not in own for p in pages):
            raise InvalidRequest("pages not free")
        self.free |= own
        self.free -= set(pages)
        self.tables[seq] = pages
        self.lengths[seq] = n_tokens
        self.next_pos[seq] = n_tokens

    def logical_rows(self, seq: int, layer: int) -> np.ndarray:
        """The sequence's rows of one layer array in logical order: uint16
        [n, width]."""
        P = self.page_size
        n = self.lengths[seq]
        t = np.asarray(self.tables[seq], dtype=np.int64)
        j = np.arange(n)
        return self.layers[layer][t[j // P], j % P]


# ---------------------------------------------------------------------------
# Step a1/a2: validation and the logical source of every new row
# ---------------------------------------------------------------------------

@dataclass
class Directive:
    """D = (s_start, s_end, R, m) for one sequence.  `stub` holds the |R|
    prefilled rows per layer array: uint16 [r_len][width] for each array (an
    MLA cache: [L][r_len][576]), or None when r_len is 0."""
    seq: int
    s_start: int
    s_end: int
    r_len: int
    stub: np.ndarray | None = None
    mode: int = AMORTIZE


def splice_sources(n: int, s_start: int, s_end: int, r_len: int):
    """Logical source of each new row after replacing [s_start, s_end) by r_len
    stub rows (Leyline section 2.2: the downstream moves by Delta).

    Returns (kind, index) arrays of length n' = n + Delta: kind 0 = old row
    `index` before the edit, kind 1 = stub row `index`; and `downstream`, true
    where the row is an old row that moved by Delta."""
    delta = r_len - (s_end - s_start)
    n_new = n + delta
    j = np.arange(n_new, dtype=np.int64)
    kind = np.where((j >= s_start) & (j < s_start + r_len), 1, 0)
    index = np.where(j < s_start, j, np.where(kind == 1, j - s_start, j - delta))
    downstream = j >= s_start + r_len
    return kind, index, downstream


def _validate_directives(state: CacheState, directives):
    seen = set()
    for d in directives:
        if d.mode in (PIN, DECAY, SCRATCH):
            raise Unsupported(f"mode {d.mode} is reserved")
        if d.mode not in (AMORTIZE, FORGET):
            raise InvalidRequest("unknown mode")
        if d.seq not in state.tables:
            raise InvalidRequest("unknown sequence")
        if d.seq in seen:
            raise InvalidRequest("sequence appears twice in one batch")
        seen.add(d.seq)
        n = state.lengths[d.seq]
        if not (0 <= d.s_start <= d.s_end <= n) or d.r_len < 0:
            raise InvalidRequest("bad span")
        if d.mode == AMORTIZE:
            if (d.r_len > 0) != (d.stub is not None):
                raise InvalidRequest("stub rows must be given iff r_len > 0")
            n_new = n + d.r_len - (d.s_end - d.s_start)
            if -(-n_new // state.page_size) > state.max_pages_per_seq:
                raise OutOfRange("sequence would not fit its page table")


# ---------------------------------------------------------------------------
# Step a3: the page plan (reuse rule, lowest-free-first allocation, release)
# ---------------------------------------------------------------------------

def page_plan(old_table, P: int, kind: np.ndarray, index: np.ndarray, reuse_pages: bool = True):
    """For each new logical page q, the old logical page it reuses, or -1 if it
    must be fresh.  A page is reused iff each of its live rows is an old row of
    one and the same old page, sitting at the same offset it will occupy.
    With reuse_pages False (the library's page-reuse setting turned off) no
    page is reused: every new page is fresh."""
    n_new = len(kind)
    if not reuse_pages:
        return [-1] * (-(-n_new // P))
    plan = []
    for q in range(-(-n_new // P)):
        lo, hi = q * P, min(q * P + P, n_new)
        k = kind[lo:hi]
        src = index[lo:hi]
        reuse = -1
        if np.all(k == 0):
            p = src[0] // P
            if np.all(src // P == p) and np.all(src % P == np.arange(lo, hi) % P):
                reuse = int(p)
        plan.append(reuse)
    return plan


def _apply(state: CacheState, requests, rotate_by, pairing, base, reuse_pages=True):
    """Carry out planned requests on a copy of `state`.

    requests: list of (seq, n_new, kind, index, downstream, stub, next_pos).
    The page plans of all requests are made first, with fresh pages taken in
    request order from the free set as it was at the start; old pages that are
    not reused are released at the end."""
    P = state.page_size
    new = state.copy()
    free_sorted = sorted(state.free)
    plans = []
    need = 0
    for (seq, n_new, kind, index, downstream, stub, npos) in requests:
        plan = page_plan(state.tables[seq], P, kind, index, reuse_pages)
        plans.append(plan)
        need += sum(1 for x in plan if x < 0)
    if need > len(free_sorted):
        raise OutOfPages(f"need {need} fresh pages, {len(free_sorted)} free")
    cursor = 0
    released = []
    for (seq, n_new, kind, index, downstream, stub, npos), plan in zip(requests, plans):
        old_t = state.tables[seq]
        new_t = []
        for reuse in plan:
            if reuse >= 0:
                new_t.append(old_t[reuse])
            else:
                new_t.append(free_sorted[cursor])
                cursor += 1
        reused = {old_t[r] for r in plan if r >= 0}
        released += [p for p in old_t if p not in reused]
        if state.layers is not None:
            _move_rows(state, new, seq, new_t, plan, n_new, kind, index, downstream, stub,
                       rotate_by.get(seq, 0), pairing, base)
        new.tables[seq] = new_t
        new.lengths[seq] = n_new
        new.next_pos[seq] = npos
    new.free -= set(free_sorted[:cursor])
    new.free |= set(released)
    return new, plans


def _move_rows(old: CacheState, new: CacheState, seq, new_t, plan, n_new, kind, index,
               downstream, stub, delta, pairing, base):
    """Write the rows of the sequence's new pages.  Fresh pages receive every
    live row (old rows copied bit-exactly, stub rows copied bit-exactly,
    downstream RoPE bands rotated by delta).  Reused pages already hold their
    rows; only the downstream bands are rotated there when delta != 0."""
    P = old.page_size
    old_t = np.asarray(old.tables[seq], dtype=np.int64)
    new_t = np.asarray(new_t, dtype=np.int64)
    j = np.arange(n_new, dtype=np.int64)
    q = j // P
    fresh = np.asarray(plan, dtype=np.int64)[q] < 0
    dst = new_t[q] * P + j % P
    is_old = kind == 0
    src = np.full(n_new, -1, dtype=np.int64)
    src[is_old] = old_t[index[is_old] // P] * P + index[is_old] % P
    rot = downstream & (delta != 0)
    for L in range(len(old.layers)):
        spec = old.spec(L)
        a_old = old.layers[L].reshape(-1, spec.width)
        a_new = new.layers[L].reshape(-1, spec.width)
        m = fresh & is_old
        a_new[dst[m]] = a_old[src[m]]
        m = fresh & ~is_old
        if np.any(m):
            a_new[dst[m]] = stub[L][index[m]]
        m = rot
        if np.any(m):
            for off, dim in spec.bands:
                a_new[dst[m], off:off + dim] = rotate_kpe_bf16(a_old[src[m], off:off + dim], delta,
                                                               rope_dim=dim, pairing=pairing, base=base)


# ---------------------------------------------------------------------------
# Entry points: splice (Leyline AMORTIZE / FORGET) and eviction (KV-streams)
# ---------------------------------------------------------------------------

def splice(state: CacheState, directives, pairing: str = "interleaved", base: float = 10000.0,
           reuse_pages: bool = True):
    """Apply a batch of directives, one per sequence.  Returns (new_state,
    plans), plans[i][q] = reused old logical page or -1 for a fresh page.
    reuse_pages False: every new page is fresh (see page_plan)."""
    _validate_directives(state, directives)
    requests, rotate_by = [], {}
    for d in directives:
        n = state.lengths[d.seq]
        if d.mode == FORGET:
            # Leyline section 2.1: FORGET hands the edit to a prefix-trimming
            # re-prefill; the cache keeps [0, s_start) and drops the rest.
            n_new = d.s_start
            j = np.arange(n_new, dtype=np.int64)
            requests.append((d.seq, n_new, np.zeros(n_new, np.int64), j,
                             np.zeros(n_new, bool), None,
                             state.next_pos[d.seq] - (n - d.s_start)))
            continue
        delta = d.r_len - (d.s_end - d.s_start)
        kind, index, downstream = splice_sources(n, d.s_start, d.s_end, d.r_len)
        rotate_by[d.seq] = delta
        requests.append((d.seq, n + delta, kind, index, downstream, d.stub,
                         state.next_pos[d.seq] + delta))
    return _apply(state, requests, rotate_by, pairing, base, reuse_pages)


def evict(state: CacheState, seqs, masks, reuse_pages: bool = True):
    """KV-streams eviction: keep exactly the rows whose mask entry is nonzero,
    in their order, unchanged (no rotation, no position reset).  reuse_pages
    False: every new page is fresh (see page_plan)."""
    if len(set(seqs)) != len(seqs):
        raise InvalidRequest("sequence appears twice in one batch")
    requests = []
    for seq, mask in zip(seqs, masks):
        if seq not in state.tables:
            raise InvalidRequest("unknown sequence")
        mask = np.asarray(mask)
        if mask.shape != (state.lengths[seq],):
            raise InvalidRequest("mask length differs from the sequence length")
        src = np.flatnonzero(mask)
        n_new = len(src)
        requests.append((seq, n_new, np.zeros(n_new, np.int64), src.astype(np.int64),
                         np.zeros(n_new, bool), None, state.next_pos[seq]))
    return _apply(state, requests, {}, "interleaved", 10000.0, reuse_pages)


def ptable_reindex(state: CacheState, seq: int, keep_pages):
    """Page-granular eviction: the new table is the old table's entries at the
    (strictly increasing) logical pages `keep_pages`; the tokens are those
    pages' live rows, in order; no row moves and no position reset."""
    if seq not in state.tables:
        raise InvalidRequest("unknown sequence")
    P = state.page_size
    n = state.lengths[seq]
    n_pages = -(-n // P)
    keep = [int(k) for k in keep_pages]
    if any(b <= a for a, b in zip(keep, keep[1:])) or any(k < 0 or k >= n_pages for k in keep):
        raise InvalidRequest("keep_pages must be strictly increasing old logical pages")
    if any(k == n_pages - 1 and n % P and i != len(keep) - 1 for i, k in enumerate(keep)):
        raise InvalidRequest("a partial tail page may only be kept last")
    live = [min(P, n - k * P) for k in keep]
    new = state.copy()
    old_t = state.tables[seq]
    new.tables[seq] = [old_t[k] for k in keep]
    new.lengths[seq] = sum(live)
    new.free |= {old_t[k] for k in range(n_pages) if k not in set(keep)}
    return new


def rope_rows(state: CacheState, seq: int, row_begin: int, angles, pairing: str = "interleaved",
              base: float = 10000.0, in_place: bool = False):
    """Per-row RoPE rotation of the sequence's logical rows
    [row_begin, row_begin + len(angles)): row row_begin + i has every RoPE band
    turned by R(angles[i]) (an angle of -position turns a stored key back to
    its position-free form, as VECTOR does before its K -> V map; "VECTOR",
    gist.science summary, method, reconstructability through OLS).

    Only layer arrays that carry bands take part.  in_place=False: returns the
    list, one per such array, of the turned rows (uint16 [n, width]), the
    state untouched.  in_place=True: returns a new state whose rows have their
    bands turned there (the other values and arrays unchanged)."""
    angles = np.asarray(angles, dtype=np.int64)
    n = len(angles)
    if seq not in state.tables:
        raise InvalidRequest("unknown sequence")
    if row_begin < 0 or row_begin + n > state.lengths[seq]:
        raise InvalidRequest("rows outside the sequence")
    P = state.page_size
    t = np.asarray(state.tables[seq], dtype=np.int64)
    j = np.arange(row_begin, row_begin + n)
    phys = t[j // P] * P + j % P if n else np.zeros(0, np.int64)
    new = state.copy() if in_place else None
    outs = []
    for L in range(len(state.layers)):
        spec = state.spec(L)
        if not spec.bands:
            continue
        rows = state.layers[L].reshape(-1, spec.width)[phys].copy()
        for off, dim in spec.bands:
            rows[:, off:off + dim] = rotate_rows_bf16(rows[:, off:off + dim], angles, rope_dim=dim,
                                                      base=base, pairing=pairing)
        if in_place:
            new.layers[L].reshape(-1, spec.width)[phys] = rows
        else:
            outs.append(rows)
    return new if in_place else outs


def algorithmic_bytes(plan, n_new, P, kind, downstream, delta, num_layers, rotate=True, specs=None):
    """Bytes the method must move for one request (its row data only): per
    layer array, 2 * row bytes per live row of a fresh page and 2 * band bytes
    per downstream row of a reused page whose bands are rotated in place
    (MLA rows: 2*1152 and 2*128)."""
    j = np.arange(n_new)
    fresh = np.asarray(plan, dtype=np.int64)[j // P] < 0 if n_new else np.zeros(0, bool)
    moved = int(np.count_nonzero(fresh))
    inplace = int(np.count_nonzero(~fresh & downstream)) if (rotate and delta != 0) else 0
    specs = list(specs) if specs is not None else [MLA_ROW] * num_layers
    return sum(2 * sp.width * 2 * moved + sum(2 * dim * 2 for _, dim in sp.bands) * inplace for sp in specs)
