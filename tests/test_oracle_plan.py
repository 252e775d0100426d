"""Pins for the oracle's data movement and page plan (Leyline summary,
sections 2.1-2.3; KV-streams summary, "how it works" and "assumptions and
limits").  The oracle is checked against brute-force rebuilds of tiny caches
with Python lists (delete the span, insert the stub; keep the masked rows),
against a content-matching search for reusable pages, against plans derived by
hand for the two splice workloads, and against special cases."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import permuted_pages, random_rows_np, sliding_window_mask, turn_drop_mask, np_rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KV = O.KV_LORA_RANK


def _make_state(P, n_tokens_per_seq, num_pages, layers=2, seed=0, permute=True, max_pages=None):
    """A pool with random rows and one permuted page table per sequence."""
    need = sum(-(-n // P) for n in n_tokens_per_seq)
    max_pages = max_pages or max(8, max(-(-n // P) for n in n_tokens_per_seq) + 8)
    st = O.CacheState.empty(layers, num_pages, P, max_pages)
    for L in range(layers):
        st.layers[L][:] = random_rows_np(seed * 100 + L, (num_pages, P, O.ROW))
    pages = permuted_pages(seed, num_pages)[:need] if permute else np.arange(need)
    at = 0
    for s, n in enumerate(n_tokens_per_seq):
        k = -(-n // P)
        st.set_pages(s, pages[at:at + k], n)
        at += k
    return st


def _check_page_accounting(before, after, seqs):
    used = [p for t in after.tables.values() for p in t]
    assert len(used) == len(set(used)), "a physical page is used twice"
    assert set(used).isdisjoint(after.free)
    assert set(used) | after.free == set(range(after.num_pages))
    # fresh pages: the lowest pages of the free set as it was before, in
    # request order then page order
    fresh = [p for s in seqs for p in after.tables[s] if p not in set(before.tables[s])]
    assert fresh == sorted(before.free)[:len(fresh)]


def _brute_reuse(old_rows_by_page, new_logical, P, q, n_new):
    """Old logical page whose rows sit, by content, at exactly the offsets new
    page q needs; None if there is none."""
    live = range(q * P, min(q * P + P, n_new))
    for p, page in enumerate(old_rows_by_page):
        if all(j % P < len(page) and np.array_equal(new_logical[j][:KV], page[j % P][:KV]) for j in live):
            return p
    return None


def _old_pages(st, seq, layer):
    P, n, t = st.page_size, st.lengths[seq], st.tables[seq]
    return [[st.layers[layer][t[p], o] for o in range(min(P, n - p * P))] for p in range(len(t))]


# -------------------------------------------------- splice: brute force ----

@pytest.mark.parametrize("P", [1, 2, 4, 16])
def test_splice_matches_list_rebuild_exhaustive(P):
    rng = np.random.default_rng(P)
    sizes = sorted({0, 1, P - 1, P, P + 1, 2 * P + 1, 3 * P} - {-1})
    cases = 0
    for n in sizes:
        for s0, s1 in itertools.combinations_with_replacement(range(n + 1), 2):
            if P == 16 and (s0 % 3 or s1 % 5) and not (s0 == s1 or s1 == n):
                continue  # thin the P=16 grid; the boundary cases stay in
            for r in sorted({0, 1, 2, 3, P + 1}):
                st = _make_state(P, [n], num_pages=3 * (-(-n // P)) + 6, layers=1, seed=cases)
                stub = random_rows_np(10_000 + cases, (1, r, O.ROW)) if r else None
                d = O.Directive(0, s0, s1, r, stub)
                new, plans = O.splice(st, [d])
                old_log = [row for row in st.logical_rows(0, 0)] if n else []
                delta = r - (s1 - s0)
                # brute force: delete the span, insert the stub
                rebuilt = old_log[:s0] + ([stub[0][k] for k in range(r)]) + old_log[s1:]
                got = new.logical_rows(0, 0) if new.lengths[0] else np.zeros((0, O.ROW), np.uint16)
                assert new.lengths[0] == len(rebuilt) == n + delta
                assert new.next_pos[0] == st.next_pos[0] + delta
                for j, row in enumerate(rebuilt):
                    assert np.array_equal(got[j][:KV], row[:KV])
                    if j < s0 + r:
                        assert np.array_equal(got[j][KV:], row[KV:])
                    else:
                        assert np.array_equal(got[j][KV:], O.rotate_kpe_bf16(row[KV:], delta))
                # reuse rule against a content search
                old_pages = _old_pages(st, 0, 0)
                for q, reuse in enumerate(plans[0]):
                    b = _brute_reuse(old_pages, rebuilt, P, q, len(rebuilt))
                    assert (reuse if reuse >= 0 else None) == b, (n, s0, s1, r, q)
                _check_page_accounting(st, new, [0])
                cases += 1
    assert cases > 20


def test_splice_special_cases():
    P = 16
    st = _make_state(P, [100], num_pages=40, layers=1, seed=3)
    # |R| = 0, s_start = s_end: nothing changes, every page reused
    new, plans = O.splice(st, [O.Directive(0, 50, 50, 0, None)])
    assert new.tables[0] == st.tables[0] and all(p >= 0 for p in plans[0])
    assert np.array_equal(new.logical_rows(0, 0), st.logical_rows(0, 0))
    # s_end = n: no downstream, nothing rotates
    stub = random_rows_np(5, (1, 3, O.ROW))
    new, _ = O.splice(st, [O.Directive(0, 90, 100, 3, stub)])
    assert new.lengths[0] == 93
    assert np.array_equal(new.logical_rows(0, 0)[:90], st.logical_rows(0, 0)[:90])
    assert np.array_equal(new.logical_rows(0, 0)[90:], stub[0])
    # whole sequence replaced by nothing
    new, plans = O.splice(st, [O.Directive(0, 0, 100, 0, None)])
    assert new.lengths[0] == 0 and new.tables[0] == [] and new.free == set(range(40))
    # |R| = |S|: Delta = 0, downstream k_pe bit-identical
    stub = random_rows_np(6, (1, 10, O.ROW))
    new, _ = O.splice(st, [O.Directive(0, 20, 30, 10, stub)])
    assert np.array_equal(new.logical_rows(0, 0)[30:], st.logical_rows(0, 0)[30:])
    # Delta > 0: a stub longer than the span
    stub = random_rows_np(7, (1, 40, O.ROW))
    new, _ = O.splice(st, [O.Directive(0, 20, 30, 40, stub)])
    assert new.lengths[0] == 130 and new.next_pos[0] == 130


def test_splice_rejects_bad_requests_and_keeps_state():
    P = 16
    st = _make_state(P, [100, 64], num_pages=20, layers=1, seed=4, max_pages=10)
    snap = st.copy()
    stub = random_rows_np(1, (1, 4, O.ROW))
    with pytest.raises(O.InvalidRequest):
        O.splice(st, [O.Directive(0, 50, 40, 0, None)])
    with pytest.raises(O.InvalidRequest):
        O.splice(st, [O.Directive(0, 50, 101, 0, None)])
    with pytest.raises(O.InvalidRequest):
        O.splice(st, [O.Directive(0, 1, 2, 4, None)])            # stub missing
    with pytest.raises(O.InvalidRequest):
        O.splice(st, [O.Directive(0, 1, 2, 4, stub), O.Directive(0, 1, 2, 0, None)])
    with pytest.raises(O.Unsupported):
        O.splice(st, [O.Directive(0, 1, 2, 0, None, O.PIN)])
    with pytest.raises(O.OutOfRange):
        O.splice(st, [O.Directive(0, 0, 0, 100, random_rows_np(2, (1, 100, O.ROW)))])
    with pytest.raises(O.OutOfPages):
        # 20 pages: 7 + 4 used, 9 free; a splice at 0 in both needs 7 + 4 fresh
        O.splice(st, [O.Directive(0, 0, 1, 4, stub), O.Directive(1, 0, 1, 4, stub)])
    assert st.tables == snap.tables and st.free == snap.free and st.lengths == snap.lengths


def test_batched_splice_allocates_in_request_order():
    P = 4
    st = _make_state(P, [20, 20, 20], num_pages=64, layers=1, seed=5)
    stubs = [random_rows_np(i, (1, 3, O.ROW)) for i in range(3)]
    ds = [O.Directive(2, 5, 9, 3, stubs[0]), O.Directive(0, 1, 2, 3, stubs[1]),
          O.Directive(1, 6, 6, 3, stubs[2])]
    new, plans = O.splice(st, ds)
    fresh_in_order = [new.tables[d.seq][q] for d, plan in zip(ds, plans)
                      for q, x in enumerate(plan) if x < 0]
    assert fresh_in_order == sorted(st.free)[:len(fresh_in_order)]
    _check_page_accounting(st, new, [2, 0, 1])
    for d in ds:
        delta = d.r_len - (d.s_end - d.s_start)
        old = st.logical_rows(d.seq, 0)
        got = new.logical_rows(d.seq, 0)
        assert np.array_equal(got[:d.s_start], old[:d.s_start])
        assert np.array_equal(got[d.s_start + d.r_len:, :KV], old[d.s_end:, :KV])
        assert np.array_equal(got[d.s_start + d.r_len:, KV:], O.rotate_kpe_bf16(old[d.s_end:, KV:], delta))


def test_forget_trims_at_span_start():
    st = _make_state(16, [100], num_pages=20, layers=1, seed=6)
    new, plans = O.splice(st, [O.Directive(0, 37, 60, 0, None, O.FORGET)])
    assert new.lengths[0] == 37 and new.next_pos[0] == 37
    assert new.tables[0] == st.tables[0][:3]
    assert np.array_equal(new.logical_rows(0, 0), st.logical_rows(0, 0)[:37])


# ----------------------------------------------- splice: hand-derived plans -

def _ranges(rs):
    return [p for a, b in rs for p in range(a, b + 1)]


def test_plan_splice_4k_one_layer_golden():
    g = json.load(open(os.path.join(GOLDEN, "splice_plans.json")))["splice_4k_1layer"]
    st = O.CacheState.empty(1, 512, 16, 300, with_rows=False)
    st.set_pages(0, range(256), 4096)
    new, plans = O.splice(st, [O.Directive(0, 1000, 3000, 16, np.zeros((1, 16, O.ROW), np.uint16))])
    assert new.lengths[0] == g["n_new"]
    assert new.tables[0] == _ranges(g["new_table_ranges"])
    assert sorted(set(st.tables[0]) - set(new.tables[0])) == _ranges(g["freed_ranges"])
    kind, index, down = O.splice_sources(4096, 1000, 3000, 16)
    assert O.algorithmic_bytes(plans[0], 2112, 16, kind, down, -1984, 1) == g["bytes"]


def test_plan_splice_32k_27_layers_golden():
    g = json.load(open(os.path.join(GOLDEN, "splice_plans.json")))["splice_32k_27layer"]
    st = O.CacheState.empty(27, 4096, 16, 2048, with_rows=False)
    T = permuted_pages(0, 2048)
    st.set_pages(0, T, 32768)
    new, plans = O.splice(st, [O.Directive(0, 8192, 14336, 24, np.zeros((27, 24, O.ROW), np.uint16))])
    assert new.lengths[0] == g["n_new"]
    t = new.tables[0]
    assert t[:g["prefix_reused"]] == list(T[:g["prefix_reused"]])
    assert t[g["prefix_reused"]:] == list(range(g["fresh_first"], g["fresh_first"] + g["fresh_pages"]))
    assert len(set(T) - set(t)) == g["freed_pages"]
    kind, index, down = O.splice_sources(32768, 8192, 14336, 24)
    assert O.algorithmic_bytes(plans[0], g["n_new"], 16, kind, down, -6120, 27) == g["bytes"]


# ----------------------------------------------------------- eviction -----

@pytest.mark.parametrize("P", [1, 2, 4, 16])
def test_evict_matches_masked_list_and_cumsum(P):
    rng = np.random.default_rng(10 + P)
    for trial in range(40):
        n = int(rng.integers(0, 5 * P + 3))
        st = _make_state(P, [n, 7], num_pages=4 * (-(-n // P)) + 12, layers=1, seed=trial)
        keep = (rng.random(n) < rng.random()).astype(np.uint8)
        new, plans = O.evict(st, [0], [keep])
        old = st.logical_rows(0, 0) if n else np.zeros((0, O.ROW), np.uint16)
        got = new.logical_rows(0, 0) if new.lengths[0] else np.zeros((0, O.ROW), np.uint16)
        dst = np.cumsum(keep.astype(np.int64)) - keep          # exclusive prefix sum
        assert new.lengths[0] == int(keep.sum())
        for i in np.flatnonzero(keep):
            assert np.array_equal(got[dst[i]], old[i])             # byte-identical, no rotation
        assert new.next_pos[0] == st.next_pos[0]
        assert new.tables[1] == st.tables[1]
        rebuilt = [old[i] for i in range(n) if keep[i]]
        old_pages = _old_pages(st, 0, 0)
        for q, reuse in enumerate(plans[0]):
            b = _brute_reuse(old_pages, rebuilt, P, q, len(rebuilt))
            assert (reuse if reuse >= 0 else None) == b
        _check_page_accounting(st, new, [0])


@pytest.mark.parametrize("P", [1, 2, 4, 16])
def test_evict_every_mask_of_short_sequences(P):
    """All 2^n keep masks of sequences of n <= 12 rows: the kept rows in order,
    the reuse rule against the content search, the page accounting."""
    for n in range(13):
        st = _make_state(P, [n], num_pages=2 * (-(-n // P)) + 4, layers=1, seed=n + 31 * P)
        old = st.logical_rows(0, 0) if n else np.zeros((0, O.ROW), np.uint16)
        old_pages = _old_pages(st, 0, 0)
        for bits in range(1 << n):
            keep = np.array([(bits >> i) & 1 for i in range(n)], np.uint8)
            new, plans = O.evict(st, [0], [keep])
            rebuilt = old[np.flatnonzero(keep)]
            got = new.logical_rows(0, 0) if new.lengths[0] else np.zeros((0, O.ROW), np.uint16)
            assert np.array_equal(got, rebuilt), (P, n, bits)
            for q, reuse in enumerate(plans[0]):
                b = _brute_reuse(old_pages, list(rebuilt), P, q, len(rebuilt))
                assert (reuse if reuse >= 0 else None) == b, (P, n, bits, q)
            _check_page_accounting(st, new, [0])


def test_evict_special_cases():
    P = 16
    st = _make_state(P, [200], num_pages=40, layers=1, seed=7)
    new, plans = O.evict(st, [0], [np.ones(200, np.uint8)])
    assert new.tables[0] == st.tables[0] and all(x >= 0 for x in plans[0])
    new, plans = O.evict(st, [0], [np.zeros(200, np.uint8)])
    assert new.lengths[0] == 0 and new.tables[0] == [] and new.free == set(range(40))
    with pytest.raises(O.InvalidRequest):
        O.evict(st, [0], [np.ones(199, np.uint8)])
    with pytest.raises(O.InvalidRequest):
        O.evict(st, [0, 0], [np.ones(200, np.uint8)] * 2)


def test_evict_sliding_window_golden():
    g = json.load(open(os.path.join(GOLDEN, "splice_plans.json")))["evict_sliding_window_16k"]
    st = O.CacheState.empty(1, 2048, g["page_size"], 1024, with_rows=False)
    T = permuted_pages(1, 1024)
    st.set_pages(0, T, g["tokens"])
    new, plans = O.evict(st, [0], [sliding_window_mask(g["tokens"], g["drop"])])
    assert sum(1 for x in plans[0] if x < 0) == g["fresh_pages"]
    assert new.tables[0] == list(T[512:])
    assert new.free == set(range(2048)) - set(T[512:])


def test_evict_turn_drops_move_most_kept_rows_at_page_16():
    """Random turn drops leave most kept rows off their page offsets, so most
    new pages are fresh at page size 16; at page size 1 every page is reused."""
    rng = np_rng(0, 3)
    keep = turn_drop_mask(rng, 16384)
    for P, lo, hi in ((16, 0.6, 1.0), (1, 0.0, 0.0)):
        st = O.CacheState.empty(1, 2 * 16384 // P + 8, P, 16384 // P, with_rows=False)
        st.set_pages(0, range(16384 // P), 16384)
        new, plans = O.evict(st, [0], [keep])
        fresh = sum(1 for x in plans[0] if x < 0)
        assert lo <= fresh / max(1, len(plans[0])) <= hi


def test_ptable_reindex():
    st = _make_state(16, [100], num_pages=20, layers=1, seed=8)
    new = O.ptable_reindex(st, 0, [0, 2, 6])
    assert new.lengths[0] == 16 + 16 + 4
    assert new.tables[0] == [st.tables[0][k] for k in (0, 2, 6)]
    old = st.logical_rows(0, 0)
    assert np.array_equal(new.logical_rows(0, 0), np.concatenate([old[0:16], old[32:48], old[96:100]]))
    with pytest.raises(O.InvalidRequest):
        O.ptable_reindex(st, 0, [6, 2])
    with pytest.raises(O.InvalidRequest):
        O.ptable_reindex(st, 0, [6, 7])


# ------------------------------------------------ page reuse turned off --
# The library's page-reuse setting (off: every page of a rewritten sequence
# is fresh).  The row values are those of the brute-force rebuilds above
# whatever the placement; the placement is pinned to the lowest free pages in
# batch order, and every old page of a rewritten sequence returns to the free
# set.

def _check_compacted(before, after, seqs, plans):
    assert all(x == -1 for pl in plans for x in pl)
    lowest = sorted(before.free)
    at = 0
    for s in seqs:
        k = len(after.tables[s])
        assert after.tables[s] == lowest[at:at + k]
        at += k
    released = set().union(*(set(before.tables[s]) for s in seqs)) if seqs else set()
    assert after.free == (before.free - set(lowest[:at])) | released


@pytest.mark.parametrize("P", [2, 4, 16])
def test_splice_without_page_reuse_matches_list_rebuild(P):
    cases = 0
    for n in sorted({0, 1, P - 1, P, P + 1, 2 * P + 1, 3 * P}):
        for s0, s1 in itertools.combinations_with_replacement(range(n + 1), 2):
            if P == 16 and (s0 % 3 or s1 % 5) and not (s0 == s1 or s1 == n):
                continue
            for r in sorted({0, 1, P + 1}):
                st = _make_state(P, [n, 5], num_pages=4 * (-(-n // P)) + 8, layers=1, seed=cases)
                stub = random_rows_np(20_000 + cases, (1, r, O.ROW)) if r else None
                new, plans = O.splice(st, [O.Directive(0, s0, s1, r, stub)], reuse_pages=False)
                old_log = list(st.logical_rows(0, 0)) if n else []
                delta = r - (s1 - s0)
                rebuilt = old_log[:s0] + [stub[0][k] for k in range(r)] + old_log[s1:]
                got = new.logical_rows(0, 0) if new.lengths[0] else np.zeros((0, O.ROW), np.uint16)
                assert new.lengths[0] == len(rebuilt)
                for j, row in enumerate(rebuilt):
                    assert np.array_equal(got[j][:KV], row[:KV])
                    want = row[KV:] if j < s0 + r else O.rotate_kpe_bf16(row[KV:], delta)
                    assert np.array_equal(got[j][KV:], want)
                _check_compacted(st, new, [0], plans)
                assert new.tables[1] == st.tables[1]       # the other sequence is untouched
                # the same rows as with page reuse on, row for row
                on, _ = O.splice(st, [O.Directive(0, s0, s1, r, stub)])
                if on.lengths[0]:
                    assert np.array_equal(on.logical_rows(0, 0), got)
                cases += 1
    assert cases > 20


def test_forget_and_batches_without_page_reuse():
    P = 4
    st = _make_state(P, [30, 17, 9], num_pages=60, layers=1, seed=5)
    # FORGET keeps the prefix rows, now in fresh pages
    new, plans = O.splice(st, [O.Directive(0, 13, 30, 0, None, mode=O.FORGET)], reuse_pages=False)
    assert new.lengths[0] == 13
    assert np.array_equal(new.logical_rows(0, 0), st.logical_rows(0, 0)[:13])
    _check_compacted(st, new, [0], plans)
    # a batch: fresh pages go out in request order
    stub = random_rows_np(6, (1, 3, O.ROW))
    dirs = [O.Directive(2, 1, 4, 3, stub), O.Directive(0, 10, 12, 0, None)]
    new, plans = O.splice(st, dirs, reuse_pages=False)
    _check_compacted(st, new, [2, 0], plans)
    # too few free pages: refused, state unchanged
    tight = _make_state(P, [30], num_pages=9, layers=1, seed=6)
    with pytest.raises(O.OutOfPages):
        O.splice(tight, [O.Directive(0, 0, 0, 0, None)], reuse_pages=False)


@pytest.mark.parametrize("P", [2, 4, 16])
def test_evict_without_page_reuse_matches_masked_list(P):
    rng = np.random.default_rng(50 + P)
    for trial in range(30):
        n = [int(rng.integers(0, 5 * P + 3)) for _ in range(3)]
        st = _make_state(P, n, num_pages=3 * sum(-(-k // P) for k in n) + 12, layers=1, seed=trial)
        masks = [(rng.random(k) < rng.random()).astype(np.uint8) for k in n]
        order = [int(x) for x in rng.permutation(3)]
        new, plans = O.evict(st, order, [masks[s] for s in order], reuse_pages=False)
        for s in range(3):
            old = st.logical_rows(s, 0) if n[s] else np.zeros((0, O.ROW), np.uint16)
            got = new.logical_rows(s, 0) if new.lengths[s] else np.zeros((0, O.ROW), np.uint16)
            assert np.array_equal(got, old[np.flatnonzero(masks[s])])
            assert new.next_pos[s] == st.next_pos[s]
        _check_compacted(st, new, order, plans)
    # keep everything: a pure compaction into the lowest free pages
    st = _make_state(P, [3 * P + 1], num_pages=20, layers=1, seed=99)
    new, plans = O.evict(st, [0], [np.ones(3 * P + 1, np.uint8)], reuse_pages=False)
    assert np.array_equal(new.logical_rows(0, 0), st.logical_rows(0, 0))
    _check_compacted(st, new, [0], plans)


# -------------------------------------------- pins catch planted mistakes --

def test_pins_catch_a_planted_sign_error(monkeypatch):
    """Flip the rotation direction inside the oracle: the fresh-RoPE pin must
    fail.  (The mistake is planted in the oracle, on the CPU.)"""
    real = O.delta_cos_sin

    def flipped(delta, rope_dim=64, base=10000.0):
        c, s = real(delta, rope_dim, base)
        return c, -s
    monkeypatch.setattr(O, "delta_cos_sin", flipped)
    k_raw = np.random.default_rng(0).standard_normal((2000, 64))
    i = np.arange(20000, 22000)
    stored = O.f32_to_bf16(O.rotate_f64(k_raw, i).astype(np.float32))
    moved = O.bf16_to_f32(O.rotate_kpe_bf16(stored, -6120)).astype(np.float64)
    fresh = O.rotate_f64(k_raw, i - 6120)
    assert np.linalg.norm(moved - fresh) / np.linalg.norm(fresh) > 0.1


def test_pins_catch_a_planted_off_by_one_in_sources(monkeypatch):
    real = O.splice_sources

    def shifted(n, s0, s1, r):
        kind, index, down = real(n, s0, s1, r)
        index = np.where(down, np.minimum(index + 1, n - 1), index)
        return kind, index, down
    monkeypatch.setattr(O, "splice_sources", shifted)
    st = _make_state(4, [12], num_pages=12, layers=1, seed=9)
    new, _ = O.splice(st, [O.Directive(0, 2, 5, 0, None)])
    old = list(st.logical_rows(0, 0))
    rebuilt = old[:2] + old[5:]
    got = new.logical_rows(0, 0)
    assert any(not np.array_equal(got[j][:KV], rebuilt[j][:KV]) for j in range(len(rebuilt)))


def test_state_without_specs_holds_mla_rows_for_any_layer_count():
    """A state made with no row layouts and given its layer arrays afterwards
    (as the benchmark's CPU leg does) splices MLA rows in every array."""
    st = O.CacheState.empty(0, 64, 16, 64, with_rows=False)
    st.layers = [random_rows_np(1 + L, (64, 16, O.ROW)) for L in range(3)]
    st.set_pages(0, list(range(10)), 150)
    stub = random_rows_np(9, (3, 4, O.ROW))
    new, _ = O.splice(st, [O.Directive(0, 20, 40, 4, stub)])
    assert new.lengths[0] == 134
    for L in range(3):
        rows = new.logical_rows(0, L)
        assert np.array_equal(rows[20:24], stub[L])
        assert np.array_equal(rows[24:, :KV], st.logical_rows(0, L)[40:, :KV])
