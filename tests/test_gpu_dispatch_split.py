"""Row kernels issued as several dispatches.

A dispatch packet counts its work-items in 32 bits, so a splice or eviction
that moves more than 2^32 16-byte chunks over all layers is cut into
dispatches over ranges of whole page tasks (the splice's in-place band
rotation first, the page-table rewrites with the last range), and a per-row
gather into ranges of whole layers.  A lowered limit
(`Pool.set_dispatch_limit`) cuts small launches the same way, so every cut is
compared here with the oracle row by row; one splice past 2^32 work-items
checks the real limit (the eviction past it is the 136-rollout compaction in
test_gpu_page_reuse.py)."""

from __future__ import annotations

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, turn_drop_mask

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch, ulp_distance
from test_gpu_gqa import GqaDevicePool

pytestmark = pytest.mark.gpu

# about four page tasks of 16 rows per dispatch on three layers
LIMIT = 16384


def _lib_splice(dp, directives):
    L = need_gpu()
    lib, ora = [], []
    for (seq, s0, s1, r, seed, mode) in directives:
        dev, host = dp.stub(seed, r if mode == O.AMORTIZE else 0)
        lib.append(L.Directive(seq, s0, s1, dev, mode))
        ora.append(O.Directive(seq, s0, s1, r if mode == O.AMORTIZE else 0, host, mode))
    expected, _ = O.splice(dp.state, ora, pairing="half" if dp.pairing else "interleaved")
    dp.pool.splice(lib)
    torch.cuda.synchronize()
    return expected


def _mla_pool(P, pairing, lengths, seed):
    pages = [-(-n // P) for n in lengths]
    dp = DevicePool(3, 3 * sum(pages) + 64, P, len(lengths), max(pages) + 8, seed=seed, pairing=pairing)
    dp.pairing = pairing
    perm = permuted_pages(seed, sum(pages))
    at = 0
    for s, n in enumerate(lengths):
        dp.set_pages(s, perm[at:at + pages[s]], n)
        at += pages[s]
    dp.snapshot_rows()
    return dp


@pytest.mark.parametrize("P,pairing,planner", [(16, 0, 0), (16, 1, 1), (4, 0, 0), (8, 1, 0)])
def test_split_mla_splice_then_evict(P, pairing, planner):
    """Four directives in one call under a lowered limit: rows moved with a
    stub (several dispatches), a span of whole pages (downstream pages turned
    in place), an insertion, a FORGET; then a turn-drop eviction of every
    sequence.  Every row of every layer against the oracle."""
    need_gpu()
    say(f"split MLA splice + evict, P={P} pairing={pairing} planner={planner}")
    lengths = [2000, 1500, 777, 1024]
    dp = _mla_pool(P, pairing, lengths, seed=60 + P)
    dp.pool.set_dispatch_limit(LIMIT)
    dp.pool.set_splice_planner(planner)
    dirs = [(0, 100, 300, 7, 61, O.AMORTIZE), (1, 64, 64 + 4 * P, 0, 62, O.AMORTIZE),
            (2, 5, 5, 3, 63, O.AMORTIZE), (3, 0, 10, 0, 64, O.FORGET)]
    expected = _lib_splice(dp, dirs)
    for s in range(4):
        compare_seq(dp, expected, s)
    assert_same_free(dp, expected)
    dp.state = expected
    rng = np_rng(70 + P, 1)
    masks = [turn_drop_mask(rng, expected.lengths[s], 20, 200) for s in range(4)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64)
    expected, _ = O.evict(dp.state, [0, 1, 2, 3], masks)
    dp.pool.evict([0, 1, 2, 3], keep, offsets)
    torch.cuda.synchronize()
    assert dp.pool.last_stats().rows_moved > 0
    for s in range(4):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    # back to the packet's own limit: the same kind of call in one dispatch
    dp.state = expected
    dp.pool.set_dispatch_limit(0)
    expected = _lib_splice(dp, [(0, 3, 40, 2, 65, O.AMORTIZE)])
    compare_seq(dp, expected, 0)
    dp.close()


def test_split_limit_is_checked():
    need_gpu()
    dp = _mla_pool(16, 0, [100], seed=5)
    from mla_paged_cache_amd.leyline import LeylineError
    for bad in (-1, 1, 1023, 2 ** 32):
        with pytest.raises(LeylineError):
            dp.pool.set_dispatch_limit(bad)
    dp.pool.set_dispatch_limit(1024)
    dp.pool.set_dispatch_limit(2 ** 32 - 1)
    dp.pool.set_dispatch_limit(0)
    dp.close()


@pytest.mark.parametrize("P,H,D,rot,pairing", [(16, 2, 64, 64, 0), (8, 4, 128, 64, 1)])
def test_split_gqa_splice_then_evict(P, H, D, rot, pairing):
    """The same on K and V planes: a moving splice, a splice of whole pages
    (bands turned in place) and an insertion in one call, then a turn-drop
    eviction, under a lowered limit; every row against the oracle."""
    need_gpu()
    say(f"split GQA splice + evict, P={P} H={H} D={D} rot={rot} pairing={pairing}")
    lengths = [1200, 900, 500]
    pages = [-(-n // P) for n in lengths]
    dp = GqaDevicePool(2, 3 * sum(pages) + 64, P, 3, max(pages) + 8, H, D, rot, seed=80 + P, pairing=pairing)
    perm = permuted_pages(80 + P, sum(pages))
    at = 0
    for s, n in enumerate(lengths):
        dp.set_pages(s, perm[at:at + pages[s]], n)
        at += pages[s]
    dp.snapshot_rows()
    dp.pool.set_dispatch_limit(LIMIT)
    expected, _ = dp.splice([(0, 50, 260, 5, 81, O.AMORTIZE), (1, 2 * P, 5 * P, 0, 82, O.AMORTIZE),
                             (2, 7, 7, 4, 83, O.AMORTIZE)])
    for s in range(3):
        assert dp.compare(expected, s) <= 1
    assert dp.pool.free_pages() == len(expected.free)
    dp.state = expected
    rng = np_rng(90 + P, 2)
    masks = [turn_drop_mask(rng, expected.lengths[s], 20, 150) for s in range(3)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64)
    expected, _ = O.evict(dp.state, [0, 1, 2], masks)
    dp.pool.evict([0, 1, 2], keep, offsets)
    torch.cuda.synchronize()
    assert dp.pool.last_stats().rows_moved > 0
    for s in range(3):
        assert dp.compare(expected, s) == 0
    assert dp.pool.free_pages() == len(expected.free)
    dp.close()


def _cmp_band_rows(got, exp, bands, width):
    mask = np.zeros(width, bool)
    for off, dim in bands:
        mask[off:off + dim] = True
    assert np.array_equal(got[:, ~mask], exp[:, ~mask])
    assert ulp_distance(got[:, mask], exp[:, mask]).max(initial=0) <= 1


def test_split_rope_rows_gather_by_layers():
    """Per-row-angle gathers under a lowered limit (one layer per dispatch):
    MLA rows gathered by page, and GQA K rows; against the oracle."""
    need_gpu()
    say("split per-row gather, MLA and GQA")
    P, n_tok = 16, 900
    pages = -(-n_tok // P)
    dp = DevicePool(5, 2 * pages, P, 1, 2 * pages, seed=7)
    dp.set_pages(0, permuted_pages(7, 2 * pages)[:pages], n_tok)
    dp.snapshot_rows()
    dp.pool.set_dispatch_limit(LIMIT)
    a = np_rng(7, 3).integers(-100000, 100000, size=500).astype(np.int64)
    out = dp.pool.rope_rows(0, 111, torch.from_numpy(a).cuda(), out=True)
    torch.cuda.synchronize()
    exp = O.rope_rows(dp.state, 0, 111, a, pairing="interleaved")
    for li in range(5):
        got = out[li].view(torch.int16).cpu().numpy().view(np.uint16)
        _cmp_band_rows(got, exp[li], [(512, 64)], O.ROW)
    dp.close()

    H, D, rot = 4, 128, 64
    g = GqaDevicePool(3, 2 * pages, P, 1, 2 * pages, H, D, rot, seed=9, pairing=1)
    g.set_pages(0, permuted_pages(9, 2 * pages)[:pages], n_tok)
    g.snapshot_rows()
    g.pool.set_dispatch_limit(LIMIT)
    out = g.pool.rope_rows(0, 40, torch.from_numpy(a).cuda(), out=True)
    torch.cuda.synchronize()
    exp = O.rope_rows(g.state, 0, 40, a, pairing=g.pairing)
    for li in range(3):
        got = out[li].reshape(500, H * D).view(torch.int16).cpu().numpy().view(np.uint16)
        _cmp_band_rows(got, exp[li], [(h * D, rot) for h in range(H)], H * D)
    g.close()


@pytest.mark.slow
def test_splice_past_2_32_work_items():
    """One batched splice whose row kernel needs more than 2^32 work-items:
    16 sequences of 150000 tokens x 27 layers at page size 16; 15 directives
    drop the first two rows for one stub row (Delta = -1: every page fresh,
    15 x 9375 x 1152 x 27 = 4.37e9 chunks), one drops a whole page (its
    downstream pages turned in place).  Page tables and free count of all
    16, rows of every sequence on layers 0 and 26 against the oracle."""
    need_gpu()
    L, P, n_tok, n_seq = 27, 16, 150000, 16
    per = -(-n_tok // P)
    assert 15 * per * P * 72 * L > 2 ** 32
    say(f"splice past 2^32 work-items: {n_seq} x {n_tok} x {L}")
    dp = DevicePool(L, 2 * n_seq * per, P, n_seq, per + 8, seed=3, host_rows=False, oracle_layers=[0, L - 1])
    dp.pairing = 0
    perm = permuted_pages(3, n_seq * per)
    for s in range(n_seq):
        dp.set_pages(s, perm[s * per:(s + 1) * per], n_tok)
    dp.snapshot_rows()
    dirs = [(s, 0, 2, 1, 300 + s, O.AMORTIZE) for s in range(15)] + [(15, 0, P, 0, 0, O.AMORTIZE)]
    expected = _lib_splice(dp, dirs)
    for s in range(n_seq):
        compare_seq(dp, expected, s)
    assert_same_free(dp, expected)
    dp.close()
