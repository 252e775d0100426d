"""GPU parity of kv_evict_compact and ll_ptable_reindex (KV-streams summary,
"how it works": dropped entries are evicted in the engine, kept entries keep
their values and positions; "assumptions and limits": 16-token blocks and
block size 1) against the CPU oracle, through the C ABI."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, sliding_window_mask, turn_drop_mask

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _evict_both(dp, seqs, masks):
    keep = np.concatenate([np.asarray(m, np.uint8) for m in masks]) if masks else np.zeros(0, np.uint8)
    offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64) if masks else []
    expected, plans = O.evict(dp.state, seqs, masks)
    dev = torch.from_numpy(keep).to("cuda") if len(keep) else torch.zeros(16, dtype=torch.uint8, device="cuda")
    dp.pool.evict(seqs, dev, offsets)
    torch.cuda.synchronize()
    return expected, plans


def _rollouts(L, n_roll, n_tok, P, seed, extra_pages=None, oracle_layers=None, host_rows=True):
    pages_per = -(-n_tok // P)
    total = n_roll * pages_per + (extra_pages if extra_pages is not None else n_roll * pages_per)
    dp = DevicePool(L, total, P, n_roll, pages_per, seed=seed, host_rows=host_rows, oracle_layers=oracle_layers)
    perm = permuted_pages(seed, n_roll * pages_per)
    for s in range(n_roll):
        dp.set_pages(s, perm[s * pages_per:(s + 1) * pages_per], n_tok)
    return dp


@pytest.mark.parametrize("P", [16, 1])
@pytest.mark.parametrize("kind", ["sliding", "turns"])
@pytest.mark.parametrize("free", ["plenty", "tight"])
def test_evict_rollouts_full_compare(P, kind, free):
    """8 rollouts x 16384 tokens x 2 layers; keep masks: drop the oldest half,
    or drop random turns of 200..2000 tokens with probability 1/2.  The device
    makes the page plan; with free pages for every page of the rollouts or
    with fewer (page size 16 only: then a shortage is possible and the call
    reads the device's verdict before it goes on).  Both must give the
    oracle's plan."""
    if free == "tight" and P == 1:
        pytest.skip("at page size 1 no page is ever fresh")
    say(f"evict 8 x 16384 x 2, P={P}, {kind}, {free} free pages")
    pages_per = 16384 // P
    dp = _rollouts(2, 8, 16384, P, seed=3, extra_pages=None if free == "plenty" else 8 * pages_per * 3 // 4)
    dp.snapshot_rows()
    rng = np_rng(3, 5)
    masks = [sliding_window_mask(16384, 8192) if kind == "sliding" else turn_drop_mask(rng, 16384)
             for _ in range(8)]
    seqs = list(rng.permutation(8))
    expected, plans = _evict_both(dp, seqs, masks)
    for s in range(8):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    st = dp.pool.last_stats()
    fresh = sum(1 for pl in plans for x in pl if x < 0)
    assert st.fresh_pages == fresh
    if P == 1 or kind == "sliding":
        assert st.rows_moved == 0
    dp.close()


def test_evict_ragged_and_degenerate_masks():
    """Lengths that are not multiples of the page size, masks that keep all,
    none, only the tail, or alternate; masks at unaligned offsets."""
    say("evict ragged")
    rng = np.random.default_rng(7)
    lengths = [0, 1, 15, 16, 17, 1000, 4097, 333]
    dp = DevicePool(2, 2 * sum(-(-n // 16) for n in lengths) + 20, 16, len(lengths), 300, seed=7)
    perm = permuted_pages(7, dp.num_pages)
    at = 0
    for s, n in enumerate(lengths):
        k = -(-n // 16)
        dp.set_pages(s, perm[at:at + k], n)
        at += k
    dp.snapshot_rows()
    masks = []
    for s, n in enumerate(lengths):
        m = [np.ones(n), np.zeros(n), (np.arange(n) >= n - 5), (np.arange(n) % 2 == 0),
             rng.random(n) < 0.7, np.ones(n), rng.random(n) < 0.1, np.arange(n) < 17][s]
        masks.append(np.asarray(m, np.uint8))
    expected, _ = _evict_both(dp, list(range(len(lengths))), masks)
    for s in range(len(lengths)):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    dp.close()


def test_evict_then_splice_keeps_positions():
    """Eviction keeps the next position; a later splice shifts it by Delta."""
    say("evict then splice")
    L = need_gpu()
    dp = DevicePool(2, 100, 16, 1, 64, seed=9)
    dp.set_pages(0, permuted_pages(9, 100)[:40], 630)
    dp.snapshot_rows()
    mask = (np.random.default_rng(9).random(630) < 0.6).astype(np.uint8)
    expected, _ = _evict_both(dp, [0], [mask])
    compare_seq(dp, expected, 0, max_ulp=0)
    assert dp.pool.seq_get(0)[1] == 630
    dp.state = expected
    dev, host = dp.stub(4, 6)
    expected2, _ = O.splice(dp.state, [O.Directive(0, 20, 50, 6, host)])
    dp.pool.splice([L.Directive(0, 20, 50, dev)])
    torch.cuda.synchronize()
    compare_seq(dp, expected2, 0)
    assert dp.pool.seq_get(0)[1] == 630 - 24
    dp.close()


def test_evict_rejects_bad_requests():
    L = need_gpu()
    dp = DevicePool(1, 20, 16, 2, 10, seed=10)
    dp.set_pages(0, list(range(5)), 70)
    keep = torch.ones(70, dtype=torch.uint8, device="cuda")
    for seqs, offs in (([1], [0]), ([0, 0], [0, 0]), ([0], [-1])):
        with pytest.raises(L.LeylineError) as ei:
            dp.pool.evict(seqs, keep, offs)
        assert ei.value.status == L.LL_EINVAL
    # masks that would run past the keep buffer never reach the library
    for k, offs in ((keep[:69], [0]), (keep, [1])):
        with pytest.raises(ValueError):
            dp.pool.evict([0], k, offs)
    assert dp.pool.seq_get(0)[0] == 70
    dp.close()


def test_ptable_reindex_matches_oracle():
    say("ptable reindex")
    L = need_gpu()
    dp = DevicePool(1, 40, 16, 1, 40, seed=12)
    dp.set_pages(0, permuted_pages(12, 40)[:10], 150)
    dp.snapshot_rows()
    expected = O.ptable_reindex(dp.state, 0, [0, 3, 4, 9])
    dp.pool.ptable_reindex(0, [0, 3, 4, 9])
    torch.cuda.synchronize()
    compare_seq(dp, expected, 0, max_ulp=0)
    assert_same_free(dp, expected)
    with pytest.raises(L.LeylineError):
        dp.pool.ptable_reindex(0, [2, 1])
    dp.close()


@pytest.mark.slow
@pytest.mark.parametrize("P", [16, 1])
@pytest.mark.parametrize("kind", ["turns", "sliding"])
def test_evict_256_rollouts_27_layers(P, kind):
    """256 rollouts x 16384 tokens x 27 layers, one call; keep masks: random
    turn drops, or the sliding window that drops the oldest half.  Page tables
    of all 256 compared; rows compared on layers 0 and 26 for 16 rollouts.  At
    page size 16 the pool also holds the fresh pages the call needs (about
    180 GB in all)."""
    say(f"evict 256 x 16384 x 27, P={P}, {kind}")
    n_roll, n_tok = 256, 16384
    pages_per = n_tok // P
    extra = int(0.5 * n_roll * pages_per) if P == 16 else 0
    dp = _rollouts(27, n_roll, n_tok, P, seed=0, extra_pages=extra, oracle_layers=[], host_rows=False)
    rng = np_rng(0, 6)
    masks = [turn_drop_mask(rng, n_tok) if kind == "turns" else sliding_window_mask(n_tok, n_tok // 2)
             for _ in range(n_roll)]
    # rows of 16 rollouts on two layers, captured before the call
    check = list(range(0, n_roll, 16))
    before = {}
    for s in check:
        t = dp.state.tables[s]
        j = np.arange(n_tok)
        phys = torch.from_numpy(np.asarray(t, np.int64)[j // P] * P + j % P).to("cuda")
        before[s] = [dp.data[L].view(-1, O.ROW)[phys].view(torch.int16).cpu().numpy().view(np.uint16)
                     for L in (0, 26)]
    expected, plans = _evict_both(dp, list(range(n_roll)), masks)
    for s in range(n_roll):
        n, pos, pages = dp.pool.seq_get(s)
        assert n == expected.lengths[s] and pos == expected.next_pos[s]
        assert list(pages) == expected.tables[s]
        assert np.array_equal(dp.table[s, :len(pages)].cpu().numpy(), pages)
    assert dp.pool.free_pages() == len(expected.free)
    for s in check:
        n, _, pages = dp.pool.seq_get(s)
        j = np.arange(n)
        phys = torch.from_numpy(pages.astype(np.int64)[j // P] * P + j % P).to("cuda")
        kept = np.flatnonzero(masks[s])
        for li, L in enumerate((0, 26)):
            got = dp.data[L].view(-1, O.ROW)[phys].view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, before[s][li][kept])
    st = dp.pool.last_stats()
    say(f"  rows moved per layer {st.rows_moved}, fresh pages {st.fresh_pages}")
    dp.close()
