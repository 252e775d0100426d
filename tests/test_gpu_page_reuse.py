"""GPU parity of the page-reuse setting turned off: every page of a sequence
that a splice ([Leyline] sections 2.1-2.3) or an eviction (KV-streams, "how it
works") rewrites is fresh, so every live row is written into the lowest free
pages -- with the same row values as with reuse on.  Against the oracle run
with reuse off, through the C ABI, rows bit for bit."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, turn_drop_mask

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch
from test_gpu_gqa import GqaDevicePool

pytestmark = pytest.mark.gpu


def _splice(dp, L, specs, reuse, noalloc=False):
    """specs: (seq, s0, s1, r, seed, mode); oracle first, then the library."""
    host_dirs, dev_dirs = [], []
    for seq, s0, s1, r, seed, mode in specs:
        dev, host = dp.stub(seed, r)
        host_dirs.append(O.Directive(seq, s0, s1, r, host, mode))
        dev_dirs.append(L.Directive(seq, s0, s1, dev, mode))
    expected, plans = O.splice(dp.state, host_dirs, reuse_pages=reuse)
    dp.pool.splice(dev_dirs, noalloc=noalloc)
    torch.cuda.synchronize()
    return expected, plans


def _evict(dp, seqs, masks, reuse):
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64)
    expected, plans = O.evict(dp.state, seqs, masks, reuse_pages=reuse)
    dp.pool.evict(seqs, keep, offsets)
    torch.cuda.synchronize()
    return expected, plans


def _check(dp, expected, seqs):
    for s in seqs:
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    dp.state = expected


@pytest.mark.parametrize("P,planner", [(8, 0), (16, 0), (16, 1)])
def test_mla_without_page_reuse(P, planner):
    L = need_gpu()
    say(f"page reuse off: MLA, page size {P}, planner {'host' if planner else 'auto'}")
    lengths = [1500, 2222, 700]
    pages = [-(-n // P) for n in lengths]
    dp = DevicePool(2, 4 * sum(pages) + 32, P, 3, max(pages) + 8, seed=40 + P)
    perm = permuted_pages(40 + P, sum(pages))
    at = 0
    for s, n in enumerate(lengths):
        dp.set_pages(s, perm[at:at + pages[s]], n)
        at += pages[s]
    dp.snapshot_rows()
    dp.pool.set_splice_planner(planner)
    dp.pool.set_page_reuse(False)

    # a batch: a stub splice, a splice whose Delta is a whole number of pages
    # (with reuse on its downstream pages would be kept and turned in place),
    # and a FORGET (the kept prefix is copied into fresh pages)
    specs = [(0, 100, 300, 7, 1, O.AMORTIZE), (1, 2 * P, 6 * P, 0, 0, O.AMORTIZE), (2, 333, 333, 0, 0, O.FORGET)]
    expected, plans = _splice(dp, L, specs, reuse=False)
    assert all(x < 0 for pl in plans for x in pl)
    assert dp.pool.last_stats().rows_rotated_inplace == 0
    _check(dp, expected, range(3))

    # an eviction with turn drops, then one that keeps every row (a pure
    # compaction into the lowest free pages)
    rng = np_rng(40, P)
    masks = [np.asarray(turn_drop_mask(rng, dp.state.lengths[s], 20, 200), np.uint8) for s in (2, 0)]
    expected, _ = _evict(dp, [2, 0], masks, reuse=False)
    _check(dp, expected, range(3))
    n1 = dp.state.lengths[1]
    expected, plans = _evict(dp, [1], [np.ones(n1, np.uint8)], reuse=False)
    assert dp.pool.last_stats().rows_moved == n1
    _check(dp, expected, range(3))

    # the allocation-free entry point follows the setting too
    n0 = dp.state.lengths[0]
    expected, _ = _splice(dp, L, [(0, n0 // 4, n0 // 2, 5, 2, O.AMORTIZE)], reuse=False, noalloc=True)
    _check(dp, expected, range(3))

    # reuse back on: pages are kept again where the rule allows
    dp.pool.set_page_reuse(True)
    n1 = dp.state.lengths[1]
    expected, plans = _splice(dp, L, [(1, P, 3 * P, 0, 0, O.AMORTIZE)], reuse=True)
    assert any(x >= 0 for x in plans[0])
    _check(dp, expected, range(3))
    dp.close()


def test_gqa_without_page_reuse():
    L = need_gpu()
    say("page reuse off: GQA pool")
    P, H, D, rot, n = 16, 4, 128, 128, 3000
    pages = -(-n // P)
    dp = GqaDevicePool(2, 5 * pages, P, 2, 2 * pages, H, D, rot, seed=44, pairing=1)
    perm = permuted_pages(44, 2 * pages)
    dp.set_pages(0, perm[:pages], n)
    dp.set_pages(1, perm[pages:], n)
    dp.snapshot_rows()
    dp.pool.set_page_reuse(False)
    lib_dirs, ora_dirs = [], []
    for seq, s0, s1, r, seed in [(0, 500, 900, 9, 3), (1, 3 * P, 7 * P, 0, 0)]:
        k, v, host = dp.stub(seed, r)
        lib_dirs.append(L.Directive(seq, s0, s1, k, O.AMORTIZE, stub_v=v))
        ora_dirs.append(O.Directive(seq, s0, s1, r, host, O.AMORTIZE))
    expected, plans = O.splice(dp.state, ora_dirs, pairing=dp.pairing, base=dp.base, reuse_pages=False)
    dp.pool.splice(lib_dirs)
    torch.cuda.synchronize()
    assert all(x < 0 for pl in plans for x in pl)
    for s in range(2):
        assert dp.compare(expected, s) == 0
    dp.state = expected
    masks = [turn_drop_mask(np_rng(44, s), dp.state.lengths[s], 50, 400) for s in range(2)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    expected, _ = O.evict(dp.state, [0, 1], masks, reuse_pages=False)
    dp.pool.evict([0, 1], keep, [0, len(masks[0])])
    torch.cuda.synchronize()
    for s in range(2):
        assert dp.compare(expected, s) == 0
    assert dp.pool.free_pages() == len(expected.free)
    dp.close()


def test_page_reuse_off_is_refused_at_page_size_1():
    L = need_gpu()
    dp = DevicePool(1, 64, 1, 1, 64, seed=1)
    with pytest.raises(L.LeylineError) as e:
        dp.pool.set_page_reuse(False)
    assert e.value.status == L.LL_EUNSUPPORTED
    dp.pool.set_page_reuse(True)
    dp.close()


@pytest.mark.slow
@pytest.mark.parametrize("n_roll", [128, 136])
def test_compaction_128_rollouts_27_layers(n_roll):
    """The compaction workload as it is timed: 128 rollouts x 16384 tokens x
    27 layers at page size 16, pool pages twice the rollouts', page reuse
    off, every row kept, one call: every row moves into the lowest free
    pages.  With 136 rollouts the row kernel needs 4.33e9 work-items, more
    than one dispatch holds, so it runs as two.  Page tables of all rollouts
    and the free count against the oracle with reuse off; rows of every
    eighth rollout on layers 0 and 26 equal the rows captured before the
    call."""
    need_gpu()
    P, n_tok, layers = 16, 16384, 27
    per = n_tok // P
    say(f"compaction {n_roll} x {n_tok} x {layers}, page reuse off, every row kept")
    dp = DevicePool(layers, 2 * n_roll * per, P, n_roll, per, seed=0, host_rows=False, oracle_layers=[])
    perm = permuted_pages(0, n_roll * per)
    for s in range(n_roll):
        dp.set_pages(s, perm[s * per:(s + 1) * per], n_tok)
    dp.pool.set_page_reuse(False)
    check = list(range(0, n_roll, 8))
    before = {}
    j = np.arange(n_tok)
    for s in check:
        phys = torch.from_numpy(np.asarray(dp.state.tables[s], np.int64)[j // P] * P + j % P).to("cuda")
        before[s] = [dp.data[l].view(-1, O.ROW)[phys].view(torch.int16).cpu().numpy() for l in (0, layers - 1)]
    masks = [np.ones(n_tok, np.uint8)] * n_roll
    expected, plans = _evict(dp, list(range(n_roll)), masks, reuse=False)
    assert all(x < 0 for pl in plans for x in pl)
    st = dp.pool.last_stats()
    assert st.rows_moved == n_roll * n_tok and st.fresh_pages == n_roll * per
    for s in range(n_roll):
        n, pos, pages = dp.pool.seq_get(s)
        assert n == expected.lengths[s] and pos == expected.next_pos[s]
        assert list(pages) == expected.tables[s]
        assert np.array_equal(dp.table[s, :len(pages)].cpu().numpy(), pages)
    assert dp.pool.free_pages() == len(expected.free)
    for s in check:
        _, _, pages = dp.pool.seq_get(s)
        phys = torch.from_numpy(pages.astype(np.int64)[j // P] * P + j % P).to("cuda")
        for li, l in enumerate((0, layers - 1)):
            got = dp.data[l].view(-1, O.ROW)[phys].view(torch.int16).cpu().numpy()
            assert np.array_equal(got, before[s][li]), (s, l)
    dp.close()
