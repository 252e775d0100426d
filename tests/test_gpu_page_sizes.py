"""GPU parity of the splice and the eviction at the page sizes where the row
kernels change their store path: page size 8 is the smallest whose pages are
whole waves (72 * 8 chunks: the stores go through a buffer descriptor on the
wave's destination page), 256 the largest page (the longest descriptor), 4
the last size below (plain non-temporal stores).  ([Leyline] sections 2.2-2.3
for the splice; KV-streams "how it works" for the eviction.)  Each case runs
a splice with stub rows, an eviction with turn drops and a second splice on
three sequences of ragged lengths, against the oracle, rows bit for bit."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, turn_drop_mask

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [4, 8, 64, 256])
def test_splice_evict_splice_across_page_sizes(P):
    L = need_gpu()
    say(f"page size {P}: splice, evict, splice on 3 ragged sequences")
    lengths = [3 * 256 + 37, 5 * 256 + 255, 2 * 256 + 1]
    pages = [-(-n // P) for n in lengths]
    max_pages = max(pages) + 4
    dp = DevicePool(2, 3 * sum(pages) + 16, P, 3, max_pages, seed=P)
    perm = permuted_pages(P, sum(pages))
    at = 0
    for s, n in enumerate(lengths):
        dp.set_pages(s, perm[at:at + pages[s]], n)
        at += pages[s]
    dp.snapshot_rows()

    # splice: each sequence loses a span and takes stub rows (Delta is not a
    # multiple of the page size, so downstream pages are fresh)
    spans = [(100, 300, 7), (P + 3, P + 3 + 500, 0), (1, 2, 40)]
    host_dirs, dev_dirs = [], []
    for s, (a, b, r) in enumerate(spans):
        dev, host = dp.stub(10 * P + s, r)
        host_dirs.append(O.Directive(s, a, b, r, host))
        dev_dirs.append(L.Directive(s, a, b, dev))
    expected, _ = O.splice(dp.state, host_dirs)
    dp.pool.splice(dev_dirs)
    torch.cuda.synchronize()
    for s in range(3):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    dp.state = expected

    # eviction with turn drops on the spliced sequences
    rng = np_rng(P, 11)
    masks = [np.asarray(turn_drop_mask(rng, dp.state.lengths[s], 20, 200), np.uint8) for s in range(3)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64)
    expected, plans = O.evict(dp.state, [2, 0, 1], [masks[2], masks[0], masks[1]])
    dp.pool.evict([2, 0, 1], keep, [offsets[2], offsets[0], offsets[1]])
    torch.cuda.synchronize()
    for s in range(3):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    assert dp.pool.last_stats().fresh_pages == sum(1 for pl in plans for x in pl if x < 0)
    dp.state = expected

    # a second splice after the eviction (the device wrote the new tables)
    n0 = dp.state.lengths[0]
    dev, host = dp.stub(20 * P, 3)
    expected, _ = O.splice(dp.state, [O.Directive(0, n0 // 3, n0 // 2, 3, host)])
    dp.pool.splice([L.Directive(0, n0 // 3, n0 // 2, dev)])
    torch.cuda.synchronize()
    for s in range(3):
        compare_seq(dp, expected, s, max_ulp=0)
    assert_same_free(dp, expected)
    dp.close()
