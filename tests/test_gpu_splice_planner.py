"""The two splice page planners against the CPU oracle, through the C ABI.

A splice ("Leyline", sections 2.1-2.3) is planned by the host either way; a
small batch whose fresh pages form few runs of consecutive page ids is then
expanded on the device from kernel arguments, any other batch (and every batch
under SPLICE_PLAN_HOST) is staged and uploaded.  Both must give the oracle's
page tables, lengths, positions and rows (c_kv and stub rows bit-exact, k_pe
within 1 bf16 ulp; 0 expected), and each call must report the planner the
rules pick: at most 16 directives (GQA: 1024 / rotary_dim), at most 256 runs."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch
from test_gpu_gqa import GqaDevicePool

pytestmark = pytest.mark.gpu

MAX_DIRS, MAX_RUNS = 16, 256


def _runs(pages):
    pages = sorted(pages)
    return sum(1 for i, x in enumerate(pages) if i == 0 or x != pages[i - 1] + 1)


def _fresh_runs(state, plans):
    need = sum(1 for plan in plans for x in plan if x < 0)
    return _runs(sorted(state.free)[:need])


def _mla_splice(dp, dirs, planner, pairing="interleaved"):
    """dirs: (seq, s0, s1, r, seed, mode).  Returns (oracle state, runs of
    the fresh pages)."""
    L = need_gpu()
    lib, ora = [], []
    for seq, s0, s1, r, seed, mode in dirs:
        rr = r if mode == O.AMORTIZE else 0
        dev, host = dp.stub(seed, rr)
        lib.append(L.Directive(seq, s0, s1, dev, mode))
        ora.append(O.Directive(seq, s0, s1, rr, host, mode))
    expected, plans = O.splice(dp.state, ora, pairing=pairing)
    dp.pool.set_splice_planner(planner)
    dp.pool.splice(lib)
    torch.cuda.synchronize()
    return expected, _fresh_runs(dp.state, plans)


def _directive(rng, seq, n, kind, P, seed):
    """One directive of the given kind on a sequence of n rows."""
    if kind == 0 and n >= 2 * P + 3:      # Delta = -2P: downstream pages kept, turned in place
        s0 = int(rng.integers(0, n - (2 * P + 3) + 1))
        return (seq, s0, s0 + 2 * P + 3, 3, seed, O.AMORTIZE)
    if kind == 1 and n > 0:               # ragged shift, either sign
        s0 = int(rng.integers(0, n))
        return (seq, s0, int(rng.integers(s0, n + 1)), int(rng.integers(0, 2 * P + 5)), seed, O.AMORTIZE)
    if kind == 2:                         # pure insertion
        s0 = int(rng.integers(0, n + 1))
        return (seq, s0, s0, int(rng.integers(1, P + 6)), seed, O.AMORTIZE)
    if kind == 3:                         # delete everything
        return (seq, 0, n, 0, seed, O.AMORTIZE)
    if kind == 4:                         # FORGET: trim at s_start
        s0 = int(rng.integers(0, n + 1))
        return (seq, s0, n, 0, seed, O.FORGET)
    if kind == 5:                         # append after the last row
        return (seq, n, n, int(rng.integers(1, 2 * P + 2)), seed, O.AMORTIZE)
    s1 = int(rng.integers(0, n + 1))      # from the first row
    return (seq, 0, s1, int(rng.integers(0, P + 3)), seed, O.AMORTIZE)


@pytest.mark.parametrize("P,pairing", [(1, 0), (4, 0), (16, 0), (16, 1)])
def test_planners_agree_batch_by_batch(P, pairing):
    """Batches of 1..20 directives of seven kinds over 20 sequences, the
    planner switched at random before each; every sequence compared with the
    oracle after every batch."""
    need_gpu()
    say(f"planners batch by batch, P={P}, pairing={pairing}")
    rng = np_rng(900 + P + pairing, 1)
    n_seq, max_rows = 20, 700
    lengths = [int(x) for x in rng.integers(0, 300, size=n_seq)]
    max_pages = -(-max_rows // P)
    used = sum(-(-n // P) for n in lengths)
    num_pages = used + 2 * n_seq * max_pages
    dp = DevicePool(2, num_pages, P, n_seq, max_pages, seed=901 + P, pairing=pairing)
    perm = permuted_pages(901 + P, used)
    at = 0
    for s, n in enumerate(lengths):
        k = -(-n // P)
        dp.set_pages(s, perm[at:at + k], n)
        at += k
    dp.snapshot_rows()
    name = "half" if pairing else "interleaved"
    seen = {0: 0, 1: 0}
    for b in range(14):
        k = int(rng.integers(1, 21))
        seqs = [int(x) for x in rng.choice(n_seq, size=k, replace=False)]
        dirs = []
        for i, s in enumerate(seqs):
            n = dp.state.lengths[s]
            d = _directive(rng, s, n, int(rng.integers(0, 7)), P, 9000 + 100 * b + i)
            if n + d[3] - (d[2] - d[1]) > max_rows:   # keep inside the table row
                d = (s, 0, n, 0, d[4], O.AMORTIZE)
            dirs.append(d)
        planner = int(rng.integers(0, 2))
        expected, runs = _mla_splice(dp, dirs, planner, name)
        st = dp.pool.last_stats()
        want = int(planner == 0 and k <= MAX_DIRS and runs <= MAX_RUNS)
        assert st.planned_on_device == want, (k, runs, planner)
        seen[want] += 1
        for s in range(n_seq):
            assert compare_seq(dp, expected, s, max_ulp=1) == 0
        assert_same_free(dp, expected)
        dp.state = expected
    say(f"  batches planned on the device {seen[1]}, staged by the host {seen[0]}")
    assert seen[0] and seen[1]
    dp.close()


def test_run_and_batch_limits_pick_the_planner():
    """Free pages every other page id: a splice needing 256 fresh pages has
    256 runs (planned on the device), one needing 257 has 257 (staged); 16
    directives are planned on the device, 17 are staged.  Each compared with
    the oracle."""
    need_gpu()
    say("planner limits")
    P, n_seq = 1, 18
    num_pages = 4096
    dp = DevicePool(1, num_pages, P, n_seq, 1100, seed=931)
    # sequence 0 holds the odd pages 1..2047 (1024 rows) and sequence 1 the
    # even pages from 2048 on, so the lowest free pages are 0, 2, 4, ...
    dp.set_pages(0, list(range(1, 2048, 2)), 1024)
    dp.set_pages(1, list(range(2048, 2048 + 512)), 512)
    for s in range(2, n_seq):
        dp.set_pages(s, list(range(2700 + 40 * s, 2700 + 40 * s + 20)), 20)
    dp.snapshot_rows()
    for grow, want in ((MAX_RUNS, 1), (MAX_RUNS + 1, 0)):
        # `grow` rows inserted at the start: at page size 1 only the stub rows
        # take fresh pages (every downstream row keeps its page, turned in
        # place), so the fresh pages are `grow` isolated even page ids
        expected, runs = _mla_splice(dp, [(1, 0, 0, grow, 7 + grow, O.AMORTIZE)], 0)
        assert runs == grow
        assert dp.pool.last_stats().planned_on_device == want
        compare_seq(dp, expected, 1)
        assert_same_free(dp, expected)
        dp.state = expected
    for k, want in ((MAX_DIRS, 1), (MAX_DIRS + 1, 0)):
        dirs = [(s, 2, 5, 1, 50 * k + s, O.AMORTIZE) for s in range(1, 1 + k)]
        expected, runs = _mla_splice(dp, dirs, 0)
        assert dp.pool.last_stats().planned_on_device == want, (k, runs)
        for s in range(n_seq):
            compare_seq(dp, expected, s)
        assert_same_free(dp, expected)
        dp.state = expected
    dp.close()


@pytest.mark.parametrize("H,D,rot,limit", [(1, 256, 256, 4), (2, 128, 128, 8)])
def test_gqa_directive_limit_follows_the_band_width(H, D, rot, limit):
    """GQA pools carry rotary_dim / 2 cos/sin pairs per directive in the
    kernel arguments: at most 1024 / rotary_dim directives are planned on the
    device, one more is staged; both match the oracle."""
    need_gpu()
    say(f"gqa planner limit H={H} D={D} rot={rot}")
    P, n_seq = 16, limit + 1
    dp = GqaDevicePool(2, 64 * n_seq + 256, P, n_seq, 64, H, D, rot, seed=941, pairing=1, base=500000.0)
    perm = permuted_pages(941, 40 * n_seq)
    for s in range(n_seq):
        dp.set_pages(s, perm[40 * s:40 * s + 40], 40 * P - 5)
    dp.snapshot_rows()
    for k, want in ((limit, 1), (limit + 1, 0)):
        dirs = [(s, 30 + s, 100 + 3 * s, 7 + s, 60 * k + s, O.AMORTIZE) for s in range(k)]
        expected, _ = dp.splice(dirs)
        assert dp.pool.last_stats().planned_on_device == want
        for s in range(n_seq):
            assert dp.compare(expected, s) == 0
        dp.state = expected
    dp.close()
