"""GPU parity of leyline_splice (Leyline summary, sections 2.1-2.3) against the
CPU oracle, through the C ABI: page tables, lengths and positions bit-exact,
moved c_kv and stub rows bit-exact, rotated k_pe within 1 bf16 ulp (the
library is built to match the oracle's float32 order exactly, so 0 is
expected and reported)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import draw_span, np_rng, permuted_pages

from gpu_common import DevicePool, assert_same_free, compare_seq, need_gpu, say, torch

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _splice_both(dp, directives):
    """directives: list of (seq, s0, s1, r_len, seed, mode).  Runs the oracle
    on the host mirror and the library on the device."""
    L = need_gpu()
    lib_dirs, ora_dirs = [], []
    for (seq, s0, s1, r, seed, mode) in directives:
        dev, host = dp.stub(seed, r if mode == O.AMORTIZE else 0)
        lib_dirs.append(L.Directive(seq, s0, s1, dev, mode))
        ora_dirs.append(O.Directive(seq, s0, s1, r if mode == O.AMORTIZE else 0, host, mode))
    expected, plans = O.splice(dp.state, ora_dirs, pairing="half" if dp.pool_pairing else "interleaved")
    dp.pool.splice(lib_dirs)
    torch.cuda.synchronize()
    return expected, plans


def _pool(L, num_pages, P, max_seqs, max_pages, seed=0, pairing=0, host_rows=True, oracle_layers=None):
    dp = DevicePool(L, num_pages, P, max_seqs, max_pages, seed=seed, host_rows=host_rows, pairing=pairing,
                    oracle_layers=oracle_layers)
    dp.pool_pairing = pairing
    return dp


def test_splice_4k_one_layer_identity_table():
    """One layer, 4096 tokens, page size 16, identity table; splice
    [1000, 3000) for 16 stub rows (Delta = -1984)."""
    say("splice_4k_1layer")
    g = json.load(open(os.path.join(GOLDEN, "splice_plans.json")))["splice_4k_1layer"]
    dp = _pool(1, 512, 16, 1, 300, seed=11)
    dp.set_pages(0, np.arange(256), 4096)
    dp.snapshot_rows()
    expected, _ = _splice_both(dp, [(0, 1000, 3000, 16, 12, O.AMORTIZE)])
    worst = compare_seq(dp, expected, 0)
    assert_same_free(dp, expected)
    st = dp.pool.last_stats()
    assert st.alg_bytes == g["bytes"] and st.fresh_pages == g["fresh_pages"]
    assert st.rows_moved == g["moved_rows"] and st.rows_rotated_inplace == g["inplace_rows"]
    say(f"  max k_pe ulp = {worst}")
    dp.close()


@pytest.mark.parametrize("P,pairing", [(1, 0), (2, 0), (16, 0), (16, 1), (32, 0)])
def test_splice_tiny_sweep(P, pairing):
    """Every span of small caches (several pages plus a ragged tail), stub
    lengths 0, 1 and P+3, two layers, page tables permuted."""
    say(f"tiny sweep P={P} pairing={pairing}")
    worst = 0
    cases = 0
    for n in sorted({1, P + 3, 3 * P + 5}):
        spans = list(itertools.combinations_with_replacement(range(0, n + 1, max(1, n // 9)), 2))
        spans += [(0, n), (n, n), (0, 0), (n // 2, n)]
        for s0, s1 in spans:
            for r in (0, 1, P + 3):
                pages_needed = -(-n // P)
                dp = _pool(2, 4 * pages_needed + 8, P, 2, 4 * pages_needed + 8, seed=cases, pairing=pairing)
                T = permuted_pages(cases, 4 * pages_needed + 8)[:pages_needed]
                dp.set_pages(1, T, n)
                dp.snapshot_rows()
                expected, _ = _splice_both(dp, [(1, s0, s1, r, 1000 + cases, O.AMORTIZE)])
                worst = max(worst, compare_seq(dp, expected, 1))
                assert_same_free(dp, expected)
                dp.close()
                cases += 1
    say(f"  {cases} cases, max k_pe ulp = {worst}")


def test_splice_32k_27_layers_full_compare():
    """27 layers, 32768 tokens, page size 16, permuted pages; splice
    [8192, 14336) for 24 stub rows (Delta = -6120), compared row by row on
    every layer -- the benchmark's own workload and launch."""
    say("splice_32k_27layer full compare")
    g = json.load(open(os.path.join(GOLDEN, "splice_plans.json")))["splice_32k_27layer"]
    dp = _pool(27, 4096, 16, 1, 2048, seed=0, host_rows=False)
    dp.set_pages(0, permuted_pages(0, 2048), 32768)
    dp.snapshot_rows()
    expected, _ = _splice_both(dp, [(0, 8192, 14336, 24, 1, O.AMORTIZE)])
    worst = compare_seq(dp, expected, 0)
    assert_same_free(dp, expected)
    st = dp.pool.last_stats()
    assert st.alg_bytes == g["bytes"] and st.fresh_pages == g["fresh_pages"] and st.freed_pages == g["freed_pages"]
    say(f"  max k_pe ulp = {worst}")
    dp.close()


def test_splice_32k_27_layers_inplace_full_compare():
    """The same sequence spliced with no stub rows: Delta = -6144, a whole
    number of 16-row pages, so every downstream page is reused and only its
    k_pe band turns in place (the in-place kernel alone, with the page-table
    rewrite); every row of every layer compared."""
    say("splice_32k_27layer_inplace full compare")
    dp = _pool(27, 4096, 16, 1, 2048, seed=0, host_rows=False)
    dp.set_pages(0, permuted_pages(0, 2048), 32768)
    dp.snapshot_rows()
    expected, _ = _splice_both(dp, [(0, 8192, 14336, 0, 1, O.AMORTIZE)])
    worst = compare_seq(dp, expected, 0)
    assert_same_free(dp, expected)
    st = dp.pool.last_stats()
    assert st.fresh_pages == 0 and st.rows_moved == 0 and st.rows_rotated_inplace == 32768 - 14336
    assert st.alg_bytes == 27 * (32768 - 14336) * 2 * 128
    say(f"  max k_pe ulp = {worst}")
    dp.close()


def _batched(L, n_tokens, n_seqs, seed, oracle_layers=None, host_rows=True):
    rng = np_rng(seed, 4)
    pages_per = n_tokens // 16
    dp = _pool(L, 2 * n_seqs * pages_per, 16, n_seqs, pages_per + 8, seed=seed, host_rows=host_rows,
               oracle_layers=oracle_layers)
    perm = permuted_pages(seed, n_seqs * pages_per)
    for s in range(n_seqs):
        dp.set_pages(s, perm[s * pages_per:(s + 1) * pages_per], n_tokens)
    dirs = []
    for s in range(n_seqs):
        d = draw_span(rng, n_tokens, min(256, n_tokens // 4), min(8192, n_tokens // 2), 8, 64,
                      start_lo=min(1024, n_tokens // 8))
        dirs.append((s, d.s_start, d.s_end, d.r_len, 100 + s, O.AMORTIZE))
    order = list(rng.permutation(n_seqs))
    return dp, [dirs[i] for i in order]


def test_splice_batched_16_sequences_small():
    """One call with 16 independent directives (span, stub and start drawn at
    random), 4096-token sequences, 3 layers, every row compared."""
    say("batched 16 x 4096 x 3")
    dp, dirs = _batched(3, 4096, 16, seed=21)
    dp.snapshot_rows()
    expected, _ = _splice_both(dp, dirs)
    for s in range(16):
        compare_seq(dp, expected, s)
    assert_same_free(dp, expected)
    dp.close()


@pytest.mark.slow
def test_splice_batched_16x32k_27_layers_sampled_layers():
    """Concurrency 16: 16 x 32768 tokens x 27 layers in one pool with one
    random directive each, one call.  Page tables of all sequences compared;
    rows compared on layers 0, 13 and 26."""
    say("batched 16 x 32768 x 27")
    dp, dirs = _batched(27, 32768, 16, seed=0, oracle_layers=[0, 13, 26], host_rows=False)
    dp.snapshot_rows()
    expected, _ = _splice_both(dp, dirs)
    for s in range(16):
        compare_seq(dp, expected, s)
    assert_same_free(dp, expected)
    dp.close()


def test_splice_half_split_pairing_moves_and_in_place():
    say("half-split pairing")
    dp = _pool(2, 64, 16, 1, 64, seed=31, pairing=1)
    dp.set_pages(0, permuted_pages(31, 64)[:20], 310)
    dp.snapshot_rows()
    # Delta = -32: downstream pages reused and rotated in place
    expected, _ = _splice_both(dp, [(0, 40, 80, 8, 5, O.AMORTIZE)])
    compare_seq(dp, expected, 0)
    dp.state = expected
    # Delta = +3: moved and rotated
    expected, _ = _splice_both(dp, [(0, 17, 18, 4, 6, O.AMORTIZE)])
    compare_seq(dp, expected, 0)
    dp.close()


def test_splice_successive_directives_and_forget():
    """Directives applied one after another on the same sequence (rows
    rotated several times), then a FORGET."""
    say("successive splices")
    dp = _pool(2, 200, 16, 2, 200, seed=41)
    dp.set_pages(0, permuted_pages(41, 200)[:63], 1000)
    dp.set_pages(1, permuted_pages(41, 200)[64:100], 570)
    dp.snapshot_rows()
    rng = np.random.default_rng(41)
    for step in range(6):
        n0 = dp.state.lengths[0]
        s0 = int(rng.integers(0, n0 // 2))
        s1 = int(rng.integers(s0, n0))
        r = int(rng.integers(0, 40))
        expected, _ = _splice_both(dp, [(0, s0, s1, r, 50 + step, O.AMORTIZE), (1, 10, 10 + step, step, 70 + step, O.AMORTIZE)])
        compare_seq(dp, expected, 0)
        compare_seq(dp, expected, 1)
        dp.state = expected
    expected, _ = _splice_both(dp, [(0, 33, 40, 0, 0, O.FORGET)])
    compare_seq(dp, expected, 0)
    compare_seq(dp, expected, 1)
    assert_same_free(dp, expected)
    dp.close()


def test_splice_edge_cases():
    say("edge cases")
    dp = _pool(1, 64, 16, 4, 8, seed=51)
    dp.set_pages(0, [5, 9, 2], 40)
    dp.set_pages(1, [7], 16)
    dp.set_pages(2, [], 0)
    dp.snapshot_rows()
    # empty batch is a no-op
    dp.pool.splice([])
    # insertion into an empty sequence; whole-sequence deletion; pure insertion
    expected, _ = _splice_both(dp, [(2, 0, 0, 5, 1, O.AMORTIZE), (1, 0, 16, 0, 0, O.AMORTIZE),
                                    (0, 40, 40, 3, 2, O.AMORTIZE)])
    for s in range(3):
        compare_seq(dp, expected, s)
    dp.state = expected
    # grow to the full page-table row (8 pages = 128 rows)
    expected, _ = _splice_both(dp, [(0, 10, 11, 128 - 42, 3, O.AMORTIZE)])
    compare_seq(dp, expected, 0)
    assert dp.pool.seq_get(0)[0] == 128
    dp.close()


def test_splice_rejects_bad_requests_and_keeps_state():
    L = need_gpu()
    say("error paths")
    dp = _pool(1, 20, 16, 3, 10, seed=61)
    dp.set_pages(0, list(range(7)), 100)
    dp.set_pages(1, list(range(7, 11)), 64)
    before = [dp.pool.seq_get(s) for s in (0, 1)]
    free = dp.pool.free_pages()
    stub, _ = dp.stub(1, 4)
    big, _ = dp.stub(2, 100)
    bad = [
        ([L.Directive(0, 50, 40)], L.LL_EINVAL),
        ([L.Directive(0, 50, 101)], L.LL_EINVAL),
        ([L.Directive(2, 0, 0)], L.LL_EINVAL),                       # unknown sequence
        ([L.Directive(0, 1, 2, stub), L.Directive(0, 3, 4)], L.LL_EINVAL),  # repeated sequence
        ([L.Directive(0, 1, 2, None, L.PIN)], L.LL_EUNSUPPORTED),
        ([L.Directive(0, 0, 0, big)], L.LL_ERANGE),
        ([L.Directive(0, 0, 1, stub), L.Directive(1, 0, 1, stub)], L.LL_ENOMEM),
    ]
    for dirs, code in bad:
        with pytest.raises(L.LeylineError) as ei:
            dp.pool.splice(dirs)
        assert ei.value.status == code, (ei.value, code)
    after = [dp.pool.seq_get(s) for s in (0, 1)]
    for (n0, p0, t0), (n1, p1, t1) in zip(before, after):
        assert n0 == n1 and p0 == p1 and np.array_equal(t0, t1)
    assert dp.pool.free_pages() == free
    dp.close()


def test_splice_is_deterministic():
    say("determinism")
    outs = []
    for _ in range(2):
        dp = _pool(2, 300, 16, 1, 300, seed=71)
        dp.set_pages(0, permuted_pages(71, 300)[:200], 3190)
        dp.snapshot_rows()
        _splice_both(dp, [(0, 700, 2100, 37, 9, O.AMORTIZE)])
        outs.append((dp.data.view(torch.int16).cpu().numpy().copy(), dp.pool.seq_get(0)[2].copy(),
                     dp.table.cpu().numpy().copy()))
        dp.close()
    # rows outside the sequence are unspecified; compare the live table and
    # the live rows
    (d0, t0, pt0), (d1, t1, pt1) = outs
    assert np.array_equal(t0, t1) and np.array_equal(pt0[0, :len(t0)], pt1[0, :len(t1)])
    rows = (t0.astype(np.int64)[:, None] * 16 + np.arange(16)).ravel()
    assert np.array_equal(d0.reshape(2, -1, O.ROW)[:, rows], d1.reshape(2, -1, O.ROW)[:, rows])


def test_splice_batch_of_40_takes_several_launches():
    """40 directives in one call (more than one launch's worth), mixed
    shapes: page-aligned shifts (in-place rotation), ragged shifts, pure
    insertions, deletions to empty, FORGET; every row compared."""
    say("batch of 40")
    rng = np.random.default_rng(81)
    n_seq = 40
    lengths = [int(x) for x in rng.integers(1, 700, size=n_seq)]
    total = sum(-(-n // 16) for n in lengths)
    dp = _pool(2, 3 * total + 64, 16, n_seq, 200, seed=81)
    perm = permuted_pages(81, 3 * total + 64)
    at = 0
    for s, n in enumerate(lengths):
        k = -(-n // 16)
        dp.set_pages(s, perm[at:at + k], n)
        at += k
    dp.snapshot_rows()
    dirs = []
    for s, n in enumerate(lengths):
        kind = s % 5
        if kind == 0:    # delta = -32: downstream pages reused, rotated in place
            s0 = int(rng.integers(0, max(1, n - 40))); s1 = min(n, s0 + 40); r = 8 if s1 - s0 == 40 else 0
        elif kind == 1:  # ragged shift
            s0 = int(rng.integers(0, n)); s1 = int(rng.integers(s0, n + 1)); r = int(rng.integers(0, 30))
        elif kind == 2:  # pure insertion
            s0 = s1 = int(rng.integers(0, n + 1)); r = int(rng.integers(1, 20))
        elif kind == 3:  # delete everything
            s0, s1, r = 0, n, 0
        else:
            s0, s1, r = int(rng.integers(0, n + 1)), n, 0
        mode = O.FORGET if kind == 4 else O.AMORTIZE
        dirs.append((s, s0, s1, r, 500 + s, mode))
    order = list(rng.permutation(n_seq))
    expected, _ = _splice_both(dp, [dirs[i] for i in order])
    for s in range(n_seq):
        compare_seq(dp, expected, s)
    assert_same_free(dp, expected)
    dp.close()


def test_sampled_profiling_times_every_nth_launch_and_keeps_results():
    """ll_pool_set_profiling(n) stamps every n-th launch, counted from the
    call; the timed bytes are the plan's algorithmic bytes plus its page-table
    entries; results are those of the oracle whether a launch is timed or not."""
    say("sampled profiling")
    dp = _pool(2, 800, 16, 1, 300, seed=91)
    dp.set_pages(0, permuted_pages(91, 800)[:250], 3990)
    dp.snapshot_rows()
    dp.pool.set_profiling(True, 3)
    per_call = []
    expected = None
    for i in range(7):   # launches 0, 3 and 6 are timed
        expected, _ = _splice_both(dp, [(0, 100 + 7 * i, 300 + 7 * i, 5 + i, 40 + i, O.AMORTIZE)])
        dp.state = expected
        st = dp.pool.last_stats()
        per_call.append(st.alg_bytes + 4 * st.table_entries)
    dp.pool.set_profiling(False)
    n, ms, b = dp.pool.profile_read(0)
    assert n == 3 and ms > 0
    assert b == per_call[0] + per_call[3] + per_call[6]
    assert dp.pool.profile_read(0) == (0, 0.0, 0)      # read clears
    compare_seq(dp, expected, 0)
    assert_same_free(dp, expected)
    dp.pool.set_profiling(True)                          # every launch
    _splice_both(dp, [(0, 0, 0, 3, 99, O.AMORTIZE)])
    dp.pool.set_profiling(False)
    assert dp.pool.profile_read(0)[0] == 1
    dp.close()
