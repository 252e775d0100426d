"""GPU parity of the KV-streams trainer-side mask ("KV-streams", onedev.kr
summary, "how it works") against the CPU oracle, through the C ABI: death
times, block-mask lists and dense bit masks are integer results and must be
bit-exact.  A last test drives the engine's own eviction (kv_evict_compact on
a pool whose rows carry token ids) through the same log and checks that after
every event the cache holds exactly the tokens the death times keep alive."""

import numpy as np
import pytest

from oracle import kvs_mask_oracle as K
from synth import EvictionEvent, compaction_log, np_rng, permuted_pages

from gpu_common import need_gpu, say, torch

pytestmark = pytest.mark.gpu


def _logs(seed, lengths, strategies, budget, turn_lo, turn_hi, every):
    out = []
    for i, (n, st) in enumerate(zip(lengths, strategies)):
        out.append((n, compaction_log(np_rng(seed, i), n, st, budget, turn_lo, turn_hi, every)))
    return out


def _check_blocks(ctx, death, d_host, bq, bk, full_check=True, sample=None):
    pn, pi, fn, fi = ctx.block_mask(death, bq, bk)
    torch.cuda.synchronize()
    pn, pi, fn, fi = (x.cpu().numpy() for x in (pn, pi, fn, fi))
    n, n_pad = d_host.shape
    nq, nk = -(-n_pad // bq), -(-n_pad // bk)
    for r in range(n):
        if full_check:
            partial, full = K.block_mask(K.visibility(d_host[r]), bq, bk)
            for i in range(nq):
                assert list(pi[r, i, :pn[r, i]]) == partial[i], (r, i)
                assert list(fi[r, i, :fn[r, i]]) == full[i], (r, i)
        else:
            for i in sample:
                q0, q1 = i * bq, min(i * bq + bq, n_pad)
                part = [j for j in range(nk) if K.tile_class(d_host[r], q0, q1, j * bk, min(j * bk + bk, n_pad)) == "partial"]
                full = [j for j in range(nk) if K.tile_class(d_host[r], q0, q1, j * bk, min(j * bk + bk, n_pad)) == "full"]
                assert list(pi[r, i, :pn[r, i]]) == part, (r, i)
                assert list(fi[r, i, :fn[r, i]]) == full, (r, i)


def test_small_batches_all_outputs():
    L = need_gpu()
    ctx = L.KvsMask(0)
    cases = [
        (256, [256, 200, 131, 1], ["window", "half", "pick", "pick"]),
        (384, [384, 383, 250], ["pick", "window", "half"]),
        (1024, [1000, 1024], ["half", "pick"]),
    ]
    for seed, (n_pad, lengths, strategies) in enumerate(cases):
        say(f"kvs small n_pad={n_pad} lengths={lengths}")
        rolls = _logs(seed, lengths, strategies, budget=120, turn_lo=4, turn_hi=40, every=3)
        death, status = ctx.death_times(rolls, n_pad)
        torch.cuda.synchronize()
        assert not status.cpu().numpy().any()
        d_host = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
        assert np.array_equal(death.cpu().numpy().astype(np.int64), d_host)
        for bq, bk in ((16, 16), (32, 64), (64, 16), (128, 128)):
            _check_blocks(ctx, death, d_host, bq, bk)
        # caller-owned outputs (uninitialised): same counts, same lists up to them
        ref = [x.cpu().numpy() for x in ctx.block_mask(death, 32, 64)]
        out = tuple(torch.empty(x.shape, dtype=torch.int32, device="cuda") for x in ref)
        got = [x.cpu().numpy() for x in ctx.block_mask(death, 32, 64, out=out)]
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[2], ref[2])
        for r in range(len(rolls)):
            for i in range(ref[0].shape[1]):
                assert np.array_equal(got[1][r, i, :ref[0][r, i]], ref[1][r, i, :ref[0][r, i]])
                assert np.array_equal(got[3][r, i, :ref[2][r, i]], ref[3][r, i, :ref[2][r, i]])
        bits = ctx.dense_mask(death)
        torch.cuda.synchronize()
        got = bits.cpu().numpy().view(np.uint32)
        for r in range(len(rolls)):
            assert np.array_equal(got[r], K.dense_bits(K.visibility(d_host[r]))), r
    ctx.close()


def test_edge_logs():
    """No events (causal), an event dropping everything, an event at the very
    end, an empty rollout, and all-padding."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 256
    rolls = [
        (256, []),
        (200, [EvictionEvent(100, np.zeros(100, np.uint8))]),
        (256, [EvictionEvent(256, np.r_[np.ones(128, np.uint8), np.zeros(128, np.uint8)])]),
        (0, []),
        (130, [EvictionEvent(1, np.zeros(1, np.uint8)), EvictionEvent(2, np.ones(1, np.uint8))]),
    ]
    death, status = ctx.death_times(rolls, n_pad)
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any()
    d_host = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
    assert np.array_equal(death.cpu().numpy().astype(np.int64), d_host)
    _check_blocks(ctx, death, d_host, 32, 32)
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    got = bits.cpu().numpy().view(np.uint32)
    for r in range(len(rolls)):
        assert np.array_equal(got[r], K.dense_bits(K.visibility(d_host[r])))
    ctx.close()


def test_mismatched_mask_sets_status_of_that_rollout_only():
    L = need_gpu()
    ctx = L.KvsMask(0)
    good = compaction_log(np_rng(5, 0), 300, "pick", 100, 4, 30, 3)
    bad = [EvictionEvent(good[0].time, good[0].keep)] + \
          [EvictionEvent(good[1].time, np.ones(len(good[1].keep) + 1, np.uint8))]
    death, status = ctx.death_times([(300, good), (300, bad), (300, good)], 384)
    torch.cuda.synchronize()
    assert list(status.cpu().numpy()) == [0, 1, 0]
    d = death.cpu().numpy().astype(np.int64)
    ref = K.death_times(384, 300, good)
    assert np.array_equal(d[0], ref) and np.array_equal(d[2], ref)
    ctx.close()


@pytest.mark.slow
def test_textworld_shaped_batch_32k():
    """Eight 32768-token rollouts (turns U[64, 512], compaction every 10 turns,
    budget 8192, the three strategies): death times bit-exact; block lists of
    sampled query blocks (128 x 128 tiles); dense bit rows sampled."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 32768
    strategies = ["window", "half", "pick"] * 3
    rolls = _logs(77, [32768] * 8, strategies[:8], budget=8192, turn_lo=64, turn_hi=512, every=10)
    say(f"kvs 8 x 32k, events per rollout {[len(ev) for _, ev in rolls]}")
    death, status = ctx.death_times(rolls, n_pad)
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any()
    d_host = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
    assert np.array_equal(death.cpu().numpy().astype(np.int64), d_host)
    _check_blocks(ctx, death, d_host, 128, 128, full_check=False, sample=[0, 1, 63, 100, 200, 255])
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 5000, 12345, 20000, 32767])
    for r in (0, 3, 7):
        got = bits[r, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, K.dense_bits(K.visibility_rows(d_host[r], rows))), r
    ctx.close()


@pytest.mark.slow
def test_bench_shaped_batch_64x32k():
    """The trainer-mask workload as it is timed: 64 rollouts of 32768 tokens
    (turns U[64, 512], compaction every 10 turns, budget 8192, the three
    strategies in turn; the same seeds), logs uploaded once, then death
    times, the 128 x 128 block mask and the dense mask into caller-owned
    outputs, twice (the second call reuses the outputs and the scratch).
    Death times of every rollout bit-exact; sampled query blocks of every
    rollout; dense rows of every rollout sampled at run edges, event times
    and at random, against the definition."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 32768
    strategies = ("window", "half", "pick")
    rolls = [(n_pad, compaction_log(np_rng(0, 10 + i), n_pad, strategies[i % 3], 8192, 64, 512, 10))
             for i in range(64)]
    say("kvs 64 x 32k, the timed workload's launches")
    logs = ctx.upload_logs(rolls)
    death, status = ctx.death_times(logs, n_pad)
    bits = ctx.dense_mask(death)
    blocks = ctx.block_mask(death, 128, 128)
    ctx.death_times(logs, n_pad, out=(death, status))
    ctx.block_mask(death, 128, 128, out=blocks)
    ctx.dense_mask(death, out=bits)
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any()
    d_host = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
    assert np.array_equal(death.cpu().numpy().astype(np.int64), d_host)
    _check_blocks(ctx, death, d_host, 128, 128, full_check=False, sample=[0, 100, 255])
    pn, pi, fn, fi = (x.cpu().numpy() for x in blocks)
    for r in range(0, 64, 9):  # the timed call's own block lists, as in the check above
        for i in (1, 128):
            q0, q1 = i * 128, i * 128 + 128
            cls = [K.tile_class(d_host[r], q0, q1, j * 128, j * 128 + 128) for j in range(256)]
            assert list(pi[r, i, :pn[r, i]]) == [j for j, c in enumerate(cls) if c == "partial"], (r, i)
            assert list(fi[r, i, :fn[r, i]]) == [j for j, c in enumerate(cls) if c == "full"], (r, i)
    rng = np_rng(64, 32)
    for r in range(64):
        times = np.array([e.time for e in rolls[r][1] if e.time < n_pad], np.int64)
        rows = np.unique(np.r_[[0, 7, 8, n_pad - 8, n_pad - 1], times - 1, times,
                              rng.integers(0, n_pad, size=6)])
        got = bits[r, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, K.dense_bits(K.visibility_rows(d_host[r], rows))), r
    del bits
    ctx.close()


def test_engine_eviction_agrees_with_death_times():
    """A one-layer MLA pool (page size 16) whose rows carry their token id in
    the first two bf16 slots; tokens are appended event by event and each
    event's keep mask goes to kv_evict_compact.  After each event the pool's
    rows are exactly the tokens k < t with d_k > t."""
    L = need_gpu()
    P, n_tok = 16, 4000
    log = compaction_log(np_rng(9, 0), n_tok, "pick", 1500, 32, 256, 4)
    ctx = L.KvsMask(0)
    death, status = ctx.death_times([(n_tok, log)], 4096)
    torch.cuda.synchronize()
    assert status.item() == 0
    d = death[0].cpu().numpy().astype(np.int64)
    pages = 2 * n_tok // P
    ids = np.zeros((1, pages, P, 576), np.uint16)
    data = torch.from_numpy(ids.view(np.int16)).view(torch.bfloat16).cuda()
    table = torch.full((1, pages), -1, dtype=torch.int32, device="cuda")
    pool = L.Pool(data, table)
    held, t_prev = [], 0
    perm = list(permuted_pages(9, pages))
    for e in log:
        # append tokens t_prev .. e.time - 1: write their ids into the next rows
        n_before = len(held)
        _, _, tab = pool.seq_get(0) if n_before or t_prev else (0, 0, np.zeros(0, np.int32))
        tab = list(tab)
        new = list(range(t_prev, e.time))
        need = -(-(n_before + len(new)) // P)
        free = [p for p in perm if p not in set(tab)]   # one sequence: every other page is free
        tab += free[:need - len(tab)]
        flat = data.view(torch.int16).view(-1, 576)
        j = np.arange(n_before, n_before + len(new))
        rows = torch.from_numpy(np.asarray(tab, np.int64)[j // P] * P + j % P).cuda()
        vals = torch.from_numpy(np.asarray(new, np.int64))
        flat[rows, 0] = (vals & 0x7FFF).to(torch.int16).cuda()
        flat[rows, 1] = (vals >> 15).to(torch.int16).cuda()
        pool.seq_set_pages(0, tab, n_before + len(new))
        held = held + new
        assert len(e.keep) == len(held)
        pool.evict([0], torch.from_numpy(e.keep).cuda(), [0])
        torch.cuda.synchronize()
        n, _, tab = pool.seq_get(0)
        j = np.arange(n)
        rows = torch.from_numpy(tab.astype(np.int64)[j // P] * P + j % P).cuda()
        got = flat[rows, :2].cpu().numpy().astype(np.int64)
        alive = got[:, 0] + (got[:, 1] << 15)
        assert np.array_equal(alive, np.flatnonzero(d[:e.time] > e.time)), e.time
        held = list(alive)
        t_prev = e.time
    pool.close()
    ctx.close()


def test_dense_mask_of_arbitrary_death_times_both_kernels():
    """Dense bits of death arrays written directly, not replayed from a log:
    exactly 15 and 16 distinct death times (the two sides of the per-key code
    limit), hundreds of distinct times, none, and values outside (k, n_pad)
    (negative, equal to k, beyond n_pad), all in one batch so that rollouts
    of both mask kernels share a launch.  Every row bit-exact against the
    definition visible(q, k) = k <= q < d_k."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    rng = np_rng(4242, 0)
    for n_pad in (1024, 1152):
        say(f"kvs dense arbitrary death times n_pad={n_pad}")
        k = np.arange(n_pad)
        rolls = []
        for n_times in (15, 16, 0, 300, 1):
            times = np.sort(rng.choice(np.arange(1, n_pad), size=n_times, replace=False)) if n_times else np.zeros(0, np.int64)
            d = np.full(n_pad, n_pad, np.int64)
            if n_times:
                dies = rng.random(n_pad) < 0.5
                pick = times[rng.integers(0, n_times, size=n_pad)]
                d = np.where(dies & (pick > k), pick, d)
                d[times - 1] = times      # every time taken: key t - 1 dies at t
            rolls.append(d)
        odd = np.full(n_pad, n_pad, np.int64)
        odd[::7] = -5                     # never visible
        odd[1::7] = k[1::7]               # d_k = k: never visible
        odd[2::7] = n_pad + 1000          # beyond the last row
        odd[3::7] = np.minimum(k[3::7] + 1, n_pad)   # visible on its own row only
        odd[4::7] = np.where(k[4::7] < 600, 600, n_pad)
        rolls.append(odd)
        d_host = np.stack(rolls)
        got_times = [len(set(int(x) for j, x in enumerate(r) if j < x < n_pad)) for r in d_host]
        assert got_times[:2] == [15, 16] and got_times[2] == 0 and got_times[3] > 15
        death = torch.from_numpy(d_host.astype(np.int32)).cuda()
        bits = ctx.dense_mask(death)
        torch.cuda.synchronize()
        got = bits.cpu().numpy().view(np.uint32)
        for r in range(len(rolls)):
            assert np.array_equal(got[r], K.dense_bits(K.visibility(d_host[r]))), (n_pad, r, got_times[r])
    ctx.close()


def test_dense_mask_at_the_smallest_pad():
    """n_pad = 128, the smallest: rows of 16 bytes (one strip of 128 keys, one
    active lane per wave, runs of 8 rows), death arrays written directly --
    causal (no death), 3 distinct death times, 20 (the rebuild walk), no key
    ever visible, every key visible on its own row only -- in one batch;
    every bit row against the definition."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 128
    k = np.arange(n_pad)
    rng = np_rng(128, 0)
    few = np.full(n_pad, n_pad, np.int64)
    times3 = np.array([9, 64, 127])
    pick = times3[rng.integers(0, 3, size=n_pad)]
    few = np.where(pick > k, pick, few)
    many = np.minimum(k + 1 + rng.integers(0, 40, size=n_pad), n_pad + 1)
    d_host = np.stack([np.full(n_pad, n_pad, np.int64), few, many, np.full(n_pad, -1, np.int64),
                       np.minimum(k + 1, n_pad)])
    counts = [len(set(int(x) for j, x in enumerate(r) if j < x < n_pad)) for r in d_host]
    assert counts[1] == 3 and counts[2] > 15
    say(f"kvs dense n_pad={n_pad}, distinct death times {counts}")
    death = torch.from_numpy(d_host.astype(np.int32)).cuda()
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    got = bits.cpu().numpy().view(np.uint32)
    for r in range(len(d_host)):
        assert np.array_equal(got[r], K.dense_bits(K.visibility(d_host[r]))), (r, counts[r])
    ctx.close()


def test_death_times_of_events_spanning_several_replay_tiles():
    """Events whose keep masks cover more than 16384 rows, the replay's tile:
    the kept count carries from tile to tile.  Masks keeping 70% and 50% at
    random, keeping everything, dropping everything; death times bit-exact,
    sampled dense rows against the definition."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 40960
    rng = np_rng(31, 0)
    t1, t2 = 38000, 40000
    keep1 = (rng.random(t1) < 0.7).astype(np.uint8)
    keep2 = (rng.random(int(keep1.sum()) + t2 - t1) < 0.5).astype(np.uint8)
    rolls = [
        (t2, [EvictionEvent(t1, keep1), EvictionEvent(t2, keep2)]),
        (n_pad, [EvictionEvent(20000, np.ones(20000, np.uint8)), EvictionEvent(n_pad, np.zeros(n_pad, np.uint8))]),
        (33000, [EvictionEvent(16385, (rng.random(16385) < 0.3).astype(np.uint8))]),
    ]
    say(f"kvs replay over several tiles, rows per event {[[len(e.keep) for e in ev] for _, ev in rolls]}")
    death, status = ctx.death_times(rolls, n_pad)
    torch.cuda.synchronize()
    assert not status.cpu().numpy().any()
    d_host = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
    assert np.array_equal(death.cpu().numpy().astype(np.int64), d_host)
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    rows = np.array([0, 16383, 16384, 20000, 37999, 38000, 39999, 40000, 40959])
    for r in range(len(rolls)):
        got = bits[r, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, K.dense_bits(K.visibility_rows(d_host[r], rows))), r
    ctx.close()


def test_dense_mask_beyond_the_pre_pass_limit():
    """n_pad = 262272, past the 262144 keys whose death-time set fits in LDS:
    the rebuild walk writes every rollout alone.  One rollout (8.6 GB of
    bits) with hundreds of distinct death times, never-visible keys and keys
    visible to the end; sampled rows against the definition."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 262272
    rng = np_rng(32, 0)
    k = np.arange(n_pad)
    d = np.minimum(k + 1 + rng.integers(0, 5000, size=n_pad), n_pad + 7)
    d[rng.random(n_pad) < 0.1] = n_pad
    d[rng.random(n_pad) < 0.05] = -1
    say(f"kvs dense n_pad={n_pad}, rebuild walk only")
    death = torch.from_numpy(d[None].astype(np.int32)).cuda()
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    rows = np.r_[[0, 127, 128, 131071, 262143, 262144, 262271], rng.integers(0, n_pad, size=5)]
    got = bits[0, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, K.dense_bits(K.visibility_rows(d, rows)))
    del bits
    ctx.close()


def test_dense_mask_of_wide_rows_both_walks():
    """n_pad = 163840: rows of 20 KiB, more than the 4 x 64 strips of 128 keys
    a lane of the code walk holds at once (five passes over a wave's run of 8
    rows), and more rebuild-walk waves than the rollout has runs of 8 rows
    (the waves of a rollout with too many death times take several).  One
    rollout with exactly 15 distinct death times (the code walk), one with
    hundreds (the rebuild walk), one with none; sampled rows -- the first and
    last row of runs, rows on each side of death times, the last rows --
    against the definition visible(q, k) = k <= q < d_k."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 163840
    rng = np_rng(33, 0)
    k = np.arange(n_pad)
    times = np.sort(rng.choice(np.arange(1, n_pad), size=15, replace=False))
    d15 = np.full(n_pad, n_pad, np.int64)
    pick = times[rng.integers(0, 15, size=n_pad)]
    d15 = np.where((rng.random(n_pad) < 0.6) & (pick > k), pick, d15)
    d15[times - 1] = times
    d15[rng.random(n_pad) < 0.05] = -3
    dmany = np.minimum(k + 1 + rng.integers(0, 3000, size=n_pad), n_pad + 5)
    dmany[rng.random(n_pad) < 0.1] = n_pad
    dnone = np.full(n_pad, n_pad, np.int64)
    d_host = np.stack([d15, dmany, dnone])
    assert len(set(int(x) for j, x in enumerate(d15) if j < x < n_pad)) == 15
    say(f"kvs dense n_pad={n_pad}: code walk in five passes, rebuild walk over several runs per wave")
    death = torch.from_numpy(d_host.astype(np.int32)).cuda()
    bits = ctx.dense_mask(death)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[[0, 7, 8, 32767, 32768, 131071, 131072, 131080, n_pad - 9, n_pad - 8, n_pad - 1],
                          times - 1, times, np.minimum(times + 1, n_pad - 1), rng.integers(0, n_pad, size=24)])
    for r in range(3):
        got = bits[r, torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, K.dense_bits(K.visibility_rows(d_host[r], rows))), r
    del bits
    ctx.close()


def test_masks_on_alternating_streams_share_the_scratch():
    """Dense and block masks of three batches issued back to back on two
    streams, then on the first again.  The first batch is long (24 rollouts
    of 16384: 805 MB of mask bits), the later ones short, so the later calls
    would overwrite the shared scratch while the first still reads it unless
    the library orders them after it on the device.  Every result compared
    with the definition (the long batch on sampled rows and query blocks)."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    rng = np_rng(33, 0)
    shapes = [(24, 16384), (4, 2048), (4, 2048)]
    batches = []
    for b, (n, n_pad) in enumerate(shapes):
        k = np.arange(n_pad)
        times = np.sort(rng.choice(np.arange(1, n_pad), size=(9, 5, 40)[b], replace=False))
        d = np.where(rng.random((n, n_pad)) < 0.6, times[rng.integers(0, len(times), size=(n, n_pad))], n_pad)
        batches.append(np.where(d > k, d, n_pad))
    streams = [torch.cuda.Stream(), torch.cuda.Stream(), None]
    # inputs and outputs made first and kept alive until the end, so that
    # only the library orders the three calls
    deaths = [torch.from_numpy(d.astype(np.int32)).cuda() for d in batches]
    bufs = []
    for n, n_pad in shapes:
        nb = n_pad // 64
        bufs.append((torch.empty((n, n_pad, n_pad // 32), dtype=torch.int32, device="cuda"),
                     tuple(torch.empty(sh, dtype=torch.int32, device="cuda")
                           for sh in ((n, nb), (n, nb, nb), (n, nb), (n, nb, nb)))))
    torch.cuda.synchronize()
    outs = []
    for death, st, (bits, blocks) in zip(deaths, streams, bufs):
        say(f"kvs masks {tuple(death.shape)} on stream {st}")
        outs.append((ctx.dense_mask(death, out=bits, stream=st), ctx.block_mask(death, 64, 64, out=blocks, stream=st)))
    torch.cuda.synchronize()
    for d, (bits, blocks) in zip(batches[1:], outs[1:]):
        got = bits.cpu().numpy().view(np.uint32)
        pn, pi, fn, fi = (x.cpu().numpy() for x in blocks)
        for r in range(d.shape[0]):
            vis = K.visibility(d[r])
            assert np.array_equal(got[r], K.dense_bits(vis)), r
            partial, full = K.block_mask(vis, 64, 64)
            for i in range(len(partial)):
                assert list(pi[r, i, :pn[r, i]]) == partial[i] and list(fi[r, i, :fn[r, i]]) == full[i], (r, i)
    d = batches[0]
    n, n_pad = d.shape
    bits, blocks = outs[0]
    rows = np.array([0, 1, 63, 64, 2047, 4096, 9999, n_pad - 1])
    idx = torch.from_numpy(rows).cuda()
    pn, pi, fn, fi = (x.cpu().numpy() for x in blocks)
    nk = n_pad // 64
    for r in range(n):
        got = bits[r, idx].cpu().numpy().view(np.uint32)
        assert np.array_equal(got, K.dense_bits(K.visibility_rows(d[r], rows))), r
        for i in (0, 1, 100, nk - 1):
            cls = [K.tile_class(d[r], i * 64, i * 64 + 64, j * 64, j * 64 + 64) for j in range(nk)]
            assert list(pi[r, i, :pn[r, i]]) == [j for j in range(nk) if cls[j] == "partial"], (r, i)
            assert list(fi[r, i, :fn[r, i]]) == [j for j in range(nk) if cls[j] == "full"], (r, i)
    ctx.close()


def test_death_times_on_alternating_streams_share_the_list_scratch():
    """Death times past the LDS list (n_pad = 50000 keeps each rollout's held
    tokens in the context's list scratch): a long call of 64 rollouts on one
    stream, a short one on another right after it, then three more on the
    first stream (the staging ring's regions taken in turn).  The short call
    reuses the list rows the long one is still replaying unless the library
    orders it after that call on the device.  Bit-exact against the oracle."""
    L = need_gpu()
    ctx = L.KvsMask(0)
    n_pad = 50000
    calls = [(0, _logs(91, [n_pad - 7 * i for i in range(64)], ["window", "half", "pick"] * 22, budget=12000,
                       turn_lo=64, turn_hi=512, every=4)),
             (1, _logs(92, [n_pad, n_pad - 1000], ["pick", "half"], budget=9000, turn_lo=64, turn_hi=512, every=3))]
    calls += [(0, _logs(93 + c, [n_pad - 300 * c], ["pick"], budget=5000, turn_lo=32, turn_hi=256, every=5))
              for c in range(3)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    logs = [ctx.upload_logs(rolls) for _, rolls in calls]
    outs = [(torch.empty((len(rolls), n_pad), dtype=torch.int32, device="cuda"),
             torch.empty(len(rolls), dtype=torch.int32, device="cuda")) for _, rolls in calls]
    torch.cuda.synchronize()
    for (si, rolls), lg, out in zip(calls, logs, outs):
        say(f"kvs death times, {len(rolls)} rollouts of up to {n_pad} on stream {si}")
        ctx.death_times(lg, n_pad, stream=streams[si], out=out)
    torch.cuda.synchronize()
    for (_, rolls), (death, status) in zip(calls, outs):
        assert not status.cpu().numpy().any()
        want = np.stack([K.death_times(n_pad, n, ev) for n, ev in rolls])
        assert np.array_equal(death.cpu().numpy().astype(np.int64), want)
    ctx.close()
