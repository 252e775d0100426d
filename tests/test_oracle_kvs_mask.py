"""Pins for the KV-streams trainer-mask oracle ("KV-streams", onedev.kr
summary, "how it works": the trainer reproduces the engine's eviction with an
attention mask so one forward pass sees what each token saw when generated).

The closed form visible(q, k) = k <= q < d_k is checked against a brute-force
replay of the engine (a Python list filtered by each keep mask), against the
oracle's own cache eviction (leyline_oracle.evict, whose rows carry token ids),
and against special cases with known masks: no event is the causal mask, a
drop-everything event leaves only the newer tokens, a sliding window is a band.
Tile classification is checked on those closed forms, bit packing against
numpy's packbits."""

import numpy as np
import pytest

from oracle import kvs_mask_oracle as K
from oracle import leyline_oracle as O
from synth import EvictionEvent, compaction_log, np_rng


@pytest.mark.parametrize("strategy", ["window", "half", "pick"])
def test_death_times_match_the_replay(strategy):
    for seed in range(6):
        n = int(np_rng(seed, 1).integers(40, 400))
        log = compaction_log(np_rng(seed, 2), n, strategy, budget=60, turn_lo=3, turn_hi=20, every_turns=3)
        assert log, "the workload must evict"
        d = K.death_times(n, n, log)
        assert np.array_equal(K.visibility(d), K.replay_visibility(n, log))


def test_death_times_match_the_engine_eviction():
    """Drive the oracle's paged cache (rows hold their token id) through the same
    events: after each event the cache's rows are exactly the tokens whose death
    time lies beyond that event."""
    n = 300
    log = compaction_log(np_rng(3, 4), n, "pick", budget=80, turn_lo=4, turn_hi=25, every_turns=2)
    d = K.death_times(n, n, log)
    P = 4
    st = O.CacheState.empty(1, 200, P, 100)
    st.set_pages(0, [], 0)
    t_prev = 0
    for e in log:
        st = _append(st, 0, list(range(t_prev, e.time)))   # tokens generated since the last event
        held = st.lengths[0]
        rows = st.logical_rows(0, 0)[:, 0].astype(np.int64)
        assert len(e.keep) == held
        st, _ = O.evict(st, [0], [e.keep])
        alive = st.logical_rows(0, 0)[:, 0].astype(np.int64) if st.lengths[0] else np.zeros(0, np.int64)
        assert np.array_equal(alive, rows[e.keep == 1])
        assert np.array_equal(np.sort(alive), np.flatnonzero(d[:e.time] > e.time))
        t_prev = e.time


def _append(st, seq, tokens):
    """Append rows carrying the given token ids to a sequence (grows its table
    with the lowest free pages)."""
    P = st.page_size
    n = st.lengths[seq]
    new = st.copy()
    table = list(new.tables[seq])
    free = sorted(new.free)
    for i, tok in enumerate(tokens):
        j = n + i
        if j // P >= len(table):
            pg = free.pop(0)
            new.free.discard(pg)
            table.append(pg)
        new.layers[0][table[j // P], j % P, 0] = tok
    new.tables[seq] = table
    new.lengths[seq] = n + len(tokens)
    return new


def test_no_event_is_the_causal_mask():
    d = K.death_times(50, 50, [])
    assert np.array_equal(K.visibility(d), np.tril(np.ones((50, 50), bool)))


def test_drop_everything_leaves_only_newer_tokens():
    d = K.death_times(30, 30, [EvictionEvent(12, np.zeros(12, np.uint8))])
    v = K.visibility(d)
    assert np.array_equal(v[:12], np.tril(np.ones((30, 30), bool))[:12])
    for q in range(12, 30):
        assert np.array_equal(np.flatnonzero(v[q]), np.arange(12, q + 1))


def test_sliding_window_is_a_band():
    """Every S tokens, evict everything older than the newest W tokens: query q
    then sees keys [max(0, t - W), q], t the last event time <= q."""
    T, S, W = 200, 10, 25
    held, log = [], []
    for t in range(S, T, S):
        held += list(range(log[-1].time if log else 0, t))
        keep = np.array([1 if k >= t - W else 0 for k in held], np.uint8)
        log.append(EvictionEvent(t, keep))
        held = [k for k, kp in zip(held, keep) if kp]
    v = K.visibility(K.death_times(T, T, log))
    for q in range(T):
        last = max([e.time for e in log if e.time <= q], default=None)
        lo = 0 if last is None else max(0, last - W)
        assert np.array_equal(np.flatnonzero(v[q]), np.arange(lo, q + 1)), q


def test_padding_keys_are_never_visible():
    d = K.death_times(64, 40, [EvictionEvent(20, np.r_[np.zeros(5, np.uint8), np.ones(15, np.uint8)])])
    v = K.visibility(d)
    assert not v[:, 40:].any()
    assert np.array_equal(v[:40, :40], K.replay_visibility(40, [EvictionEvent(20, np.r_[np.zeros(5, np.uint8),
                                                                                       np.ones(15, np.uint8)])]))


def test_bad_logs_are_rejected():
    with pytest.raises(K.InvalidLog):
        K.death_times(20, 20, [EvictionEvent(10, np.ones(9, np.uint8))])
    with pytest.raises(K.InvalidLog):
        K.death_times(20, 20, [EvictionEvent(10, np.ones(10, np.uint8)), EvictionEvent(10, np.ones(10, np.uint8))])
    with pytest.raises(K.InvalidLog):
        K.death_times(20, 20, [EvictionEvent(21, np.ones(21, np.uint8))])


def test_block_mask_of_the_causal_mask():
    """Causal, T = 256, tiles 32 x 64: query block i is full on key blocks
    fully below its first row and partial on the one(s) crossing the diagonal."""
    T, bq, bk = 256, 32, 64
    partial, full = K.block_mask(K.visibility(K.death_times(T, T, [])), bq, bk)
    for i in range(T // bq):
        q0, q1 = i * bq, (i + 1) * bq
        assert full[i] == [j for j in range(T // bk) if (j + 1) * bk - 1 <= q0]
        assert partial[i] == [j for j in range(T // bk) if j * bk <= q1 - 1 and not (j + 1) * bk - 1 <= q0]


def test_block_mask_of_drop_everything():
    """After an event at 128 that drops all of 0..127, query blocks from 128 on
    have no visible tile left of key block 2 (tiles 64 x 64)."""
    T = 256
    d = K.death_times(T, T, [EvictionEvent(128, np.zeros(128, np.uint8))])
    partial, full = K.block_mask(K.visibility(d), 64, 64)
    assert full[1] == [0] and partial[1] == [1]
    assert full[2] == [] and partial[2] == [2]
    assert full[3] == [2] and partial[3] == [3]


def test_dense_bits_match_packbits():
    rng = np_rng(1, 1)
    v = rng.random((37, 70)) < 0.5
    words = K.dense_bits(v)
    ref = np.packbits(np.pad(v, ((0, 0), (0, 26))), axis=1, bitorder="little").view("<u4")
    assert np.array_equal(words, ref)


def test_pins_catch_an_off_by_one_event_time(monkeypatch):
    """Planted: the event applied one token late (queries at t still see the
    dropped keys); the replay pin must fail."""
    real = K.death_times

    def planted(n_pad, n_tokens, events):
        d = real(n_pad, n_tokens, events)
        dropped = (d < n_pad) & (d > np.arange(n_pad))
        d[dropped] += 1
        return d

    monkeypatch.setattr(K, "death_times", planted)
    with pytest.raises(AssertionError):
        test_death_times_match_the_replay("pick")


def test_row_and_tile_restrictions_agree_with_the_whole_mask():
    n = 300
    log = compaction_log(np_rng(8, 1), n, "half", budget=90, turn_lo=5, turn_hi=30, every_turns=2)
    d = K.death_times(320, n, log)
    v = K.visibility(d)
    rows = [0, 17, 150, 299, 319]
    assert np.array_equal(K.visibility_rows(d, rows), v[rows])
    partial, full = K.block_mask(v, 32, 64)
    for i in range(10):
        for j in range(5):
            c = K.tile_class(d, 32 * i, min(32 * i + 32, 320), 64 * j, min(64 * j + 64, 320))
            assert c == ("full" if j in full[i] else "partial" if j in partial[i] else "empty")
