"""Random sequences of pool operations against the oracle, checked after every
operation: batched splices ("Leyline", sections 2.1-2.3; AMORTIZE and
FORGET; the page plan expanded on the device or staged by the host, picked at
random per call), evictions ("KV-streams", "how it works"; the device's page
plan, with page shortages that its verdict decides), page reuse on or off
for each splice and eviction (picked at random above page size 1),
page-granular reindex, per-row rotation in place ("VECTOR", method),
sequence alloc / set_pages / free, and requests that must fail and leave the
pool as it was.  Page sizes 1, 4 and 16; MLA pools and GQA pools.

Rows that become live without a splice or eviction writing them (a new
sequence, new pages) are filled with fresh seeded rows on both sides, as a
prefill would; every other row must stay identical to the oracle's."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import random_rows_np

from gpu_common import DevicePool, compare_seq, need_gpu, say, torch
from test_gpu_gqa import GqaDevicePool

pytestmark = pytest.mark.gpu

LAYERS, MAX_SEQS, MAX_LEN = 2, 5, 700


class Mirror:
    """An MLA pool and its oracle state."""
    pairing, base = "interleaved", 10000.0

    def __init__(self, P, seed):
        self.L = need_gpu()
        self.P = P
        # about 1600 rows: five sequences of up to 700 rows do not all fit, so
        # allocations and splices get refused and evictions now and then find
        # fewer free pages than they would need if every new page were fresh
        # (the device's verdict then decides)
        self.num_pages = {1: 1600, 4: 400, 16: 100}[P]
        self.max_pages = -(-MAX_LEN * 2 // P)
        self.dp = self.make_pool(seed)
        self.dp.snapshot_rows()
        self.rng = np.random.default_rng(seed)
        self.keep_alive = []
        self.live = set()
        self.seed = seed * 100000
        self.short_evictions = 0
        # splice planner per call: its own stream of draws, so the operations
        # themselves do not depend on it
        self.plan_rng = np.random.default_rng(seed + 1)
        self.splice_planned = {0: 0, 1: 0}
        # page reuse per splice / eviction (off for a quarter of the calls
        # above page size 1): a stream of draws of its own too
        self.reuse_rng = np.random.default_rng(seed + 2)
        self.reuse_off_calls = 0

    def reuse_for_call(self):
        reuse = self.P == 1 or self.reuse_rng.random() >= 0.25
        self.dp.pool.set_page_reuse(reuse)
        self.reuse_off_calls += not reuse
        return reuse

    @property
    def state(self):
        return self.dp.state

    @state.setter
    def state(self, st):
        self.dp.state = st

    def next_seed(self):
        self.seed += 1
        return self.seed

    # -- pool-kind specifics
    def make_pool(self, seed):
        return DevicePool(LAYERS, self.num_pages, self.P, MAX_SEQS, self.max_pages, seed=seed)

    def device_arrays(self):
        """(device tensor viewed [rows][width], index of its oracle array)."""
        return [(self.dp.data[l].view(-1, O.ROW), l) for l in range(LAYERS)]

    def stub(self, r):
        """(keyword arguments of the library's Directive, the oracle's stub)."""
        host = random_rows_np(self.next_seed(), (LAYERS, r, O.ROW))
        dev = torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16)
        self.keep_alive.append(dev)
        return {"stub": dev}, host

    def compare(self, seq, max_ulp):
        compare_seq(self.dp, self.state, seq, max_ulp=max_ulp)

    def prefill(self, seq, first=0):
        """Fresh rows in the sequence's live rows [first, n) on both sides."""
        n = self.state.lengths[seq]
        if n <= first:
            return
        t = np.asarray(self.state.tables[seq], np.int64)
        j = np.arange(first, n)
        phys = t[j // self.P] * self.P + j % self.P
        idx = torch.from_numpy(phys).cuda()
        for dev, a in self.device_arrays():
            rows = random_rows_np(self.next_seed(), (len(j), dev.shape[1]))
            dev[idx] = torch.from_numpy(rows.view(np.int16)).cuda().view(torch.bfloat16)
            self.state.layers[a].reshape(-1, dev.shape[1])[phys] = rows
        torch.cuda.synchronize()

    def check_books(self):
        for s in range(MAX_SEQS):
            if s in self.live:
                n, pos, pages = self.dp.pool.seq_get(s)
                assert n == self.state.lengths[s] and pos == self.state.next_pos[s], (s, n, pos)
                assert list(pages) == list(self.state.tables[s]), s
                assert np.array_equal(self.dp.table[s, :len(pages)].cpu().numpy(), pages), s
            else:
                with pytest.raises(self.L.LeylineError):
                    self.dp.pool.seq_get(s)
        assert self.dp.pool.free_pages() == len(self.state.free)

    def check_rows(self):
        for s in sorted(self.live):
            self.compare(s, 0)

    # -- operations
    def op_alloc(self):
        free_ids = [s for s in range(MAX_SEQS) if s not in self.live]
        if not free_ids:
            return "alloc: no id"
        n = int(self.rng.integers(0, MAX_LEN))
        need = -(-n // self.P)
        if need > len(self.state.free):
            with pytest.raises(self.L.LeylineError):
                self.dp.pool.seq_alloc(n)
            return "alloc: refused"
        sid = self.dp.pool.seq_alloc(n)
        assert sid == free_ids[0]
        self.state.set_pages(sid, sorted(self.state.free)[:need], n)
        self.live.add(sid)
        self.prefill(sid)
        return f"alloc {sid} n={n}"

    def op_free(self):
        if not self.live:
            return "free: none"
        s = int(self.rng.choice(sorted(self.live)))
        self.dp.pool.seq_free(s)
        self.state.free |= set(self.state.tables.pop(s))
        del self.state.lengths[s], self.state.next_pos[s]
        self.live.discard(s)
        return f"free {s}"

    def op_set_pages(self):
        if not self.live:
            return "set_pages: none"
        s = int(self.rng.choice(sorted(self.live)))
        n_old = self.state.lengths[s]
        n = int(self.rng.integers(0, MAX_LEN))
        need = -(-n // self.P)
        own = list(self.state.tables[s])
        pool = own + sorted(self.state.free)
        if need > len(pool):
            return "set_pages: no room"
        pages = [int(x) for x in self.rng.permutation(pool)[:need]]
        self.dp.set_pages(s, pages, n)
        self.prefill(s)
        return f"set_pages {s} n={n_old}->{n}"

    def op_splice(self):
        if not self.live:
            return "splice: none"
        k = int(self.rng.integers(1, min(3, len(self.live)) + 1))
        seqs = [int(x) for x in self.rng.choice(sorted(self.live), size=k, replace=False)]
        lib, ora = [], []
        for s in seqs:
            n = self.state.lengths[s]
            s0 = int(self.rng.integers(0, n + 1))
            s1 = int(self.rng.integers(s0, n + 1))
            mode = O.FORGET if self.rng.random() < 0.15 else O.AMORTIZE
            r = int(self.rng.integers(0, 2 * self.P + 4)) if mode == O.AMORTIZE else 0
            kw, host = self.stub(r) if r else ({}, None)
            lib.append(self.L.Directive(s, s0, s1, mode=mode, **kw))
            ora.append(O.Directive(s, s0, s1, r, host, mode))
        reuse = self.reuse_for_call()
        try:
            expected, _ = O.splice(self.state, ora, pairing=self.pairing, base=self.base, reuse_pages=reuse)
        except O.OracleError:
            with pytest.raises(self.L.LeylineError):
                self.dp.pool.splice(lib)
            return "splice: refused"
        self.dp.pool.set_splice_planner(int(self.plan_rng.integers(0, 2)))
        self.dp.pool.splice(lib)
        self.splice_planned[self.dp.pool.last_stats().planned_on_device] += 1
        self.state = expected
        return f"splice {[(d.seq, d.s_start, d.s_end, d.r_len, d.mode) for d in ora]} reuse {reuse}"

    def op_evict(self):
        if not self.live:
            return "evict: none"
        k = int(self.rng.integers(1, min(3, len(self.live)) + 1))
        seqs = [int(x) for x in self.rng.choice(sorted(self.live), size=k, replace=False)]
        masks = []
        for s in seqs:
            n = self.state.lengths[s]
            kind = int(self.rng.integers(0, 4))
            if kind == 0:
                m = np.ones(n, np.uint8)
            elif kind == 1:
                m = np.zeros(n, np.uint8)
            elif kind == 2:
                m = (self.rng.random(n) < self.rng.random()).astype(np.uint8)
            else:   # runs
                m = np.repeat(self.rng.integers(0, 2, size=-(-n // 7)), 7)[:n].astype(np.uint8)
            masks.append(m)
        keep = np.concatenate(masks) if masks else np.zeros(0, np.uint8)
        offsets = np.concatenate([[0], np.cumsum([len(m) for m in masks])[:-1]]).astype(np.int64)
        dev = torch.from_numpy(keep).cuda() if len(keep) else torch.zeros(16, dtype=torch.uint8, device="cuda")
        self.keep_alive.append(dev)
        if self.P > 1 and len(self.state.free) < sum(len(self.state.tables[s]) for s in seqs):
            self.short_evictions += 1   # a shortage was possible: the verdict decided
        reuse = self.reuse_for_call()
        try:
            expected, _ = O.evict(self.state, seqs, masks, reuse_pages=reuse)
        except O.OracleError:
            with pytest.raises(self.L.LeylineError):
                self.dp.pool.evict(seqs, dev, offsets)
            return "evict: refused"
        self.dp.pool.evict(seqs, dev, offsets)
        self.state = expected
        return f"evict {seqs} reuse {reuse}"

    def op_reindex(self):
        cand = [s for s in sorted(self.live) if self.state.lengths[s] > 0]
        if not cand:
            return "reindex: none"
        s = int(self.rng.choice(cand))
        n = self.state.lengths[s]
        n_pages = -(-n // self.P)
        keep = sorted(int(x) for x in np.flatnonzero(self.rng.random(n_pages) < 0.6))
        if n % self.P and n_pages - 1 in keep and keep[-1] != n_pages - 1:
            keep.remove(n_pages - 1)
        self.dp.pool.ptable_reindex(s, keep)
        self.state = O.ptable_reindex(self.state, s, keep)
        return f"reindex {s} keep {len(keep)}/{n_pages}"

    def pressure(self):
        """A full pool: an allocation and a splice that need more pages than
        are free are refused with nothing changed; an eviction whose worst
        case exceeds the free pages succeeds after reading the verdict."""
        self.dp.pool.set_page_reuse(True)
        for s in sorted(self.live):
            self.dp.pool.seq_free(s)
            self.state.free |= set(self.state.tables.pop(s))
            del self.state.lengths[s], self.state.next_pos[s]
        self.live.clear()
        cap_rows = self.num_pages * self.P
        big = min(MAX_LEN, cap_rows // 2 - 5 * self.P)
        for _ in range(2):
            sid = self.dp.pool.seq_alloc(big)
            self.state.set_pages(sid, sorted(self.state.free)[:-(-big // self.P)], big)
            self.live.add(sid)
            self.prefill(sid)
        rest = len(self.state.free) * self.P
        with pytest.raises(self.L.LeylineError):
            self.dp.pool.seq_alloc(rest + self.P)          # one page short
        self.check_books()
        if self.P > 1:
            # insertion at row 1 of a stub that is not a whole number of
            # pages: every page from the first on is fresh
            r = self.P + 1
            kw, host = self.stub(r)
            with pytest.raises(O.OutOfPages):
                O.splice(self.state, [O.Directive(0, 1, 1, r, host)], pairing=self.pairing, base=self.base)
            with pytest.raises(self.L.LeylineError):
                self.dp.pool.splice([self.L.Directive(0, 1, 1, **kw)])
            self.check_books()
            self.check_rows()
            assert len(self.state.free) < sum(len(self.state.tables[s]) for s in (0, 1))
            self.short_evictions += 1
        # whole pages kept or dropped (every new page a reuse), and one row
        # dropped 3 pages before the end (a few fresh pages)
        m0 = np.repeat(self.rng.integers(0, 2, size=-(-big // self.P)), self.P)[:big].astype(np.uint8)
        m1 = np.ones(big, np.uint8)
        m1[max(0, big - 3 * self.P)] = 0
        masks = [m0, m1]
        self.state, _ = O.evict(self.state, [0, 1], masks)
        keep = torch.from_numpy(np.concatenate(masks)).cuda()
        self.dp.pool.evict([0, 1], keep, np.array([0, big], np.int64))
        torch.cuda.synchronize()
        self.check_books()
        self.check_rows()

    def op_rope(self):
        cand = [s for s in sorted(self.live) if self.state.lengths[s] > 0]
        if not cand:
            return "rope: none"
        s = int(self.rng.choice(cand))
        n = self.state.lengths[s]
        r0 = int(self.rng.integers(0, n))
        cnt = int(self.rng.integers(1, n - r0 + 1))
        angles = self.rng.integers(-100000, 100000, size=cnt).astype(np.int64)
        a = torch.from_numpy(angles).cuda()
        self.keep_alive.append(a)
        self.dp.pool.rope_rows(s, r0, a)
        self.state = O.rope_rows(self.state, s, r0, angles, pairing=self.pairing, base=self.base, in_place=True)
        torch.cuda.synchronize()
        # bands within 1 ulp (device and host float64 sincos may differ at a
        # rounding tie); then the oracle takes the device's rows so that later
        # operations start from identical bits
        self.compare(s, 1)
        self.dp.snapshot_rows()
        return f"rope {s} [{r0}, {r0 + cnt})"


class GqaMirror(Mirror):
    """A GQA pool (3 KV heads x 64, RoPE on the first 32 values of each head,
    half-split pairs, base 500000) and its oracle state (K and V arrays per
    layer)."""
    H, D, ROT = 3, 64, 32
    pairing, base = "half", 500000.0

    def make_pool(self, seed):
        return GqaDevicePool(LAYERS, self.num_pages, self.P, MAX_SEQS, self.max_pages, self.H, self.D, self.ROT,
                             seed=seed, pairing=1, base=self.base)

    def device_arrays(self):
        out = []
        for l in range(LAYERS):
            out += [(self.dp.k[l].view(-1, self.H * self.D), 2 * l), (self.dp.v[l].view(-1, self.H * self.D), 2 * l + 1)]
        return out

    def stub(self, r):
        k, v, host = self.dp.stub(self.next_seed(), r)
        self.keep_alive += [k, v]
        return {"stub": k, "stub_v": v}, host

    def compare(self, seq, max_ulp):
        assert self.dp.compare(self.state, seq) <= max_ulp


@pytest.mark.parametrize("kind", ["mla", "gqa"])
@pytest.mark.parametrize("P", [1, 4, 16])
def test_random_operation_sequences(P, kind):
    say(f"random operations, {kind}, P={P}")
    m = (Mirror if kind == "mla" else GqaMirror)(P, seed=700 + P + (50 if kind == "gqa" else 0))
    for _ in range(3):
        m.op_alloc()
    ops = [m.op_splice] * 5 + [m.op_evict] * 4 + [m.op_reindex, m.op_rope, m.op_alloc, m.op_free, m.op_set_pages]
    log = []
    for step in range(240):
        op = ops[int(m.rng.integers(0, len(ops)))]
        log.append(op())
        torch.cuda.synchronize()
        try:
            m.check_books()
            if step % 8 == 7:
                m.check_rows()
        except AssertionError:
            say("  last operations: " + " | ".join(log[-6:]))
            raise
    m.check_rows()
    refused = sum(1 for x in log if "refused" in x)
    kinds = {}
    for x in log:
        kinds[x.split(" ")[0].rstrip(":")] = kinds.get(x.split(" ")[0].rstrip(":"), 0) + 1
    say(f"  {len(log)} operations {kinds}; {refused} refused as the oracle refused them; "
        f"{m.short_evictions} evictions short of their all-fresh need; splices planned on the device "
        f"{m.splice_planned[1]}, staged {m.splice_planned[0]}; page reuse off for {m.reuse_off_calls} calls")
    assert m.splice_planned[0] and m.splice_planned[1]
    assert P == 1 or m.reuse_off_calls > 0
    m.pressure()
    m.keep_alive.clear()
    m.dp.close()
