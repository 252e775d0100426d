"""GPU parity of the splice and the eviction on GQA / MHA pools (Leyline
summary, section 5: the directive carries over to GQA/MHA caches, only the
rotation step changes) against the CPU oracle, through the C ABI.

Per checked layer: V rows and the non-rotary K values bit-exact, every K
head's RoPE band within 1 bf16 ulp (0 expected: the kernel follows the
oracle's float32 order), page tables, lengths and positions bit-exact."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import draw_span, np_rng, permuted_pages, random_rows_np, random_rows_torch, turn_drop_mask

from gpu_common import need_gpu, say, torch, ulp_distance

pytestmark = pytest.mark.gpu


class GqaDevicePool:
    """A GQA pool on cuda:0 and its host mirror for the oracle (K and V arrays
    of the checked layers, in that order per layer)."""

    def __init__(self, L, num_pages, P, max_seqs, max_pages, H, D, rot, seed=0, pairing=0, base=10000.0,
                 host_rows=True, oracle_layers=None):
        leyline = need_gpu()
        self.L, self.P, self.H, self.D, self.rot = L, P, H, D, rot
        self.pairing = "half" if pairing else "interleaved"
        self.base = base
        shape = (L, num_pages, P, H, D)
        if host_rows:
            self.k = torch.from_numpy(random_rows_np(seed, shape).view(np.int16)).view(torch.bfloat16).to("cuda")
            self.v = torch.from_numpy(random_rows_np(seed + 1, shape).view(np.int16)).view(torch.bfloat16).to("cuda")
        else:
            self.k = random_rows_torch(seed, shape, "cuda")
            self.v = random_rows_torch(seed + 1, shape, "cuda")
        self.table = torch.full((max_seqs, max_pages), -1, dtype=torch.int32, device="cuda")
        self.pool = leyline.GqaPool(self.k, self.v, self.table, rotary_dim=rot, rope_base=base, pairing=pairing)
        self.oracle_layers = list(range(L)) if oracle_layers is None else list(oracle_layers)
        specs = []
        for _ in self.oracle_layers:
            specs += [O.gqa_k_row(H, D, rot), O.plain_row(H * D)]
        self.state = O.CacheState.empty(len(specs), num_pages, P, max_pages, with_rows=False, specs=specs)

    def _host(self, t):
        return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(t.shape[0], t.shape[1], -1).copy()

    def snapshot_rows(self):
        self.state.layers = []
        for l in self.oracle_layers:
            self.state.layers += [self._host(self.k[l]), self._host(self.v[l])]

    def set_pages(self, seq, pages, n):
        self.pool.seq_set_pages(seq, pages, n)
        self.state.set_pages(seq, pages, n)

    def stub(self, seed, r):
        """(K stub, V stub) on the device [L][r][H][D] and the oracle's list of
        per-array host rows."""
        if r == 0:
            return None, None, None
        k = random_rows_np(seed, (self.L, r, self.H, self.D))
        v = random_rows_np(seed + 7, (self.L, r, self.H, self.D))
        host = []
        for l in self.oracle_layers:
            host += [k[l].reshape(r, -1), v[l].reshape(r, -1)]
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
        return to_dev(k), to_dev(v), host

    def splice(self, directives):
        """directives: (seq, s0, s1, r, seed, mode); oracle then library."""
        L = need_gpu()
        lib, ora = [], []
        for seq, s0, s1, r, seed, mode in directives:
            rr = r if mode == O.AMORTIZE else 0
            k, v, host = self.stub(seed, rr)
            lib.append(L.Directive(seq, s0, s1, k, mode, stub_v=v))
            ora.append(O.Directive(seq, s0, s1, rr, host, mode))
        expected, plans = O.splice(self.state, ora, pairing=self.pairing, base=self.base)
        self.pool.splice(lib)
        torch.cuda.synchronize()
        return expected, plans

    def compare(self, expected, seq):
        """Returns the largest RoPE-band ulp distance seen."""
        n, pos, pages = self.pool.seq_get(seq)
        assert n == expected.lengths[seq] and pos == expected.next_pos[seq]
        assert list(pages) == list(expected.tables[seq])
        assert np.array_equal(self.table[seq, :len(pages)].cpu().numpy(), pages)
        if n == 0:
            return 0
        P, H, D, rot = self.P, self.H, self.D, self.rot
        j = np.arange(n)
        phys = torch.from_numpy(pages.astype(np.int64)[j // P] * P + j % P).to("cuda")
        worst = 0
        for li, l in enumerate(self.oracle_layers):
            gk = self.k[l].reshape(-1, H * D)[phys].view(torch.int16).cpu().numpy().view(np.uint16)
            gv = self.v[l].reshape(-1, H * D)[phys].view(torch.int16).cpu().numpy().view(np.uint16)
            ek = expected.logical_rows(seq, 2 * li)
            ev = expected.logical_rows(seq, 2 * li + 1)
            assert np.array_equal(gv, ev), f"V differs (layer {l})"
            gk, ek = gk.reshape(n, H, D), ek.reshape(n, H, D)
            assert np.array_equal(gk[..., rot:], ek[..., rot:]), f"non-rotary K differs (layer {l})"
            d = int(ulp_distance(gk[..., :rot], ek[..., :rot]).max())
            worst = max(worst, d)
            assert worst <= 1, f"K band differs by {worst} ulp (layer {l})"
        return worst

    def close(self):
        self.pool.close()
        del self.k, self.v, self.table
        torch.cuda.empty_cache()


SHAPES = [  # (H, D, rotary_dim, pairing)
    (2, 64, 64, 0),
    (2, 128, 128, 1),
    (4, 128, 64, 1),     # partial rotary, half-split inside the band
    (1, 32, 16, 0),      # rows of 4 chunks: tasks not wave-aligned at small pages
    (3, 64, 32, 1),      # odd head count
]


@pytest.mark.parametrize("P", [1, 4, 16])
@pytest.mark.parametrize("H,D,rot,pairing", SHAPES)
def test_gqa_splice_tiny_sweep(P, H, D, rot, pairing):
    say(f"gqa tiny sweep P={P} H={H} D={D} rot={rot} pairing={pairing}")
    rng = np_rng(P * 100 + H * 10 + rot, 3)
    worst = 0
    for case in range(10):
        n = int(rng.integers(1, 5 * P + 7))
        s0 = int(rng.integers(0, n + 1))
        s1 = int(rng.integers(s0, n + 1))
        r = int(rng.choice([0, 1, P + 3]))
        pages = -(-n // P)
        num_pages = 3 * pages + 3 * (-(-(P + 3) // P)) + 8
        dp = GqaDevicePool(2, num_pages, P, 2, num_pages, H, D, rot, seed=case, pairing=pairing)
        dp.set_pages(1, permuted_pages(case, num_pages)[:pages], n)
        dp.snapshot_rows()
        expected, _ = dp.splice([(1, s0, s1, r, 100 + case, O.AMORTIZE)])
        worst = max(worst, dp.compare(expected, 1))
        assert dp.pool.free_pages() == len(expected.free)
        dp.close()
    say(f"  max band ulp = {worst}")


def test_gqa_batched_splice_with_forget_mha():
    """MHA-like rows (16 heads of 64, RoPE on the first 32 of each), three
    sequences in one call: a shrinking splice, a growing one, a FORGET."""
    say("gqa batched MHA P=16")
    P, H, D, rot = 16, 16, 64, 32
    dp = GqaDevicePool(2, 1200, P, 3, 400, H, D, rot, seed=4, pairing=1)
    lens = [2000, 1500, 900]
    perm = permuted_pages(4, 1200)
    at = 0
    for s, n in enumerate(lens):
        k = -(-n // P)
        dp.set_pages(s, perm[at:at + k], n)
        at += k
    dp.snapshot_rows()
    expected, _ = dp.splice([(0, 300, 1700, 40, 1, O.AMORTIZE), (1, 100, 120, 77, 2, O.AMORTIZE),
                             (2, 500, 600, 0, 3, O.FORGET)])
    worst = max(dp.compare(expected, s) for s in range(3))
    assert dp.pool.free_pages() == len(expected.free)
    st = dp.pool.last_stats()
    moved = st.rows_moved
    layers = 2
    assert st.alg_bytes == 2 * layers * 2 * (H * D * 2) * moved + layers * 2 * (H * rot * 2) * st.rows_rotated_inplace
    say(f"  max band ulp = {worst}, rows moved {moved}, rotated in place {st.rows_rotated_inplace}")
    dp.close()


@pytest.mark.slow
def test_gqa_llama8b_shape_32k_splice():
    """Llama-3-8B-shaped cache: 32 layers, 8 KV heads of 128, RoPE on all 128
    (half-split, base 500000), page size 16, one 32768-token sequence on
    permuted pages; splice [8192, 14336) for 24 stub rows (Delta = -6120).
    Layers 0, 13 and 31 are compared in full."""
    say("gqa llama8b 32k splice")
    P, H, D, rot, L = 16, 8, 128, 128, 32
    tokens, pool_pages = 32768, 4096
    dp = GqaDevicePool(L, pool_pages, P, 1, pool_pages, H, D, rot, seed=21, pairing=1, base=500000.0,
                       host_rows=False, oracle_layers=[0, 13, 31])
    dp.set_pages(0, permuted_pages(21, pool_pages)[:tokens // P], tokens)
    dp.snapshot_rows()
    expected, _ = dp.splice([(0, 8192, 14336, 24, 5, O.AMORTIZE)])
    worst = dp.compare(expected, 0)
    st = dp.pool.last_stats()
    row = H * D * 2
    assert st.alg_bytes == L * 2 * 2 * row * st.rows_moved + L * 2 * H * rot * 2 * st.rows_rotated_inplace
    say(f"  max band ulp = {worst}; moved {st.rows_moved} rows, {st.alg_bytes / 1e9:.3f} GB")
    dp.close()


@pytest.mark.parametrize("P,plan", [(16, "device"), (16, "host"), (1, "device")])
def test_gqa_evict_turn_drops(P, plan):
    """KV-streams eviction on a GQA pool: two sequences of 4096 tokens, random
    turn drops; K and V rows move unchanged.  The device makes the page plan,
    with free pages for every page of both sequences or with fewer (a
    shortage is then possible and the call reads the device's verdict before
    the rows move)."""
    say(f"gqa evict P={P}, {plan} plan")
    L_ = need_gpu()
    H, D, rot = 8, 64, 64
    n = 4096
    pages = n // P
    extra = 2 * pages + 16 if plan == "device" else pages
    dp = GqaDevicePool(2, 2 * pages + extra, P, 2, pages, H, D, rot, seed=8 + P)
    perm = permuted_pages(8, 2 * pages + extra)
    dp.set_pages(0, perm[:pages], n)
    dp.set_pages(1, perm[pages:2 * pages], n)
    dp.snapshot_rows()
    rng = np_rng(8, P)
    masks = [turn_drop_mask(rng, n, 50, 400), turn_drop_mask(rng, n, 50, 400)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    expected, _ = O.evict(dp.state, [0, 1], masks)
    dp.pool.evict([0, 1], keep, [0, n])
    torch.cuda.synchronize()
    for s in range(2):
        assert dp.compare(expected, s) == 0
    assert dp.pool.free_pages() == len(expected.free)
    st = dp.pool.last_stats()
    assert st.alg_bytes == 2 * 2 * 2 * H * D * 2 * st.rows_moved
    dp.close()
    del L_


@pytest.mark.slow
def test_gqa_evict_llama8b_shape_32_rollouts():
    """The GQA eviction workload as it is timed: 32 rollouts x 16384 tokens x
    32 layers of K and V planes (8 KV heads x 128), page size 16, pool pages
    1.5 x the rollouts', random turn drops (the same seeds), one call.  Page
    tables of all 32 rollouts and the free count against the oracle; K and V
    rows of 8 rollouts on layers 0 and 31 equal the kept rows captured before
    the call."""
    need_gpu()
    layers, H, D, P, n_roll, n_tok = 32, 8, 128, 16, 32, 16384
    per = n_tok // P
    say(f"gqa evict {n_roll} x {n_tok} x {layers} (K and V, {H} x {D}), P={P}")
    dp = GqaDevicePool(layers, n_roll * per * 3 // 2, P, n_roll, per, H, D, D, seed=0, pairing=1, base=500000.0,
                       host_rows=False, oracle_layers=[])
    perm = permuted_pages(0, n_roll * per)
    for s in range(n_roll):
        dp.set_pages(s, perm[s * per:(s + 1) * per], n_tok)
    rng = np_rng(0, 7)
    masks = [turn_drop_mask(rng, n_tok) for _ in range(n_roll)]
    check = list(range(0, n_roll, 4))
    j = np.arange(n_tok)
    before = {}
    for s in check:
        phys = torch.from_numpy(np.asarray(dp.state.tables[s], np.int64)[j // P] * P + j % P).to("cuda")
        before[s] = [t[l].reshape(-1, H * D)[phys].view(torch.int16).cpu().numpy()
                     for l in (0, layers - 1) for t in (dp.k, dp.v)]
    keep = torch.from_numpy(np.concatenate(masks)).to("cuda")
    expected, _ = O.evict(dp.state, list(range(n_roll)), masks)
    dp.pool.evict(list(range(n_roll)), keep, np.arange(n_roll, dtype=np.int64) * n_tok)
    torch.cuda.synchronize()
    for s in range(n_roll):
        n, pos, pages = dp.pool.seq_get(s)
        assert n == expected.lengths[s] and pos == expected.next_pos[s]
        assert list(pages) == list(expected.tables[s])
        assert np.array_equal(dp.table[s, :len(pages)].cpu().numpy(), pages)
    assert dp.pool.free_pages() == len(expected.free)
    for s in check:
        n, _, pages = dp.pool.seq_get(s)
        jj = np.arange(n)
        phys = torch.from_numpy(pages.astype(np.int64)[jj // P] * P + jj % P).to("cuda")
        kept = np.flatnonzero(masks[s])
        got = [t[l].reshape(-1, H * D)[phys].view(torch.int16).cpu().numpy()
               for l in (0, layers - 1) for t in (dp.k, dp.v)]
        for a, b in zip(got, before[s]):
            assert np.array_equal(a, b[kept]), s
    dp.close()


def test_gqa_evict_then_splice():
    """An eviction followed by a splice on the same GQA sequence."""
    say("gqa evict then splice")
    P, H, D, rot = 16, 4, 128, 128
    n = 3000
    pages = -(-n // P)
    dp = GqaDevicePool(2, 4 * pages, P, 1, 2 * pages, H, D, rot, seed=30, pairing=1)
    dp.set_pages(0, permuted_pages(30, 4 * pages)[:pages], n)
    dp.snapshot_rows()
    mask = turn_drop_mask(np_rng(30, 1), n, 100, 600)
    expected, _ = O.evict(dp.state, [0], [mask])
    dp.pool.evict([0], torch.from_numpy(mask).to("cuda"), [0])
    torch.cuda.synchronize()
    dp.compare(expected, 0)
    dp.state = expected
    m = expected.lengths[0]
    d = draw_span(np_rng(30, 2), m, 16, max(17, m // 3), 1, 40, start_lo=0)
    expected, _ = dp.splice([(0, d.s_start, d.s_end, d.r_len, 31, O.AMORTIZE)])
    assert dp.compare(expected, 0) == 0
    dp.close()


def test_gqa_directive_errors():
    L = need_gpu()
    P, H, D = 16, 2, 64
    dp = GqaDevicePool(1, 64, P, 1, 64, H, D, 64, seed=2)
    dp.set_pages(0, np.arange(4), 64)
    k, v, _ = dp.stub(3, 5)
    with pytest.raises(ValueError):
        dp.pool.splice([L.Directive(0, 10, 20, k, stub_v=None)])
    # through the C ABI directly: K rows without V rows
    arr = (L._Directive * 1)()
    arr[0] = L._Directive(0, L.AMORTIZE, 10, 20, 5, k.data_ptr(), 0, None, 0)
    assert L._lib.leyline_splice(dp.pool._h, arr, 1, None) == L.LL_EINVAL
    arr[0] = L._Directive(0, L.AMORTIZE, 10, 20, 5, k.data_ptr(), 0, v.data_ptr() + 8, 0)
    assert L._lib.leyline_splice(dp.pool._h, arr, 1, None) == L.LL_EINVAL
    n, pos, pages = dp.pool.seq_get(0)
    assert n == 64 and list(pages) == [0, 1, 2, 3]
    dp.close()
    # an MLA pool refuses V rows
    data = torch.zeros((1, 8, P, O.ROW), dtype=torch.bfloat16, device="cuda")
    table = torch.full((1, 8), -1, dtype=torch.int32, device="cuda")
    pool = L.Pool(data, table)
    pool.seq_set_pages(0, [0, 1], 32)
    stub = torch.zeros((1, 2, O.ROW), dtype=torch.bfloat16, device="cuda")
    arr[0] = L._Directive(0, L.AMORTIZE, 4, 8, 2, stub.data_ptr(), 0, stub.data_ptr(), 0)
    assert L._lib.leyline_splice(pool._h, arr, 1, None) == L.LL_EINVAL
    pool.close()
