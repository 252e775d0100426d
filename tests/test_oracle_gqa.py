"""Pins for the oracle's GQA/MHA rows (Leyline summary, section 5: the directive
carries over to GQA/MHA caches, only the rotation step changes).  A GQA cache
has, per layer, a K array whose rows hold H heads of D values with RoPE on the
first rotary_dim values of every head, and a V array with no RoPE.

The oracle's GQA splice is checked against: a brute-force list rebuild (V and
the non-rotary K values bit-exact); the exact rotation of every rotated head
written as a complex exponential, within one bf16 ulp; the MLA splice, which a
one-head K (D = 64) plus a 512-wide V must reproduce bit for bit; eviction as a
masked list; the byte count done by hand for a Llama-3-8B-shaped layer."""

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, random_rows_np, turn_drop_mask


def _gqa_state(P, n, num_pages, H, D, rot, layers=1, seed=0):
    specs = []
    for _ in range(layers):
        specs += [O.gqa_k_row(H, D, rot), O.plain_row(H * D)]
    st = O.CacheState.empty(len(specs), num_pages, P, num_pages, specs=specs)
    for a, sp in enumerate(specs):
        st.layers[a][:] = random_rows_np(seed * 100 + a, (num_pages, P, sp.width))
    k = -(-n // P)
    st.set_pages(0, permuted_pages(seed, num_pages)[:k], n)
    return st, specs


def _exact_band(bits, delta, rot, pairing, base=10000.0):
    """The band turned by delta, in float64: pair j is the complex number
    x + iy times exp(i delta theta_j), theta_j = base^(-2j/rot)."""
    x = O.bf16_to_f32(bits).astype(np.float64)
    half = rot // 2
    j = np.arange(half)
    ix, iy = (2 * j, 2 * j + 1) if pairing == "interleaved" else (j, j + half)
    th = base ** (-2.0 * j / rot)
    z = (x[..., ix] + 1j * x[..., iy]) * np.exp(1j * delta * th)
    out = np.empty_like(x)
    out[..., ix], out[..., iy] = z.real, z.imag
    return out


def _bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (float64)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("H,D,rot,pairing", [(2, 128, 128, "interleaved"), (2, 128, 128, "half"),
                                             (3, 64, 32, "interleaved"), (1, 128, 64, "half"),
                                             (4, 32, 16, "interleaved")])
def test_gqa_splice_matches_list_rebuild(H, D, rot, pairing):
    rng = np.random.default_rng(H * 1000 + D + rot)
    P = 4
    for case in range(12):
        n = int(rng.integers(1, 40))
        s0 = int(rng.integers(0, n + 1))
        s1 = int(rng.integers(s0, n + 1))
        r = int(rng.integers(0, 9))
        st, specs = _gqa_state(P, n, 64, H, D, rot, seed=case)
        stub = [random_rows_np(500 + 10 * case + a, (r, sp.width)) for a, sp in enumerate(specs)] if r else None
        new, _ = O.splice(st, [O.Directive(0, s0, s1, r, stub)], pairing=pairing)
        delta = r - (s1 - s0)
        assert new.lengths[0] == n + delta and new.next_pos[0] == st.next_pos[0] + delta
        for a in range(2):
            old = list(st.logical_rows(0, a))
            rebuilt = np.array(old[:s0] + [stub[a][k] for k in range(r)] + old[s1:], np.uint16)
            got = new.logical_rows(0, a)
            if a == 1:
                assert np.array_equal(got, rebuilt.reshape(got.shape))          # V untouched
                continue
            g = got.reshape(-1, H, D)
            e = rebuilt.reshape(-1, H, D)
            assert np.array_equal(g[..., rot:], e[..., rot:])                   # non-rotary K dims
            assert np.array_equal(g[:s0 + r, :, :rot], e[:s0 + r, :, :rot])     # prefix and stub
            down = e[s0 + r:, :, :rot]
            if delta == 0 or len(down) == 0:
                assert np.array_equal(g[s0 + r:, :, :rot], down)
                continue
            exact = _exact_band(down, delta, rot, pairing)
            err = np.abs(O.bf16_to_f32(g[s0 + r:, :, :rot]).astype(np.float64) - exact)
            assert np.all(err <= _bf16_ulp(exact) + 1e-30), (case, np.max(err / _bf16_ulp(exact)))


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_one_head_gqa_reproduces_mla(pairing):
    """K = one 64-wide head, all rotary, V = 512 wide: the GQA splice is the MLA
    splice with c_kv in V and k_pe in K."""
    P, n, pages = 16, 300, 64
    mla = O.CacheState.empty(2, pages, P, pages)
    for L in range(2):
        mla.layers[L][:] = random_rows_np(L, (pages, P, O.ROW))
    T = permuted_pages(1, pages)[:-(-n // P)]
    mla.set_pages(0, T, n)
    specs = [O.gqa_k_row(1, 64, 64), O.plain_row(512)] * 2
    gqa = O.CacheState.empty(4, pages, P, pages, specs=specs)
    for L in range(2):
        gqa.layers[2 * L][:] = mla.layers[L][..., 512:]
        gqa.layers[2 * L + 1][:] = mla.layers[L][..., :512]
    gqa.set_pages(0, T, n)
    stub = random_rows_np(9, (2, 7, O.ROW))
    gstub = [stub[0][:, 512:], stub[0][:, :512], stub[1][:, 512:], stub[1][:, :512]]
    a, pa = O.splice(mla, [O.Directive(0, 40, 210, 7, stub)], pairing=pairing)
    b, pb = O.splice(gqa, [O.Directive(0, 40, 210, 7, gstub)], pairing=pairing)
    assert pa == pb and a.tables == b.tables and a.lengths == b.lengths
    for L in range(2):
        assert np.array_equal(a.logical_rows(0, L)[:, 512:], b.logical_rows(0, 2 * L))
        assert np.array_equal(a.logical_rows(0, L)[:, :512], b.logical_rows(0, 2 * L + 1))


def test_gqa_evict_is_masked_list():
    P, n = 16, 500
    st, specs = _gqa_state(P, n, 64, 2, 64, 64, layers=2, seed=4)
    mask = turn_drop_mask(np_rng(4, 1), n, 20, 80)
    new, _ = O.evict(st, [0], [mask])
    keep = np.flatnonzero(mask)
    for a in range(len(specs)):
        assert np.array_equal(new.logical_rows(0, a), st.logical_rows(0, a)[keep])
    assert new.next_pos[0] == st.next_pos[0]


def test_gqa_rotated_head_keeps_attention_scores():
    """With rotary_dim 128 (a Llama-style head), a key stored at position i and
    turned by Delta scores against a query at m + Delta as it did at m, up to
    bf16 rounding of the stored key."""
    rng = np_rng(11, 0)
    D = 128
    q = rng.standard_normal((64, D))
    k = rng.standard_normal((64, D))
    i = rng.integers(1000, 5000, size=64)
    m = i + rng.integers(1, 4000, size=64)
    delta = -777
    stored = O.f32_to_bf16(O.rotate_f64(k, i, rope_dim=D).astype(np.float32))
    moved = O.rotate_kpe_bf16(stored, delta, rope_dim=D)
    before = np.sum(O.rotate_f64(q, m, rope_dim=D) * O.bf16_to_f32(stored), axis=-1)
    after = np.sum(O.rotate_f64(q, m + delta, rope_dim=D) * O.bf16_to_f32(moved), axis=-1)
    scale = np.linalg.norm(q, axis=-1) * np.linalg.norm(k, axis=-1)
    assert np.max(np.abs(after - before) / scale) < 1e-2


def test_gqa_algorithmic_bytes_by_hand():
    """Llama-3-8B-shaped layer (8 KV heads of 128, RoPE on all 128): a moved row
    reads and writes 2 KiB of K and 2 KiB of V; an in-place rotated row reads
    and writes its 2 KiB of K."""
    specs = [O.gqa_k_row(8, 128, 128), O.plain_row(1024)]
    n, P = 64, 16
    kind, index, down = O.splice_sources(n, 10, 20, 10)      # Delta = 0
    plan = [-1, 1, 2, 3]
    got = O.algorithmic_bytes(plan, n, P, kind, down, 0, 2, specs=specs)
    assert got == 16 * 2 * (2048 + 2048)
    kind, index, down = O.splice_sources(n, 10, 20, 6)       # Delta = -4
    plan = [-1, -1, 2, 3]                                     # only the tail reuses (it cannot)
    got = O.algorithmic_bytes(plan, 60, P, kind, down, -4, 2, specs=specs)
    n_down_reused = int(np.count_nonzero(down[32:]))
    assert got == 32 * 2 * 4096 + n_down_reused * 2 * 2048


def test_pins_catch_theta_over_the_wrong_width(monkeypatch):
    """Planted: the band's theta computed over the MLA width (64) instead of the
    band's own width; the list-rebuild pin must fail."""
    real = O.rotate_kpe_bf16

    def planted(bits, delta, rope_dim=64, base=10000.0, pairing="interleaved"):
        if rope_dim == 128:   # the MLA routine applied to each 64-wide half
            return np.concatenate([real(bits[..., :64], delta, 64, base, pairing),
                                   real(bits[..., 64:], delta, 64, base, pairing)], axis=-1)
        return real(bits, delta, rope_dim, base, pairing)

    monkeypatch.setattr(O, "rotate_kpe_bf16", planted)
    # with rot = 128 the planted version rotates two 64-wide halves
    with pytest.raises(AssertionError):
        test_gqa_splice_matches_list_rebuild(2, 128, 128, "interleaved")
