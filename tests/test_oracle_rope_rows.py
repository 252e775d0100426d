"""Pins for the oracle's per-row-angle RoPE rotation (each row turned by its own
angle steps, e.g. back by its position as VECTOR does before reconstructing V
from K; "VECTOR", gist.science summary, method: reconstructability through
OLS, keys inverse-rotated before reconstruction).

Checked against: the float64 complex exponential for the per-row tables
(within float32 rounding), a high-precision argument reduction for angles up
to 2^31 radians, the directive rotation for a constant angle, the recovery of
position-free keys from stored bf16(RoPE(p) k) rows, composition, and a
row-by-row rebuild of the gathered and in-place results on MLA and GQA
caches."""

from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import leyline_oracle as O
from synth import np_rng, permuted_pages, random_rows_np


def test_row_tables_match_the_complex_exponential():
    rng = np_rng(1, 0)
    a = rng.integers(-200000, 200000, size=200)
    c, s = O.row_cos_sin(a)
    th = 10000.0 ** (-2.0 * np.arange(32) / 64)
    z = np.exp(1j * a[:, None].astype(np.float64) * th[None, :])
    assert np.max(np.abs(c - z.real)) <= 2 ** -24 * 1.01
    assert np.max(np.abs(s - z.imag)) <= 2 ** -24 * 1.01


def test_large_angles_against_a_long_reduction():
    """theta_0 = 1, so column 0 is cos/sin of the integer a itself; reduce a
    modulo 2 pi with 60 significant digits and compare."""
    getcontext().prec = 60
    pi = Decimal("3.14159265358979323846264338327950288419716939937510582097494459")
    for a in (2 ** 31 - 1, -(2 ** 31), 1234567891, 987654321, 2 ** 30 + 7):
        r = Decimal(a) % (2 * pi)
        c, s = O.row_cos_sin([a])
        # Taylor series in Decimal on the reduced argument
        x = r - pi  # in [-pi, pi): cos(x + pi) = -cos(x)
        term, cos_x, sin_x = Decimal(1), Decimal(0), Decimal(0)
        for k in range(60):
            if k % 4 == 0:
                cos_x += term
            elif k % 4 == 1:
                sin_x += term
            elif k % 4 == 2:
                cos_x -= term
            else:
                sin_x -= term
            term = term * x / (k + 1)
        assert abs(float(c[0, 0]) - float(-cos_x)) <= 2 ** -24
        assert abs(float(s[0, 0]) - float(-sin_x)) <= 2 ** -24


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_constant_angle_is_the_directive_rotation(pairing):
    rows = random_rows_np(3, (100, 64))
    for a in (0, 1, -6120, 31337):
        got = O.rotate_rows_bf16(rows, np.full(100, a), pairing=pairing)
        assert np.array_equal(got, O.rotate_kpe_bf16(rows, a, pairing=pairing))
    assert np.array_equal(O.rotate_rows_bf16(rows, np.zeros(100, np.int64)), rows)


@pytest.mark.parametrize("rope_dim", [64, 128])
def test_back_rotation_recovers_position_free_keys(rope_dim):
    rng = np_rng(4, rope_dim)
    k = rng.standard_normal((500, rope_dim))
    p = rng.integers(0, 131072, size=500)
    stored = O.f32_to_bf16(O.rotate_f64(k, p, rope_dim=rope_dim).astype(np.float32))
    back = O.bf16_to_f32(O.rotate_rows_bf16(stored, -p, rope_dim=rope_dim)).astype(np.float64)
    rel = np.linalg.norm(back - k) / np.linalg.norm(k)
    assert rel < 4e-3            # two bf16 roundings
    wrong = O.bf16_to_f32(O.rotate_rows_bf16(stored, p, rope_dim=rope_dim)).astype(np.float64)
    assert np.linalg.norm(wrong - k) / np.linalg.norm(k) > 0.5


def test_per_row_rotations_compose():
    rng = np_rng(5, 0)
    rows = random_rows_np(5, (300, 64))
    a = rng.integers(-50000, 50000, size=300)
    b = rng.integers(-50000, 50000, size=300)
    two = O.bf16_to_f32(O.rotate_rows_bf16(O.rotate_rows_bf16(rows, a), b)).astype(np.float64)
    one = O.bf16_to_f32(O.rotate_rows_bf16(rows, a + b)).astype(np.float64)
    assert np.linalg.norm(two - one) / np.linalg.norm(one) < 5e-3


def _mla_state(n, P=16, pages=64, layers=2, seed=0):
    st = O.CacheState.empty(layers, pages, P, pages)
    for L in range(layers):
        st.layers[L][:] = random_rows_np(seed + L, (pages, P, O.ROW))
    st.set_pages(0, permuted_pages(seed, pages)[:-(-n // P)], n)
    return st


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_rope_rows_gather_and_in_place_on_mla(pairing):
    st = _mla_state(700)
    a = np_rng(6, 0).integers(-10 ** 6, 10 ** 6, size=250)
    outs = O.rope_rows(st, 0, 300, a, pairing=pairing)
    new = O.rope_rows(st, 0, 300, a, pairing=pairing, in_place=True)
    for L in range(2):
        rows = st.logical_rows(0, L)
        for i in range(250):
            exp = rows[300 + i].copy()
            exp[512:] = O.rotate_kpe_bf16(exp[512:], int(a[i]), pairing=pairing)
            assert np.array_equal(outs[L][i], exp)
        after = new.logical_rows(0, L)
        assert np.array_equal(after[300:550], outs[L])
        assert np.array_equal(after[:300], rows[:300]) and np.array_equal(after[550:], rows[550:])
        assert np.array_equal(st.logical_rows(0, L), rows)       # the input state is untouched


def test_rope_rows_on_gqa_turns_only_k_bands():
    H, D, rot = 4, 64, 32
    specs = [O.gqa_k_row(H, D, rot), O.plain_row(H * D)]
    st = O.CacheState.empty(2, 32, 4, 32, specs=specs)
    for i, sp in enumerate(specs):
        st.layers[i][:] = random_rows_np(10 + i, (32, 4, sp.width))
    st.set_pages(0, permuted_pages(1, 32)[:20], 77)
    a = np_rng(7, 0).integers(-5000, 5000, size=40)
    outs = O.rope_rows(st, 0, 30, a, pairing="half")
    assert len(outs) == 1                                       # V carries no band
    k = st.logical_rows(0, 0)[30:70].reshape(40, H, D)
    got = outs[0].reshape(40, H, D)
    assert np.array_equal(got[..., rot:], k[..., rot:])
    for h in range(H):
        assert np.array_equal(got[:, h, :rot], O.rotate_rows_bf16(k[:, h, :rot], a, rope_dim=rot, pairing="half"))
    new = O.rope_rows(st, 0, 30, a, pairing="half", in_place=True)
    assert np.array_equal(new.logical_rows(0, 1), st.logical_rows(0, 1))


def test_rope_rows_rejects_rows_outside_the_sequence():
    st = _mla_state(100)
    with pytest.raises(O.InvalidRequest):
        O.rope_rows(st, 0, 90, np.zeros(11, np.int64))
    with pytest.raises(O.InvalidRequest):
        O.rope_rows(st, 3, 0, np.zeros(1, np.int64))


def test_pins_catch_a_sign_error_in_the_row_table(monkeypatch):
    real = O.row_cos_sin
    monkeypatch.setattr(O, "row_cos_sin", lambda angles, rope_dim=64, base=10000.0:
                        real(-np.asarray(angles, np.int64), rope_dim, base))
    with pytest.raises(AssertionError):
        test_back_rotation_recovers_position_free_keys(64)
