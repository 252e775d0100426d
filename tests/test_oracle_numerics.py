"""Pins for the oracle's numerics: bf16 storage, RoPE frequencies and the
delta-rotation (Leyline summary, section 2.2; fp32 rotation on bf16 storage,
section 4.3).  Every check here compares the oracle with something other than
itself: a library conversion, a closed form, a second formulation of the
rotation (complex exponentials), an exact float64 value within a stated
rounding bound, or an invariant of the mathematics."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import leyline_oracle as O
from synth import random_normal_np, random_rows_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 -----

def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_random_and_edge_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-38),   # denormal range
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.0e38, -3.0e38], np.float32),
        # ties: low half exactly 0x8000, even and odd upper halves
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x7F7F8000, 0x00008000,
                  0x3F807FFF, 0x3F808001], np.uint32).view(np.float32),
    ])
    assert np.array_equal(O.f32_to_bf16(x), _torch_bf16_bits(x))


def test_bf16_ties_go_to_even_and_overflow_to_inf():
    words = np.array([0x3F808000, 0x3F818000, 0x7F7FFFFF, 0xFF7FFFFF], np.uint32)
    out = O.f32_to_bf16(words.view(np.float32))
    assert list(out) == [0x3F80, 0x3F82, 0x7F80, 0xFF80]


def test_bf16_nan_stays_nan():
    words = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF], np.uint32)
    out = O.f32_to_bf16(words.view(np.float32))
    assert np.all(np.isnan(O.bf16_to_f32(out)))


def test_bf16_widening_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = O.bf16_to_f32(bits)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert np.all(same)


# ------------------------------------------------------- RoPE frequencies --

def test_theta_closed_forms():
    th = O.rope_theta(64, 10000.0)
    assert len(th) == 32
    assert th[0] == 1.0
    assert abs(th[8] - 0.1) < 1e-16       # 10000^(-16/64) = 10^-1
    assert abs(th[16] - 0.01) < 1e-17     # 10000^(-32/64) = 10^-2
    assert abs(th[24] - 0.001) < 1e-18    # 10000^(-48/64) = 10^-3
    assert all(a > b for a, b in zip(th, th[1:]))


def test_worked_rotation_values():
    """Closed-form worked values: a unit x-vector in pair 0 (theta = 1) rotated
    by one step lands on (cos 1, sin 1); pair 16 (theta = 0.01) rotated by 100
    steps turns by the same 1 radian.  Stored under tests/golden."""
    with open(os.path.join(GOLDEN, "rope_worked_values.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        k = np.zeros(64)
        ix, iy = O.pair_index(64, case["pairing"])
        j = case["pair"]
        k[ix[j]], k[iy[j]] = case["x"], case["y"]
        out = O.rotate_f64(k, case["steps"], pairing=case["pairing"])
        assert abs(out[ix[j]] - case["x_out"]) < 1e-12, case
        assert abs(out[iy[j]] - case["y_out"]) < 1e-12, case
        others = np.delete(out, [ix[j], iy[j]])
        assert np.all(others == 0.0)


# ------------------------------------------- rotation: float64 invariants --

@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_rotation_equals_complex_exponential(pairing):
    """Second formulation: pair j as the complex number x + iy multiplied by
    exp(i * steps * theta_j)."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((50, 64))
    steps = rng.integers(-50000, 50000, size=50)
    ix, iy = O.pair_index(64, pairing)
    th = np.array([10000.0 ** (-2 * j / 64) for j in range(32)])
    z = (k[:, ix] + 1j * k[:, iy]) * np.exp(1j * steps[:, None] * th[None, :])
    out = O.rotate_f64(k, steps, pairing=pairing)
    assert np.allclose(out[:, ix], z.real, atol=1e-12, rtol=0)
    assert np.allclose(out[:, iy], z.imag, atol=1e-12, rtol=0)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_rotation_closure_and_fresh_rope(pairing):
    """R(a)R(b) = R(a+b); a key stored at position i and rotated by Delta
    equals RoPE applied afresh at i + Delta (Leyline section 2.2)."""
    rng = np.random.default_rng(2)
    k_raw = rng.standard_normal((64, 64))
    i = rng.integers(0, 131072, size=64)
    d = rng.integers(-20000, 20000, size=64)
    stored = O.rotate_f64(k_raw, i, pairing=pairing)
    moved = O.rotate_f64(stored, d, pairing=pairing)
    fresh = O.rotate_f64(k_raw, i + d, pairing=pairing)
    assert np.max(np.abs(moved - fresh)) < 1e-9


def test_attention_scores_preserved_for_downstream_pairs():
    """A query at m' = m + Delta and a downstream key rotated by Delta give the
    same RoPE score as before the splice (the attention maths of the original
    context is kept, Leyline section 2.2).  A rotation by -Delta does not."""
    rng = np.random.default_rng(3)
    q_raw = rng.standard_normal((32, 64))
    k_raw = rng.standard_normal((32, 64))
    m = rng.integers(20000, 40000, size=32)
    i = rng.integers(10000, 19999, size=32)
    delta = -6120
    before = np.sum(O.rotate_f64(q_raw, m) * O.rotate_f64(k_raw, i), axis=-1)
    k_moved = O.rotate_f64(O.rotate_f64(k_raw, i), delta)
    after = np.sum(O.rotate_f64(q_raw, m + delta) * k_moved, axis=-1)
    assert np.max(np.abs(after - before)) < 1e-9
    wrong = np.sum(O.rotate_f64(q_raw, m + delta) * O.rotate_f64(O.rotate_f64(k_raw, i), -delta), axis=-1)
    assert np.max(np.abs(wrong - before)) > 1e-2


def test_half_split_is_interleaved_on_permuted_dims():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((10, 64))
    perm = np.empty(64, np.int64)
    perm[0::2] = np.arange(32)          # interleaved slot 2j <- half-split dim j
    perm[1::2] = np.arange(32) + 32     # interleaved slot 2j+1 <- dim j+32
    a = O.rotate_f64(k, 777, pairing="half")
    b = O.rotate_f64(k[:, perm], 777, pairing="interleaved")
    assert np.allclose(a[:, perm], b, atol=1e-13)


# -------------------------------------------- rotation: bf16/fp32 mode -----

def test_delta_cos_sin_is_float32_of_float64_values():
    for delta in (-6120, -1984, 1, 12345, -130000):
        c, s = O.delta_cos_sin(delta)
        th = np.array([10000.0 ** (-2 * j / 64) for j in range(32)])
        cc, ss = np.cos(delta * th), np.sin(delta * th)
        assert c.dtype == np.float32 and s.dtype == np.float32
        # float32 rounding of a value within ~1e-16 of the exact one
        assert np.all(np.abs(c.astype(np.float64) - cc) <= 2.0 ** -24 * np.abs(cc) + 1e-15)
        assert np.all(np.abs(s.astype(np.float64) - ss) <= 2.0 ** -24 * np.abs(ss) + 1e-15)


def _bf16_ulp(v):
    v = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(v)) - 7)


@pytest.mark.parametrize("pairing", ["interleaved", "half"])
def test_bf16_rotation_within_half_ulp_of_exact(pairing):
    """Each output element lies within half a bf16 ulp (plus the float32
    rounding budget of two products, one sum and the float32 cos/sin) of the
    exact rotation of the same bf16 inputs."""
    bits = random_rows_np(5, (4000, 64))
    for delta in (-6120, -1984, 37, 100000):
        out = O.rotate_kpe_bf16(bits, delta, pairing=pairing)
        x64 = O.bf16_to_f32(bits).astype(np.float64)
        exact = O.rotate_f64(x64, delta, pairing=pairing)
        got = O.bf16_to_f32(out).astype(np.float64)
        ix, iy = O.pair_index(64, pairing)
        mag = np.empty_like(x64)
        mag[:, ix] = mag[:, iy] = np.abs(x64[:, ix]) + np.abs(x64[:, iy])
        tol = 0.5 * _bf16_ulp(np.maximum(np.abs(exact), np.abs(got))) + 8 * 2.0 ** -24 * mag
        assert np.all(np.abs(got - exact) <= tol)


def test_bf16_rotation_zero_delta_is_bit_identical():
    bits = random_rows_np(6, (1000, 64))
    assert np.array_equal(O.rotate_kpe_bf16(bits, 0), bits)


def test_bf16_rotation_relative_l2_to_fresh_rope():
    """Rows stored as bf16(RoPE(i) k_raw), rotated by Delta in fp32 and stored
    again in bf16, stay within relative L2 5e-3 of RoPE(i + Delta) k_raw in
    float64 (two bf16 roundings: about 2.35e-3 on N(0,1) data)."""
    k_raw = random_normal_np(7, (20000, 64))
    i = np.arange(14336, 14336 + 20000)
    delta = -6120
    stored = O.f32_to_bf16(O.rotate_f64(k_raw, i).astype(np.float32))
    moved = O.bf16_to_f32(O.rotate_kpe_bf16(stored, delta)).astype(np.float64)
    fresh = O.rotate_f64(k_raw, i + delta)
    rel = np.linalg.norm(moved - fresh) / np.linalg.norm(fresh)
    assert 1.5e-3 < rel < 3.5e-3
    assert rel <= 5e-3


def test_bf16_rotation_composes_within_tolerance():
    """Two successive rotations stay near one rotation by the sum (closure on
    bf16 storage, up to one extra rounding)."""
    bits = random_rows_np(8, (5000, 64))
    a = O.rotate_kpe_bf16(O.rotate_kpe_bf16(bits, -300), -700)
    b = O.rotate_kpe_bf16(bits, -1000)
    fa, fb = O.bf16_to_f32(a).astype(np.float64), O.bf16_to_f32(b).astype(np.float64)
    assert np.linalg.norm(fa - fb) / np.linalg.norm(fb) < 5e-3
