"""Pins for the oracle's rotary embedding (reading: interleaved pairs,
counter-clockwise rotation by p * base**(-2i/d_rope), 0-based positions)."""
import math

import numpy as np
import pytest

from oracle import brute
from oracle.mla_oracle import rope_inv_freq, rope_rotate


def test_two_dim_rotation_values():
    # d_rope = 2 has the single frequency base**0 = 1: position p rotates by p radians.
    for p in (0, 1, 2, 7):
        x = rope_rotate(np.array([1.0, 0.0]), p, 10000.0)
        y = rope_rotate(np.array([0.0, 1.0]), p, 10000.0)
        assert x == pytest.approx([math.cos(p), math.sin(p)], abs=1e-15)
        assert y == pytest.approx([-math.sin(p), math.cos(p)], abs=1e-15)


def test_frequencies():
    assert rope_inv_freq(8, 10000.0) == pytest.approx([1.0, 0.1, 0.01, 0.001], rel=1e-15)
    assert rope_inv_freq(64, 10000.0)[-1] == pytest.approx(10000.0 ** (-62 / 64), rel=1e-15)
    # pair i of a unit vector turns by exactly p * theta_i
    v = np.zeros(8)
    v[4] = 1.0                                 # pair 2, theta = 0.01
    out = rope_rotate(v, 100, 10000.0)
    assert math.atan2(out[5], out[4]) == pytest.approx(1.0, abs=1e-14)
    assert np.all(out[[0, 1, 2, 3, 6, 7]] == 0.0)


def test_identity_at_zero_and_norm():
    rng = np.random.default_rng(0)
    v = rng.standard_normal((5, 64))
    assert np.array_equal(rope_rotate(v, 0, 10000.0), v)
    for p in (1, 17, 4095, 131071):
        r = rope_rotate(v, p, 10000.0)
        assert np.linalg.norm(r, axis=1) == pytest.approx(np.linalg.norm(v, axis=1), rel=1e-13)


def test_relative_position_property():
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(5, 2), (100, 99), (4096, 17), (131071, 65536)]:
        lhs = rope_rotate(a, m, 10000.0) @ rope_rotate(b, n, 10000.0)
        rhs = rope_rotate(a, m - n, 10000.0) @ b
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


def test_composition():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(16)
    assert rope_rotate(rope_rotate(v, 3, 500.0), 4, 500.0) == pytest.approx(rope_rotate(v, 7, 500.0), abs=1e-13)


def test_matches_scalar_rotation_at_long_positions():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(64)
    for p in (32769, 131071):
        assert rope_rotate(v, p, 10000.0) == pytest.approx(brute.rotate(list(v), p, 10000.0), abs=1e-10)


def test_rotation_does_not_commute_with_absorption():
    """Rotating the folded d_c-wide query and scoring it against unrotated
    latents is not full-RoPE attention: scores change by O(1) and the ranking
    changes ("Multi-head Latent Attention: the KV cache, compressed", section
    "RoPE, and why the explanations stop here")."""
    rng = np.random.default_rng(4)
    n, d_c, hd, p = 8, 16, 8, 7
    c = rng.standard_normal((n, d_c))
    w_uk = rng.standard_normal((d_c, hd))
    q = rng.standard_normal(hd)
    keys = c @ w_uk
    correct = np.array([rope_rotate(q, p, 10000.0) @ rope_rotate(keys[t], t, 10000.0) for t in range(n)])
    wrong = np.array([rope_rotate(w_uk @ q, p, 10000.0) @ c[t] for t in range(n)])
    assert np.max(np.abs(correct - wrong)) > 1.0
    assert not np.array_equal(np.argsort(correct), np.argsort(wrong))


def test_latent_rows_rotate_only_the_rope_block_at_each_tokens_position():
    """The cached row [c | k_rope] of a token: c = x W_dkv unrotated, k_rope =
    the tail of x W_dkv turned pair by pair by position * base**(-2i/d_rope),
    written here as multiplication by a complex exponential."""
    from oracle.mla_oracle import latent_rows

    rng = np.random.default_rng(17)
    d_model, d_c, d_rope, base = 24, 12, 8, 10000.0
    x = rng.standard_normal((5, d_model))
    w = rng.standard_normal((d_model, d_c + d_rope))
    positions = np.array([0, 1, 9, 300, 4095])
    rows = latent_rows(x, w, positions, d_c, base)
    u = x @ w
    assert np.array_equal(rows[:, :d_c], u[:, :d_c])          # content block untouched
    assert np.array_equal(rows[0], u[0])                      # position 0: no rotation
    for t, p in enumerate(positions):
        z = u[t, d_c::2] + 1j * u[t, d_c + 1::2]
        turn = np.exp(1j * p * base ** (-2.0 * np.arange(d_rope // 2) / d_rope))
        want = z * turn
        assert rows[t, d_c::2] == pytest.approx(want.real, abs=1e-12)
        assert rows[t, d_c + 1::2] == pytest.approx(want.imag, abs=1e-12)
