"""Pins for the rotary-prologue oracle (CPU only).

Each test ties the oracle to something other than itself: textbook RoPE as
complex multiplication, hand-derived frequencies of the released
configuration, hand-computed rotations of unit vectors, and invariants of a
rotation by angles linear in the position. A swapped pair layout (halves
instead of neighbours), a sign flip, slowing the wrong pairs, multiplying by
the factor instead of dividing, a position off by one or a table indexed by
the row instead of the position fails at least one of them.
"""

import math

import numpy as np
import pytest

from oracle import (KIMI_K2_ROPE, apply_rope, mla_attention, rope_cos_sin, rope_positions,
                    yarn_inv_freq)

ALPHA = float(np.float32(192.0 ** -0.5))


def test_factor_one_is_textbook_rope_as_complex_multiplication():
    """Without scaling, pair i turns by pos * theta^(-2i/64): the same as
    multiplying x_{2i} + i x_{2i+1} by exp(i pos w_i)."""
    w = yarn_inv_freq(theta=10000.0, factor=1.0)
    assert np.allclose(w, [10000.0 ** (-k / 32) for k in range(32)], rtol=1e-15, atol=0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 5, 64))
    cos, sin = rope_cos_sin(40, theta=10000.0, factor=1.0)
    pos = np.array([[0, 7, 8, 20, 39], [3, 3, 1, 0, 38]])
    got = apply_rope(x, pos, cos, sin)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * pos[:, None, :, None] * w)
    assert np.max(np.abs(got[..., 0::2] - z.real)) <= 1e-13
    assert np.max(np.abs(got[..., 1::2] - z.imag)) <= 1e-13


def test_released_configuration_frequencies():
    """theta 50000, L = 4096, beta_fast = beta_slow = 1, factor 32. Pair i
    completes r_i = 4096 * 50000^(-i/32) / (2 pi) turns within L; by hand,
    r_19 = 1.057 and r_20 = 0.754, so pairs 0..19 keep their frequency and
    pairs 20..31 (wavelengths longer than 4096) turn 32 times slower."""
    w = yarn_inv_freq(**KIMI_K2_ROPE)
    base = np.array([50000.0 ** (-k / 32) for k in range(32)])
    want = np.where(np.arange(32) <= 19, base, base / 32.0)
    assert np.allclose(w, want, rtol=1e-15, atol=0)


def test_ramp_end_points_and_midpoint():
    """Between beta_slow and beta_fast the blend is linear in r: choose
    beta_fast so that pair 12 sits exactly halfway, where its frequency is the
    mean of the kept and the slowed one."""
    theta, L, s = 50000.0, 4096, 32.0
    base = np.array([theta ** (-k / 32) for k in range(32)])
    r12 = L * base[12] / (2 * math.pi)
    lo = 1.0
    hi = 2 * r12 - lo
    w = yarn_inv_freq(theta=theta, factor=s, original_max_position=L, beta_fast=hi, beta_slow=lo)
    assert w[12] == pytest.approx(base[12] * (1 + 1 / s) / 2, rel=1e-12)
    r = L * base / (2 * math.pi)
    assert np.all(w[r >= hi] == base[r >= hi])               # fast pairs untouched
    assert np.allclose(w[r < lo], base[r < lo] / s, rtol=1e-15)
    mid = (r > lo) & (r < hi)
    assert mid.sum() >= 3
    assert np.all((w[mid] > base[mid] / s) & (w[mid] < base[mid]))
    # the blend factor grows with r
    f = (w[mid] / base[mid] - 1 / s) / (1 - 1 / s)
    assert np.all(np.diff(f[np.argsort(r[mid])]) > 0)


def test_unit_vectors_by_hand():
    """Pair 0 keeps w_0 = 1: e_0 at position 1 becomes (cos 1, sin 1), e_1
    becomes (-sin 1, cos 1). Pair 31 is slowed: e_62 at position p turns by
    p * 50000^(-31/32) / 32."""
    cos, sin = rope_cos_sin(3000, **KIMI_K2_ROPE)
    x = np.zeros((1, 1, 3, 64))
    x[0, 0, 0, 0] = 1.0
    x[0, 0, 1, 1] = 1.0
    x[0, 0, 2, 62] = 1.0
    got = apply_rope(x, np.array([[1, 1, 2999]]), cos, sin)
    exp0 = np.zeros(64)
    exp0[0], exp0[1] = math.cos(1.0), math.sin(1.0)
    exp1 = np.zeros(64)
    exp1[0], exp1[1] = -math.sin(1.0), math.cos(1.0)
    a = 2999 * 50000.0 ** (-31 / 32) / 32
    exp2 = np.zeros(64)
    exp2[62], exp2[63] = math.cos(a), math.sin(a)
    assert np.max(np.abs(got[0, 0, 0] - exp0)) <= 1e-15
    assert np.max(np.abs(got[0, 0, 1] - exp1)) <= 1e-15
    assert np.max(np.abs(got[0, 0, 2] - exp2)) <= 1e-12


def test_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 4, 6, 64))
    cos, sin = rope_cos_sin(9000, **KIMI_K2_ROPE)
    got0 = apply_rope(x, np.zeros((2, 6), dtype=np.int64), cos, sin)
    assert np.array_equal(got0, x)
    pos = rng.integers(0, 9000, size=(2, 6))
    got = apply_rope(x, pos, cos, sin)
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = got[..., 0::2] ** 2 + got[..., 1::2] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 1e-12


def test_scores_depend_on_relative_position_only():
    """<R(m) q, R(n) k> = <R(m - n) q, k> for every pair of positions."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    cos, sin = rope_cos_sin(20000, **KIMI_K2_ROPE)
    for m, n in [(5, 3), (4100, 17), (19999, 19000), (7, 7)]:
        lhs = np.sum(apply_rope(q, np.array([[m]]), cos, sin) * apply_rope(k, np.array([[n]]), cos, sin))
        rhs = np.sum(apply_rope(q, np.array([[m - n]]), cos, sin) * k)
        assert lhs == pytest.approx(rhs, abs=1e-11)


def test_positions_follow_the_cached_length():
    """New token i sits at past_len + i (or past_lens[b] + i); rotating a whole
    sequence and keeping its last T rows is rotating those rows after the
    cached ones."""
    assert rope_positions(2, 3, past_len=5).tolist() == [[5, 6, 7], [5, 6, 7]]
    assert rope_positions(2, 2, past_lens=[0, 9]).tolist() == [[0, 1], [9, 10]]
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 2, 12, 64))
    cos, sin = rope_cos_sin(12, **KIMI_K2_ROPE)
    full = apply_rope(x, rope_positions(1, 12), cos, sin)
    tail = apply_rope(x[:, :, 8:], rope_positions(1, 4, past_len=8), cos, sin)
    assert np.array_equal(full[:, :, 8:], tail)


def test_attention_is_unchanged_when_every_position_shifts():
    """With RoPE applied to the query and key rotary parts at their positions,
    the attention output depends on positions only through their differences:
    moving the whole sequence by d positions changes nothing."""
    rng = np.random.default_rng(4)
    B, H, T, P = 1, 2, 5, 3
    S = P + T
    qn, qp = rng.standard_normal((B, H, T, 128)), rng.standard_normal((B, H, T, 64))
    kn, kp = rng.standard_normal((B, H, S, 128)), rng.standard_normal((B, 1, S, 64))
    v = rng.standard_normal((B, H, S, 128))
    cos, sin = rope_cos_sin(6000, **KIMI_K2_ROPE)
    outs = []
    for d in (0, 1, 4093, 5000):
        q_rot = apply_rope(qp, rope_positions(B, T, past_len=P + d), cos, sin)
        k_rot = apply_rope(kp, rope_positions(B, S, past_len=d), cos, sin)
        outs.append(mla_attention(qn, q_rot, kn, k_rot, v, P, ALPHA))
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-12
    # ... and the rotation does matter: unrotated keys give another result
    q_rot = apply_rope(qp, rope_positions(B, T, past_len=P), cos, sin)
    assert np.max(np.abs(mla_attention(qn, q_rot, kn, kp, v, P, ALPHA) - outs[0])) > 1e-3
