"""Pins for the padded, variable-length prefill oracle (CPU only)."""

import numpy as np
import pytest

from oracle import mla_attention, mla_prefill_varlen

ALPHA = float(np.float32(192.0 ** -0.5))


def _rand(B, H, Tmax, Smax, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Tmax, 128)), rng.standard_normal((B, H, Tmax, 64)),
            rng.standard_normal((B, H, Smax, 128)), rng.standard_normal((B, 1, Smax, 64)),
            rng.standard_normal((B, H, Smax, 128)))


def test_explicit_4d_mask_over_the_padded_matrix():
    """Scores of every padded query against every padded key, plus a 4D mask
    built from the causal offset P_b and the 2D padding mask of the keys:
    rows below T_b match; padded rows are 0."""
    tq, pp = np.array([5, 1, 8, 3]), np.array([4, 0, 2, 9])
    B, H, Tmax, Smax = 4, 3, 8, 12
    qn, qp, kn, kp, v = _rand(B, H, Tmax, Smax, 1)
    got = mla_prefill_varlen(qn, qp, kn, kp, v, tq, pp, ALPHA)
    s = np.einsum("bhid,bhjd->bhij", qn, kn) + np.einsum("bhid,bjd->bhij", qp, kp[:, 0])
    i = np.arange(Tmax)[:, None]
    j = np.arange(Smax)[None, :]
    for b in range(B):
        keep = (j <= pp[b] + i) & (j < pp[b] + tq[b])          # causal offset and 2D padding
        z = ALPHA * s[b] + np.where(keep, 0.0, -np.inf)[None]
        for h in range(H):
            for q in range(tq[b]):
                row = z[h, q] - z[h, q].max()
                p = np.exp(row) / np.exp(row).sum()
                assert np.max(np.abs(got[b, h, q] - p @ v[b, h])) <= 1e-12
        assert not np.any(got[b, :, tq[b]:])


def test_padded_rows_are_never_read():
    tq, pp = np.array([3, 6, 0]), np.array([5, 1, 4])
    B, H, Tmax, Smax = 3, 2, 6, 10
    qn, qp, kn, kp, v = _rand(B, H, Tmax, Smax, 2)
    base = mla_prefill_varlen(qn, qp, kn, kp, v, tq, pp, ALPHA)
    for b in range(B):
        qn[b, :, tq[b]:] = np.nan
        qp[b, :, tq[b]:] = np.nan
        kn[b, :, pp[b] + tq[b]:] = np.nan
        kp[b, :, pp[b] + tq[b]:] = np.nan
        v[b, :, pp[b] + tq[b]:] = np.nan
    got = mla_prefill_varlen(qn, qp, kn, kp, v, tq, pp, ALPHA)
    assert np.array_equal(got, base)


def test_equal_lengths_are_the_dense_prefill():
    B, H, Tmax, Smax = 2, 3, 5, 9
    x = _rand(B, H, Tmax, Smax, 3)
    got = mla_prefill_varlen(*x, np.full(B, Tmax), np.full(B, Smax - Tmax), ALPHA)
    assert np.array_equal(got, mla_attention(*x, Smax - Tmax, ALPHA))


def test_zero_queries_give_causal_prefix_means():
    tq, pp = np.array([4, 2]), np.array([3, 0])
    B, H, Tmax, Smax = 2, 2, 4, 8
    qn, qp, kn, kp, v = _rand(B, H, Tmax, Smax, 4)
    qn[:] = 0.0
    qp[:] = 0.0
    got = mla_prefill_varlen(qn, qp, kn, kp, v, tq, pp, ALPHA)
    for b in range(B):
        for q in range(tq[b]):
            assert np.max(np.abs(got[b, :, q] - v[b, :, :pp[b] + q + 1].mean(axis=1))) <= 1e-12


def test_batch_permutation_and_errors():
    tq, pp = np.array([2, 5, 1]), np.array([6, 0, 3])
    x = _rand(3, 2, 5, 8, 5)
    perm = np.array([1, 2, 0])
    base = mla_prefill_varlen(*x, tq, pp, ALPHA)
    got = mla_prefill_varlen(*(t[perm] for t in x), tq[perm], pp[perm], ALPHA)
    assert np.array_equal(got, base[perm])
    with pytest.raises(ValueError):
        mla_prefill_varlen(*x, np.array([6, 1, 1]), pp, ALPHA)      # beyond Tmax
    with pytest.raises(ValueError):
        mla_prefill_varlen(*x, tq, np.array([7, 0, 0]), ALPHA)      # past + queries beyond Smax
