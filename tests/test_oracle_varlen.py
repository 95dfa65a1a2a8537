"""Pins for the right-padded, variable-length decode oracle (CPU only).

Each test checks oracle.mla_varlen against something other than its own code
path: an explicit 2D padding mask added to the scores of the whole cache
(the "Causal mask" page's 2D mask handed to the 4D builder), closed forms,
NaN planted in the padding, and symmetry.
"""

import numpy as np
import pytest

from oracle import mla_decode_varlen, mla_decode_varlen_rows

ALPHA = float(np.float32(192.0 ** -0.5))


def _rand(B, H, cap, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, 1, 128)), rng.standard_normal((B, H, 1, 64)),
            rng.standard_normal((B, H, cap, 128)), rng.standard_normal((B, 1, cap, 64)),
            rng.standard_normal((B, H, cap, 128)))


def test_padding_rows_are_never_read():
    lens = np.array([5, 9, 1, 0, 12])
    B, H, cap = len(lens), 3, 12
    qn, qp, kn, kp, v = _rand(B, H, cap, 1)
    base = mla_decode_varlen(qn, qp, kn, kp, v, lens, ALPHA)
    for b, L in enumerate(lens):
        kn[b, :, L:] = np.nan
        kp[b, :, L:] = np.nan
        v[b, :, L:] = np.nan
    got = mla_decode_varlen(qn, qp, kn, kp, v, lens, ALPHA)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, base)


def test_explicit_padding_mask_over_the_whole_cache():
    """Scores against every cache row, 0 / -inf added from the 2D mask
    [1]*L + [0]*(cap-L), softmax over all rows: the same output."""
    lens = np.array([7, 1, 16, 3])
    B, H, cap = len(lens), 4, 16
    qn, qp, kn, kp, v = _rand(B, H, cap, 2)
    s = (np.einsum("bhd,bhjd->bhj", qn[:, :, 0], kn)
         + np.einsum("bhd,bjd->bhj", qp[:, :, 0], kp[:, 0]))
    mask2d = (np.arange(cap)[None, :] < lens[:, None]).astype(np.int64)   # 1 keeps, 0 pads
    z = ALPHA * s + np.where(mask2d[:, None, :] == 1, 0.0, -np.inf)
    z -= z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=-1, keepdims=True)
    ref = np.einsum("bhj,bhjd->bhd", p, v)
    got = mla_decode_varlen(qn, qp, kn, kp, v, lens, ALPHA)[:, :, 0]
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_zero_queries_give_prefix_means():
    lens = np.array([4, 11, 2])
    B, H, cap = len(lens), 2, 11
    qn, qp, kn, kp, v = _rand(B, H, cap, 3)
    qn[:] = 0.0
    qp[:] = 0.0
    got = mla_decode_varlen(qn, qp, kn, kp, v, lens, ALPHA)
    for b, L in enumerate(lens):
        assert np.max(np.abs(got[b, :, 0] - v[b, :, :L].mean(axis=1))) <= 1e-12


def test_one_key_sequences_return_their_value_and_empty_ones_zero():
    lens = np.array([1, 0, 1])
    B, H, cap = len(lens), 3, 6
    qn, qp, kn, kp, v = _rand(B, H, cap, 4)
    got = mla_decode_varlen(qn, qp, kn, kp, v, lens, ALPHA)
    assert np.array_equal(got[0, :, 0], v[0, :, 0])
    assert np.array_equal(got[2, :, 0], v[2, :, 0])
    assert np.array_equal(got[1], np.zeros_like(got[1]))


def test_batch_permutation_moves_lengths_with_sequences():
    lens = np.array([3, 8, 5, 1])
    B, H, cap = len(lens), 2, 8
    x = _rand(B, H, cap, 5)
    perm = np.array([2, 0, 3, 1])
    base = mla_decode_varlen(*x, lens, ALPHA)
    got = mla_decode_varlen(*(t[perm] for t in x), lens[perm], ALPHA)
    assert np.array_equal(got, base[perm])


def test_rows_variant_matches():
    lens = np.array([6, 0, 9])
    x = _rand(3, 4, 9, 6)
    full = mla_decode_varlen(*x, lens, ALPHA)
    rows = [(0, 3), (1, 0), (2, 2), (2, 0)]
    got = mla_decode_varlen_rows(*x, lens, ALPHA, rows)
    for n, (b, h) in enumerate(rows):
        assert np.array_equal(got[n], full[b, h, 0])


def test_length_errors():
    x = _rand(2, 1, 4, 7)
    with pytest.raises(ValueError):
        mla_decode_varlen(*x, np.array([5, 1]), ALPHA)
    with pytest.raises(ValueError):
        mla_decode_varlen(*x, np.array([-1, 1]), ALPHA)
    with pytest.raises(ValueError):
        mla_decode_varlen(*x, np.array([1, 1, 1]), ALPHA)
