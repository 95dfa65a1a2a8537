"""Pins for the paged-cache decode oracle (CPU only).

Each test checks oracle.mla_paged against something other than its own
gather: the pinned variable-length oracle on a contiguous layout, block
relabelling, NaN planted where no sequence reads, the append done by hand
first, and closed forms.
"""

import numpy as np
import pytest

from oracle import mla_decode_paged, mla_decode_varlen

ALPHA = float(np.float32(192.0 ** -0.5))


def _paged(B, H, nblocks, bs, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, 1, 128)), rng.standard_normal((B, H, 1, 64)),
            rng.standard_normal((nblocks, H, bs, 128)), rng.standard_normal((nblocks, bs, 64)),
            rng.standard_normal((nblocks, H, bs, 128)))


def _new(B, H, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, 1, 128)), rng.standard_normal((B, 1, 1, 64)),
            rng.standard_normal((B, H, 1, 128)))


def test_contiguous_table_is_the_variable_length_decode():
    """Sequence b owning blocks b*M .. b*M+M-1 in order is a cache [B,H,M*bs]
    laid out block by block."""
    B, H, bs, M = 3, 2, 4, 3
    qn, qp, kn, kp, v = _paged(B, H, B * M, bs, 1)
    table = np.arange(B * M).reshape(B, M)
    lens = np.array([12, 5, 1])
    ck = kn.reshape(B, M, H, bs, 128).transpose(0, 2, 1, 3, 4).reshape(B, H, M * bs, 128)
    cp = kp.reshape(B, M * bs, 64)[:, None]
    cv = v.reshape(B, M, H, bs, 128).transpose(0, 2, 1, 3, 4).reshape(B, H, M * bs, 128)
    ref = mla_decode_varlen(qn, qp, ck, cp, cv, lens, ALPHA)
    got, _ = mla_decode_paged(qn, qp, kn, kp, v, table, lens, ALPHA)
    assert np.array_equal(got, ref)


def test_relabelling_blocks_changes_nothing():
    B, H, bs, M, N = 2, 3, 4, 3, 9
    qn, qp, kn, kp, v = _paged(B, H, N, bs, 2)
    table = np.array([[4, 0, 7], [2, 8, 5]])
    lens = np.array([10, 7])
    base, _ = mla_decode_paged(qn, qp, kn, kp, v, table, lens, ALPHA)
    perm = np.random.default_rng(3).permutation(N)          # physical block i -> perm[i]
    kn2, kp2, v2 = np.empty_like(kn), np.empty_like(kp), np.empty_like(v)
    kn2[perm], kp2[perm], v2[perm] = kn, kp, v
    got, _ = mla_decode_paged(qn, qp, kn2, kp2, v2, perm[table], lens, ALPHA)
    assert np.array_equal(got, base)


def test_unowned_blocks_and_rows_are_never_read():
    B, H, bs, N = 2, 2, 4, 6
    qn, qp, kn, kp, v = _paged(B, H, N, bs, 4)
    table = np.array([[1, 3], [5, 0]])
    lens = np.array([6, 3])
    base, _ = mla_decode_paged(qn, qp, kn, kp, v, table, lens, ALPHA)
    for blk in (2, 4):                       # owned by no sequence
        kn[blk], kp[blk], v[blk] = np.nan, np.nan, np.nan
    kn[3, :, 2:], kp[3, 2:], v[3, :, 2:] = np.nan, np.nan, np.nan   # seq 0: rows 6, 7
    kn[5, :, 3:], kp[5, 3:], v[5, :, 3:] = np.nan, np.nan, np.nan   # seq 1: row 3
    kn[0], kp[0], v[0] = np.nan, np.nan, np.nan                     # seq 1's second block
    got, _ = mla_decode_paged(qn, qp, kn, kp, v, table, lens, ALPHA)
    assert np.array_equal(got, base)


def test_append_equals_writing_first():
    B, H, bs, N = 3, 2, 4, 8
    qn, qp, kn, kp, v = _paged(B, H, N, bs, 5)
    new = _new(B, H, 6)
    table = np.array([[0, 1], [2, 3], [7, 6]])
    lens = np.array([5, 8, 1])
    got, (kn2, kp2, v2) = mla_decode_paged(qn, qp, kn, kp, v, table, lens, ALPHA, new=new)
    # by hand: row L-1 of each sequence takes the new rows
    kh, ph, vh = kn.copy(), kp.copy(), v.copy()
    for b, (blk, r) in enumerate([(1, 0), (3, 3), (7, 0)]):
        kh[blk, :, r] = new[0][b, :, 0]
        ph[blk, r] = new[1][b, 0, 0]
        vh[blk, :, r] = new[2][b, :, 0]
    assert np.array_equal(kn2, kh) and np.array_equal(kp2, ph) and np.array_equal(v2, vh)
    ref, _ = mla_decode_paged(qn, qp, kh, ph, vh, table, lens, ALPHA)
    assert np.array_equal(got, ref)
    # the appended one-key sequence returns its new value exactly
    assert np.array_equal(got[2, :, 0], new[2][2, :, 0])
    # the input pages are not modified
    assert not np.array_equal(kn, kh)


def test_zero_length_and_errors():
    qn, qp, kn, kp, v = _paged(2, 1, 3, 4, 7)
    table = np.array([[0, 1], [2, 0]])
    got, _ = mla_decode_paged(qn, qp, kn, kp, v, table, np.array([0, 3]), ALPHA)
    assert not np.any(got[0])
    with pytest.raises(ValueError):
        mla_decode_paged(qn, qp, kn, kp, v, table, np.array([9, 1]), ALPHA)
