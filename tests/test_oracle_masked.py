"""Pins for the 2D-padding-mask oracle (CPU only).

Each test ties mla_attention_masked to something other than itself: the dense
oracle, the variable-length decode oracle, the unpadded sequence under a
shorter cache, a scalar brute force that leaves hidden keys out of the sums,
and invariants (hidden rows are never read; rows with no visible key are 0).
A mask applied to queries instead of keys, an index off by the cached length,
an OR instead of an AND of the two masks, or a hidden key that still reaches
the sums fails at least one of them.
"""

import math

import numpy as np
import pytest

from oracle import mla_attention, mla_attention_masked, mla_decode_varlen, visible_keys

ALPHA = float(np.float32(192.0 ** -0.5))


def _rand(B, H, T, S, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, T, 128)), rng.standard_normal((B, H, T, 64)),
            rng.standard_normal((B, H, S, 128)), rng.standard_normal((B, 1, S, 64)),
            rng.standard_normal((B, H, S, 128)))


def test_all_ones_mask_is_the_dense_oracle():
    B, H, T, P = 2, 3, 7, 5
    x = _rand(B, H, T, P + T, 1)
    got = mla_attention_masked(*x, np.ones((B, P + T), dtype=np.uint8), P, ALPHA)
    assert np.max(np.abs(got - mla_attention(*x, P, ALPHA))) <= 1e-12


def test_right_padding_in_decode_is_the_varlen_decode():
    """One query at position S-1 with the mask [1]*L_b + [0]*(S-L_b): the
    variable-length decode over rows [0, L_b)."""
    B, H, S = 4, 3, 11
    lens = np.array([11, 1, 6, 0])
    x = _rand(B, H, 1, S, 2)
    mask = (np.arange(S)[None, :] < lens[:, None]).astype(np.uint8)
    got = mla_attention_masked(*x, mask, S - 1, ALPHA)
    ref = mla_decode_varlen(*x, lens, ALPHA)
    assert np.max(np.abs(got - ref)) <= 1e-12
    assert not np.any(got[3])


@pytest.mark.parametrize("pad", [0, 3, 9, 12])
def test_left_padding_is_the_unpadded_sequence(pad):
    """Keys are post-RoPE, so positions enter only through the mask: a
    sequence left-padded by `pad` hidden positions gives the unpadded
    sequence's result with `pad` fewer cached keys; queries whose position is
    still inside the padding see nothing and give 0."""
    H, T, P = 2, 6, 9
    S = P + T
    qn, qp, kn, kp, v = _rand(1, H, T, S, 3 + pad)
    mask = (np.arange(S) >= pad).astype(np.uint8)[None, :]
    got = mla_attention_masked(qn, qp, kn, kp, v, mask, P, ALPHA)
    if pad <= P:
        ref = mla_attention(qn, qp, kn[:, :, pad:], kp[:, :, pad:], v[:, :, pad:], P - pad, ALPHA)
        assert np.max(np.abs(got - ref)) <= 1e-12
    else:
        dead = pad - P              # queries at positions < pad see no key
        assert not np.any(got[:, :, :dead])
        ref = mla_attention(qn[:, :, dead:], qp[:, :, dead:], kn[:, :, pad:], kp[:, :, pad:],
                            v[:, :, pad:], 0, ALPHA)
        assert np.max(np.abs(got[:, :, dead:] - ref)) <= 1e-12


def test_hidden_rows_are_never_read():
    B, H, T, P = 3, 2, 5, 8
    S = P + T
    x = list(_rand(B, H, T, S, 4))
    rng = np.random.default_rng(5)
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    mask[:, 0] = 1
    base = mla_attention_masked(*x, mask, P, ALPHA)
    hidden = mask == 0
    for k in (2, 3, 4):                      # k_nope, k_pe, v rows of hidden keys
        for b in range(B):
            x[k][b, :, hidden[b]] = np.nan
    got = mla_attention_masked(*x, mask, P, ALPHA)
    assert np.array_equal(got, base)


def test_brute_force_tiny_random_masks():
    """Scalar loops with math.fsum over the visible keys only."""
    B, H, T, P = 2, 2, 4, 3
    S = P + T
    qn, qp, kn, kp, v = _rand(B, H, T, S, 6)
    rng = np.random.default_rng(7)
    mask = (rng.random((B, S)) < 0.5).astype(np.uint8)
    got = mla_attention_masked(qn, qp, kn, kp, v, mask, P, ALPHA)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                vis = [j for j in range(S) if j <= P + i and mask[b, j]]
                if not vis:
                    assert not np.any(got[b, h, i])
                    continue
                z = [ALPHA * (math.fsum(qn[b, h, i, d] * kn[b, h, j, d] for d in range(128))
                              + math.fsum(qp[b, h, i, d] * kp[b, 0, j, d] for d in range(64)))
                     for j in vis]
                zm = max(z)
                e = [math.exp(t - zm) for t in z]
                den = math.fsum(e)
                for d in range(0, 128, 17):
                    ref = math.fsum(e[n] * v[b, h, j, d] for n, j in enumerate(vis)) / den
                    assert abs(got[b, h, i, d] - ref) <= 1e-12


def test_visible_keys_and_errors():
    vis = visible_keys(np.array([[0, 1, 1, 0, 1]]), 2, 3)
    assert vis.tolist() == [[[False, True, True, False, False], [False, True, True, False, True]]]
    x = _rand(1, 1, 2, 5, 8)
    with pytest.raises(ValueError):
        mla_attention_masked(*x, np.ones((1, 4)), 3, ALPHA)       # mask narrower than the keys
    with pytest.raises(ValueError):
        mla_attention_masked(*x, np.ones((2, 5)), 3, ALPHA)       # one row per sequence


@pytest.mark.parametrize("B,H,T,P", [(2, 3, 6, 4), (3, 2, 1, 20)])
def test_against_torch_sdpa_fp64(B, H, T, P):
    """An independent library routine: torch SDPA in fp64 on the CPU with the
    combined boolean mask (causal offset AND 2D mask); rows with a visible key
    compared (SDPA leaves rows with none undefined)."""
    torch = pytest.importorskip("torch")
    S = P + T
    qn, qp, kn, kp, v = _rand(B, H, T, S, 30 + B + T)
    rng = np.random.default_rng(31 + B)
    mask = (rng.random((B, S)) < 0.6).astype(np.uint8)
    got = mla_attention_masked(qn, qp, kn, kp, v, mask, P, ALPHA)
    q = torch.from_numpy(np.concatenate([qn, qp], -1))
    k = torch.from_numpy(np.concatenate([kn, np.broadcast_to(kp, (B, H, S, 64))], -1))
    allowed = (torch.arange(S)[None, None, :] <= (P + torch.arange(T))[None, :, None]) & \
        torch.from_numpy(mask.astype(bool))[:, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, torch.from_numpy(v),
                                                           attn_mask=allowed[:, None], scale=ALPHA)
    live = allowed.any(-1).numpy()                      # [B, T]
    for b in range(B):
        for i in range(T):
            if live[b, i]:
                np.testing.assert_allclose(got[b, :, i], ref.numpy()[b, :, i], rtol=0, atol=1e-12)
            else:
                assert not np.any(got[b, :, i])
