"""Pins for the latent-cache decode oracle (CPU only).

Each test checks oracle.mla_latent against something other than its own
formula: the already pinned attention oracle on hand-built keys and values,
a closed form, or the absorbed evaluation order written out independently.
"""

import numpy as np
import pytest

from oracle import (KV_B_PER_HEAD, KV_LORA_RANK, decompress_kv, mla_attention,
                    mla_decode_latent, mla_decode_latent_rows)
from seeded_inputs import LATENT_WORKLOADS, latent_random_inputs

ALPHA = float(np.float32(192.0 ** -0.5))


def _rand(B, H, S, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, 1, 128)), rng.standard_normal((B, H, 1, 64)),
            rng.standard_normal((B, S, KV_LORA_RANK)), rng.standard_normal((B, 1, S, 64)))


def _selector_weight(H, k_off, v_off, k_scale=None):
    """kv_b_proj weight whose head h copies latent dims [k_off[h], +128) into its key
    and [v_off[h], +128) into its value (times k_scale[h] for the key)."""
    w = np.zeros((H * KV_B_PER_HEAD, KV_LORA_RANK))
    for h in range(H):
        s = 1.0 if k_scale is None else k_scale[h]
        for d in range(128):
            w[h * KV_B_PER_HEAD + d, k_off[h] + d] = s
            w[h * KV_B_PER_HEAD + 128 + d, v_off[h] + d] = 1.0
    return w


def test_kv_b_proj_shape_follows_the_config():
    # "Scale scores": out features = num_heads * (q_head_dim - qk_rope_head_dim + v_head_dim);
    # config.json: 64 heads, 128 + 64 query/key dims, 128 value dims, kv_lora_rank 512.
    heads, q_head_dim, rope, vdim = 64, 128 + 64, 64, 128
    assert KV_B_PER_HEAD * heads == heads * (q_head_dim - rope + vdim) == 16384
    assert KV_LORA_RANK == 512
    w = latent_random_inputs(1, 64, 3, seed=0)["w_kv_b"]
    assert w.shape == (16384, 512)
    assert LATENT_WORKLOADS["latent_decode_p1000"].S == 1001


def test_selector_weights_give_attention_over_latent_slices():
    """Head h's key is latent dims [k_off[h], +128), its value [v_off[h], +128):
    the result must equal the pinned attention oracle on those slices."""
    B, H, S = 2, 5, 9
    qn, qp, c, kp = _rand(B, H, S, 1)
    k_off = [(37 * h) % 384 for h in range(H)]
    v_off = [(101 * h + 13) % 384 for h in range(H)]
    w = _selector_weight(H, k_off, v_off)
    kn = np.stack([c[:, :, k_off[h]:k_off[h] + 128] for h in range(H)], axis=1)
    vv = np.stack([c[:, :, v_off[h]:v_off[h] + 128] for h in range(H)], axis=1)
    ref = mla_attention(qn, qp, kn, kp, vv, S - 1, ALPHA)
    got = mla_decode_latent(qn, qp, c, kp, w, S - 1, ALPHA)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_key_half_scales_per_head():
    """Scaling head h's key block by (h+1) scales only that head's scores."""
    B, H, S = 1, 4, 7
    qn, qp, c, kp = _rand(B, H, S, 2)
    k_off, v_off = [0] * H, [256] * H
    w = _selector_weight(H, k_off, v_off, k_scale=[h + 1.0 for h in range(H)])
    kn = np.stack([(h + 1.0) * c[:, :, :128] for h in range(H)], axis=1)
    vv = np.stack([c[:, :, 256:384] for _ in range(H)], axis=1)
    ref = mla_attention(qn, qp, kn, kp, vv, S - 1, ALPHA)
    assert np.max(np.abs(mla_decode_latent(qn, qp, c, kp, w, S - 1, ALPHA) - ref)) <= 1e-12


def test_flat_scores_give_projected_latent_mean():
    """No key signal (key half zero, q_pe zero): every weight is 1/S, so the
    output of head h is its value projection of the latent mean (closed form)."""
    B, H, S = 2, 3, 11
    qn, qp, c, kp = _rand(B, H, S, 3)
    rng = np.random.default_rng(4)
    w = rng.standard_normal((H * KV_B_PER_HEAD, KV_LORA_RANK))
    for h in range(H):
        w[h * KV_B_PER_HEAD:h * KV_B_PER_HEAD + 128] = 0.0
    qp[:] = 0.0
    got = mla_decode_latent(qn, qp, c, kp, w, S - 1, ALPHA)
    for b in range(B):
        mean = c[b].mean(axis=0)
        for h in range(H):
            wv = w[h * KV_B_PER_HEAD + 128:(h + 1) * KV_B_PER_HEAD]
            assert np.max(np.abs(got[b, h, 0] - wv @ mean)) <= 1e-12


def test_absorbed_order_matches():
    """The absorbed evaluation order, written out here with einsum:
    q~ = W_k^T q_nope, scores = q~.c + q_pe.k_pe, o = W_v (sum_j p_j c_j).
    Equal to decompress-then-attend up to fp64 rounding."""
    B, H, S = 2, 4, 13
    qn, qp, c, kp = _rand(B, H, S, 5)
    rng = np.random.default_rng(6)
    w = rng.standard_normal((H * KV_B_PER_HEAD, KV_LORA_RANK)) / np.sqrt(KV_LORA_RANK)
    wr = w.reshape(H, KV_B_PER_HEAD, KV_LORA_RANK)
    wk, wv = wr[:, :128, :], wr[:, 128:, :]
    qt = np.einsum("bhd,hdr->bhr", qn[:, :, 0], wk)                      # [B,H,512]
    s = (np.einsum("bhr,bsr->bhs", qt, c) + np.einsum("bhd,bsd->bhs", qp[:, :, 0], kp[:, 0])) * ALPHA
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    olat = np.einsum("bhs,bsr->bhr", p, c)
    ref = np.einsum("hdr,bhr->bhd", wv, olat)
    got = mla_decode_latent(qn, qp, c, kp, w, S - 1, ALPHA)[:, :, 0]
    assert np.max(np.abs(got - ref)) <= 1e-10


def test_decompress_blocks_are_per_head_key_then_value():
    H = 3
    w = np.zeros((H * KV_B_PER_HEAD, KV_LORA_RANK))
    w[1 * KV_B_PER_HEAD + 5, 7] = 1.0          # head 1, key dim 5 <- latent dim 7
    w[2 * KV_B_PER_HEAD + 128 + 9, 3] = 2.0    # head 2, value dim 9 <- 2 * latent dim 3
    c = np.zeros((1, 2, KV_LORA_RANK))
    c[0, 1, 7] = 1.5
    c[0, 0, 3] = -1.0
    kn, vv = decompress_kv(c, w, H)
    assert kn.shape == (1, H, 2, 128) and vv.shape == (1, H, 2, 128)
    assert kn[0, 1, 1, 5] == 1.5 and np.count_nonzero(kn) == 1
    assert vv[0, 2, 0, 9] == -2.0 and np.count_nonzero(vv) == 1


def test_rows_variant_and_bf16_inputs():
    x = latent_random_inputs(2, 3, 20, seed=7)
    full = mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], 20, ALPHA)
    rows = [(0, 0), (1, 2), (0, 1)]
    got = mla_decode_latent_rows(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], 20,
                                 ALPHA, rows)
    for n, (b, h) in enumerate(rows):
        assert np.max(np.abs(got[n] - full[b, h, 0])) <= 1e-12


def test_shape_errors():
    x = latent_random_inputs(1, 2, 4, seed=8)
    with pytest.raises(ValueError):
        mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"][:-1], 4, ALPHA)
    with pytest.raises(ValueError):
        mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"][:, :, :500], x["k_pe"], x["w_kv_b"], 4,
                          ALPHA)
    with pytest.raises(ValueError):  # S != past_len + 1
        mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], 3, ALPHA)
