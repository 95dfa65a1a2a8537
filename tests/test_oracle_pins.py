"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test fixes the oracle against a closed form, an invariant of causal
softmax attention, a brute-force scalar evaluation that hides keys by leaving
them out of the sums (not by an additive mask), an independent library
attention routine, or a shape printed on the pages. Together they are chosen
so that a dropped term, a wrong sign or index, a transposed operand, a mask off
by one or a head-local rotary key fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (
    attention_probs,
    bf16_bits_to_f64,
    causal_mask_4d,
    mla_attention,
    mla_attention_rows,
)
from seeded_inputs import WORKLOADS, f32_to_bf16_bits, random_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ALPHA = float(np.float32(192.0 ** -0.5))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(x):
    return bf16_bits_to_f64(x)


def _rand_f64(rng, shape, scale=1.0):
    """Random inputs already on the bf16 grid, as fp64."""
    return f64(f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32)))


def _problem(B, H, T, P, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    S = P + T
    return dict(
        q_nope=_rand_f64(rng, (B, H, T, 128), scale),
        q_pe=_rand_f64(rng, (B, H, T, 64), scale),
        k_nope=_rand_f64(rng, (B, H, S, 128), scale),
        k_pe=_rand_f64(rng, (B, 1, S, 64), scale),
        v=_rand_f64(rng, (B, H, S, 128)),
    )


def _run(p, P, scale=ALPHA):
    return mla_attention(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], P, scale)


# --------------------------------------------------------------------------
# bf16 handling of inputs


def test_bf16_bits_exact_values():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0]
    got = bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)


def test_generator_rounds_to_nearest_even():
    above_tie = np.nextafter(np.float32(1.00390625), np.float32(2.0))
    x = np.array([1.0, 1.00390625, 1.01171875, above_tie, -1.00390625, 3.0e38], dtype=np.float32)
    got = f32_to_bf16_bits(x)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x7F62]


# --------------------------------------------------------------------------
# brute force: scalar loops, hidden keys simply excluded from the sums


def _brute_force(p, P, alpha):
    B, H, T, _ = p["q_nope"].shape
    out = np.zeros((B, H, T, 128))
    for b in range(B):
        for h in range(H):
            for i in range(T):
                visible = range(P + i + 1)
                z = []
                for j in visible:
                    s = math.fsum(float(p["q_nope"][b, h, i, d]) * float(p["k_nope"][b, h, j, d])
                                  for d in range(128))
                    s += math.fsum(float(p["q_pe"][b, h, i, d]) * float(p["k_pe"][b, 0, j, d])
                                   for d in range(64))
                    z.append(alpha * s)
                zmax = max(z)
                w = [math.exp(zj - zmax) for zj in z]
                tot = math.fsum(w)
                for d in range(128):
                    out[b, h, i, d] = math.fsum(w[j] * float(p["v"][b, h, j, d]) for j in visible) / tot
    return out


@pytest.mark.parametrize("B,H,T,P", [(1, 2, 4, 0), (2, 2, 3, 2), (1, 3, 1, 4)])
def test_brute_force_scalar(B, H, T, P):
    p = _problem(B, H, T, P, seed=11 + 7 * P + T)
    got = _run(p, P)
    want = _brute_force(p, P, ALPHA)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# an independent library routine: torch SDPA in fp64 on the CPU, with an
# explicit bottom-right boolean mask (its is_causal flag aligns top-left)


@pytest.mark.parametrize("B,H,T,P", [(2, 3, 5, 0), (2, 4, 7, 9), (1, 2, 1, 33)])
def test_against_torch_sdpa_fp64(B, H, T, P):
    torch = pytest.importorskip("torch")
    p = _problem(B, H, T, P, seed=5 + B + H + T + P)
    S = P + T
    q = torch.from_numpy(np.concatenate([p["q_nope"], p["q_pe"]], -1))
    k = torch.from_numpy(np.concatenate([p["k_nope"], np.broadcast_to(p["k_pe"], (B, H, S, 64))], -1))
    v = torch.from_numpy(p["v"])
    allowed = torch.arange(S)[None, :] <= (P + torch.arange(T))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=allowed, scale=ALPHA)
    np.testing.assert_allclose(_run(p, P), ref.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms


@pytest.mark.parametrize("P", [0, 3, 7])
def test_zero_query_gives_causal_prefix_mean(P):
    """All scores 0 -> uniform weights over the visible keys -> prefix means."""
    B, H, T = 2, 3, 5
    p = _problem(B, H, T, P, seed=P)
    p["q_nope"][:] = 0.0
    p["q_pe"][:] = 0.0
    got = _run(p, P)
    csum = np.cumsum(p["v"], axis=2)
    counts = P + np.arange(T) + 1
    want = csum[:, :, P:, :] / counts[None, None, :, None]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def _two_key_closed_form(alpha, s0, s1, v0, v1):
    p0 = 1.0 / (1.0 + math.exp(alpha * (s1 - s0)))
    return p0 * v0 + (1.0 - p0) * v1


@pytest.mark.parametrize("part", ["nope", "rope", "both"])
def test_two_key_closed_form(part):
    """T=1, P=1: one query against two keys; the weight of key 0 is
    1/(1+exp(alpha*(s1-s0))). The rotary key is one tensor for all heads, and
    each head has its own query scale a_h, so every head has its own weight."""
    H = 3
    rng = np.random.default_rng(3)
    q_nope = np.zeros((1, H, 1, 128))
    q_pe = np.zeros((1, H, 1, 64))
    k_nope = np.zeros((1, H, 2, 128))
    k_pe = np.zeros((1, 1, 2, 64))
    v = _rand_f64(rng, (1, H, 2, 128))
    a = [1.5, -2.0, 0.75]
    c_nope = [(0.5, 2.0), (1.0, -1.0), (3.0, 0.25)]  # per head, keys 0 and 1
    c_rope = (-1.25, 2.5)  # shared by all heads
    for h in range(H):
        if part in ("nope", "both"):
            q_nope[0, h, 0, 17] = a[h]
            k_nope[0, h, 0, 17], k_nope[0, h, 1, 17] = c_nope[h]
        if part in ("rope", "both"):
            q_pe[0, h, 0, 5] = a[h]
    if part in ("rope", "both"):
        k_pe[0, 0, 0, 5], k_pe[0, 0, 1, 5] = c_rope
    got = mla_attention(q_nope, q_pe, k_nope, k_pe, v, 1, ALPHA)
    for h in range(H):
        s0 = s1 = 0.0
        if part in ("nope", "both"):
            s0 += a[h] * c_nope[h][0]
            s1 += a[h] * c_nope[h][1]
        if part in ("rope", "both"):
            s0 += a[h] * c_rope[0]
            s1 += a[h] * c_rope[1]
        want = _two_key_closed_form(ALPHA, s0, s1, v[0, h, 0], v[0, h, 1])
        np.testing.assert_allclose(got[0, h, 0], want, rtol=0, atol=1e-14)


def test_scale_is_taken_as_fp32():
    """The scale crosses the ABI as a 32-bit float: 0.1 means fp32(0.1)."""
    q_nope = np.zeros((1, 1, 1, 128)); q_nope[0, 0, 0, 0] = 4.0
    k_nope = np.zeros((1, 1, 2, 128)); k_nope[0, 0, 1, 0] = 3.0
    v = np.zeros((1, 1, 2, 128)); v[0, 0, 0, 0] = 1.0
    got = mla_attention(q_nope, np.zeros((1, 1, 1, 64)), k_nope, np.zeros((1, 1, 2, 64)), v, 1, 0.1)
    a32 = float(np.float32(0.1))
    assert got[0, 0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(a32 * 12.0)), abs=1e-16)
    assert a32 != 0.1


def test_constant_values_reproduce_the_constant():
    B, H, T, P = 2, 3, 6, 4
    p = _problem(B, H, T, P, seed=21, scale=2.0)
    c = np.random.default_rng(1).standard_normal((B, H, 1, 128))
    p["v"] = np.broadcast_to(c, p["v"].shape).copy()
    got = _run(p, P)
    np.testing.assert_allclose(got, np.broadcast_to(c, got.shape), rtol=1e-14, atol=1e-14)


def test_one_key_row_returns_first_value():
    p = _problem(2, 3, 5, 0, seed=8)
    got = _run(p, 0)
    assert np.array_equal(got[:, :, 0, :], p["v"][:, :, 0, :])


def test_single_query_single_key_returns_value():
    p = _problem(2, 2, 1, 0, seed=9)
    assert np.array_equal(_run(p, 0), p["v"])


# --------------------------------------------------------------------------
# softmax rows and the mask


@pytest.mark.parametrize("P", [0, 5])
def test_softmax_rows(P):
    B, H, T = 2, 2, 7
    p = _problem(B, H, T, P, seed=30 + P, scale=2.0)
    probs = attention_probs(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], P, ALPHA)
    assert probs.shape == (B, H, T, P + T)
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-12)
    visible = np.arange(P + T)[None, :] <= (P + np.arange(T))[:, None]
    assert np.all(probs[..., ~visible] == 0.0)
    assert np.all(probs[..., visible] > 0.0)


def test_mask_builder_is_bottom_right_aligned():
    m = causal_mask_4d(2, 3, 2)
    assert m.shape == (2, 1, 3, 5)
    want = np.array([[0, 0, 0, -np.inf, -np.inf], [0, 0, 0, 0, -np.inf], [0, 0, 0, 0, 0]])
    assert np.array_equal(m[1, 0], want)


def test_future_keys_do_not_change_earlier_rows():
    B, H, T, P = 1, 2, 6, 3
    p = _problem(B, H, T, P, seed=40)
    base = _run(p, P)
    i0 = 2  # rows 0..i0 see keys 0..P+i0
    q = {k: v.copy() for k, v in p.items()}
    rng = np.random.default_rng(99)
    for name in ("k_nope", "k_pe", "v"):
        q[name][:, :, P + i0 + 1:, :] = rng.standard_normal(q[name][:, :, P + i0 + 1:, :].shape) * 50
    new = _run(q, P)
    assert np.array_equal(new[:, :, : i0 + 1], base[:, :, : i0 + 1])
    assert not np.allclose(new[:, :, i0 + 1:], base[:, :, i0 + 1:])


# --------------------------------------------------------------------------
# structure: heads, batches, decode, chunked prefill


def test_head_permutation_equivariance_with_shared_rotary_key():
    B, H, T, P = 2, 5, 4, 3
    p = _problem(B, H, T, P, seed=50)
    perm = np.array([3, 0, 4, 1, 2])
    q = dict(p)
    for name in ("q_nope", "q_pe", "k_nope", "v"):
        q[name] = p[name][:, perm]
    np.testing.assert_allclose(_run(q, P), _run(p, P)[:, perm], rtol=0, atol=1e-15)


def test_batch_permutation_moves_the_rotary_key_with_its_batch():
    B, H, T, P = 3, 2, 3, 2
    p = _problem(B, H, T, P, seed=51)
    perm = np.array([2, 0, 1])
    q = {k: v[perm] for k, v in p.items()}
    np.testing.assert_allclose(_run(q, P), _run(p, P)[perm], rtol=0, atol=1e-15)


def test_decode_equals_last_row_of_prefill():
    B, H, S = 2, 3, 37
    p = _problem(B, H, S, 0, seed=60)
    full = _run(p, 0)
    dec = mla_attention(p["q_nope"][:, :, -1:], p["q_pe"][:, :, -1:], p["k_nope"], p["k_pe"], p["v"],
                        S - 1, ALPHA)
    np.testing.assert_allclose(dec[:, :, 0], full[:, :, -1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("P", [1, 16, 29])
def test_chunked_prefill_equals_suffix_of_full_prefill(P):
    B, H, S = 1, 2, 40
    p = _problem(B, H, S, 0, seed=70 + P)
    full = _run(p, 0)
    chunk = mla_attention(p["q_nope"][:, :, P:], p["q_pe"][:, :, P:], p["k_nope"], p["k_pe"], p["v"],
                          P, ALPHA)
    np.testing.assert_allclose(chunk, full[:, :, P:], rtol=0, atol=1e-12)


def test_rows_variant_matches_full_oracle():
    p = random_inputs(2, 3, 9, 4, seed=3)
    full = mla_attention(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], 4, ALPHA)
    rows = [(0, 0, 0), (1, 2, 8), (0, 1, 4), (1, 2, 3), (0, 1, 5)]
    got = mla_attention_rows(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], 4, ALPHA, rows)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[b, h, i], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# shape contract (ValueError, as in the attention-core excerpt)


def test_shape_errors():
    p = _problem(1, 2, 3, 2, seed=1)
    with pytest.raises(ValueError):
        _run(p, 1)  # S = 5 != 1 + 3
    with pytest.raises(ValueError):
        mla_attention(p["q_nope"], p["q_pe"], p["k_nope"], np.concatenate([p["k_pe"]] * 2, 1), p["v"], 2, ALPHA)
    with pytest.raises(ValueError):
        mla_attention_rows(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], 2, ALPHA, [(0, 2, 0)])


def test_shapes_printed_on_the_pages():
    with open(os.path.join(GOLDEN, "page_shapes.json")) as f:
        g = json.load(f)
    d = g["decode_scores"]
    wl = WORKLOADS["decode_p1000"]
    assert (wl.B, wl.H, wl.T, wl.S, wl.past_len) == (d["B"], d["heads"], d["queries"], d["keys"], d["past_len"])
    p = _problem(1, 64, 1, 1000, seed=2)
    probs = attention_probs(p["q_nope"], p["q_pe"], p["k_nope"], p["k_pe"], p["v"], 1000, ALPHA)
    assert probs.shape == (d["B"], d["heads"], d["queries"], d["keys"])
    out = _run(p, 1000)
    assert out.shape[1:] == (g["value_mix_output"]["heads"], 1, g["value_mix_output"]["v_head_dim"])
    hd = g["head_dims"]
    from oracle import QK_NOPE_HEAD_DIM, QK_ROPE_HEAD_DIM, V_HEAD_DIM
    assert (QK_NOPE_HEAD_DIM, QK_ROPE_HEAD_DIM, V_HEAD_DIM) == (
        hd["qk_nope_head_dim"], hd["qk_rope_head_dim"], hd["v_head_dim"])
    assert all(w.H == hd["num_attention_heads"] for k, w in WORKLOADS.items() if k != "tiny_prefill")


# --------------------------------------------------------------------------
# regression fixture written by tests/golden/make_golden.py (oracle only)


def test_tiny_prefill_regression_fixture():
    path = os.path.join(GOLDEN, "tiny_prefill_oracle.npz")
    wl = WORKLOADS["tiny_prefill"]
    from seeded_inputs import host_inputs
    x = host_inputs(wl, seed=0)
    got = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], wl.past_len, wl.softmax_scale)
    ref = np.load(path, allow_pickle=False)
    for name in ("q_nope", "q_pe", "k_nope", "k_pe", "v"):
        assert np.array_equal(ref[name], x[name]), name
    np.testing.assert_allclose(got, ref["out"], rtol=0, atol=1e-13)
