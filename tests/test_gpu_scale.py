"""Any finite softmax_scale, through the C ABI, on every attention path.

The pages multiply the scores by softmax_scale without stating its value
("Similarities" page, "Query-key similarity"), so the library takes any finite
scale. A zero scale gives every visible key the same weight: the output is
the mean of the visible values, a closed form computed here with cumulative
sums, not with the oracle. A negative scale is checked against the fp64
oracle, which applies the scale as written.
"""

import numpy as np
import pytest

from oracle import (KIMI_K2_ROPE, apply_rope, bf16_bits_to_f64, mla_attention, mla_attention_masked,
                    mla_decode_latent, mla_decode_paged, mla_decode_varlen, mla_prefill_varlen,
                    rope_cos_sin, rope_positions)
from seeded_inputs import (latent_random_inputs, left_pad_mask, paged_host_inputs, paged_layout,
                           random_inputs)

from _gpu_util import assert_parity, log, to_host_f64, upload

pytestmark = pytest.mark.gpu

NEG = -float(np.float32(192.0 ** -0.5))


def _m():
    import attention_mla_causal_amd as m
    return m


def _sync():
    import torch
    torch.cuda.synchronize()


def _prefix_means(v_bits, past_len):
    """Zero scale: query i sees keys 0..past_len+i with equal weight, so its
    output is the mean of those value rows."""
    v = bf16_bits_to_f64(v_bits)                      # [B, H, S, 128]
    c = np.cumsum(v, axis=2)
    T = v.shape[2] - past_len
    n = np.arange(past_len + 1, past_len + T + 1, dtype=np.float64)[None, None, :, None]
    return c[:, :, past_len:] / n


# (B, H, T, P): one workgroup per query tile (64 heads), and a small grid that
# the prefill splits over key ranges (merged by log-sum-exp in a second kernel)
PREFILL = [(1, 64, 300, 200), (1, 4, 700, 1500)]


@pytest.mark.parametrize("B,H,T,P", PREFILL)
def test_prefill_zero_scale_gives_prefix_means(B, H, T, P):
    log(f"case prefill scale 0 B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=500 + H)
    d = upload(x)
    out = _m().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, 0.0)
    _sync()
    assert_parity(to_host_f64(out), _prefix_means(x["v"], P), "prefill scale 0")


@pytest.mark.parametrize("B,H,T,P", PREFILL)
def test_prefill_negative_scale(B, H, T, P):
    log(f"case prefill scale {NEG:.4f} B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=600 + H)
    d = upload(x)
    out = _m().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, NEG)
    _sync()
    ref = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, NEG)
    assert_parity(to_host_f64(out), ref, "prefill negative scale")


def test_prefill_negative_scale_is_positive_scale_with_negated_query():
    """scale * q.k = (-scale) * (-q).k: the negative-scale call and the
    positive-scale call on the negated query agree bit for bit (flipping bf16
    sign bits is exact)."""
    import torch
    B, H, T, P = 1, 8, 256, 100
    log("case prefill scale sign symmetry")
    x = random_inputs(B, H, T, P, seed=61)
    d = upload(x)
    a = _m().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, NEG, split=False)
    b = _m().mla_attn_prefill(-d["q_nope"], -d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, -NEG,
                              split=False)
    _sync()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# (B, H, P): splits merged inside the kernel, and by the merge kernel (H = 5)
DECODE = [(1, 64, 1000), (1, 5, 1999), (32, 16, 300)]


@pytest.mark.parametrize("B,H,P", DECODE)
def test_decode_zero_and_negative_scale(B, H, P):
    log(f"case decode scales B={B} H={H} P={P}")
    x = random_inputs(B, H, 1, P, seed=700 + H)
    d = upload(x)
    z = _m().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, 0.0)
    n = _m().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, NEG)
    _sync()
    assert_parity(to_host_f64(z), _prefix_means(x["v"], P), "decode scale 0")
    ref = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, NEG)
    assert_parity(to_host_f64(n), ref, "decode negative scale")


def test_decode_rope_negative_scale():
    import torch
    B, H, P = 1, 16, 1500
    S = P + 1
    log(f"case rotary decode negative scale B={B} H={H} P={P}")
    x = random_inputs(B, H, 1, P, seed=71)
    d = upload(x)
    tab = _m().mla_rope_table(S, device=torch.device("cuda"))
    out = _m().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, NEG,
                               rope_table=tab)
    _sync()
    cos, sin = rope_cos_sin(S, **KIMI_K2_ROPE)
    q_rot = apply_rope(bf16_bits_to_f64(x["q_pe"]), rope_positions(B, 1, past_len=P), cos, sin)
    ref = mla_attention(x["q_nope"], q_rot, x["k_nope"], x["k_pe"], x["v"], P, NEG)
    assert_parity(to_host_f64(out), ref, "rotary decode negative scale")


@pytest.mark.parametrize("scale", [0.0, NEG])
def test_varlen_decode_scales(scale):
    import torch
    B, H, cap = 4, 16, 1100
    lens = np.array([1001, 1, 0, 517], dtype=np.int32)
    log(f"case varlen decode scale {scale}")
    x = random_inputs(B, H, 1, cap - 1, seed=81)
    d = upload(x)
    sl = torch.as_tensor(lens, device="cuda")
    out = _m().mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], sl, cap, scale)
    _sync()
    ref = mla_decode_varlen(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], lens, scale)
    assert_parity(to_host_f64(out), ref, f"varlen decode scale {scale}")


@pytest.mark.parametrize("scale", [0.0, NEG])
def test_paged_decode_with_append_scales(scale):
    import torch
    lens = np.array([1001, 1, 129, 64], dtype=np.int32)
    H, bs = 16, 64
    log(f"case paged decode scale {scale}")
    table, N = paged_layout(lens, bs, seed=3)
    x = paged_host_inputs(len(lens), H, N, bs, seed=91)
    d = upload(x)
    tb = torch.as_tensor(table, device="cuda")
    sl = torch.as_tensor(lens, device="cuda")
    out = _m().mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"], d["v_pages"],
                                     tb, sl, int(lens.max()), scale,
                                     new=(d["k_nope_new"], d["k_pe_new"], d["v_new"]))
    _sync()
    ref, _ = mla_decode_paged(x["q_nope"], x["q_pe"], x["k_nope_pages"], x["k_pe_pages"], x["v_pages"],
                              table, lens, scale, new=(x["k_nope_new"], x["k_pe_new"], x["v_new"]))
    assert_parity(to_host_f64(out), ref, f"paged decode scale {scale}")


@pytest.mark.parametrize("scale", [0.0, NEG])
def test_masked_paths_scales(scale):
    import torch
    B, H, T, P = 3, 8, 200, 100
    S = P + T
    pads = np.array([0, 37, 250])
    log(f"case masked prefill and decode scale {scale}")
    mask_np = left_pad_mask(S, pads)
    mask = torch.as_tensor(mask_np, device="cuda")
    x = random_inputs(B, H, T, P, seed=101)
    d = upload(x)
    out = _m().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], mask, P, scale)
    _sync()
    ref = mla_attention_masked(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], mask_np, P, scale)
    assert_parity(to_host_f64(out), ref, f"masked prefill scale {scale}")
    xd = random_inputs(B, H, 1, S - 1, seed=102)
    dd = upload(xd)
    od = _m().mla_attn_decode_masked(dd["q_nope"], dd["q_pe"], dd["k_nope"], dd["k_pe"], dd["v"], mask,
                                     S - 1, scale)
    _sync()
    refd = mla_attention_masked(xd["q_nope"], xd["q_pe"], xd["k_nope"], xd["k_pe"], xd["v"], mask_np,
                                S - 1, scale)
    assert_parity(to_host_f64(od), refd, f"masked decode scale {scale}")


@pytest.mark.parametrize("scale", [0.0, NEG])
def test_varlen_prefill_scales(scale):
    import torch
    B, H, Tmax, Smax = 3, 8, 300, 900
    q_lens = np.array([300, 1, 129], dtype=np.int32)
    past = np.array([600, 0, 40], dtype=np.int32)
    log(f"case varlen prefill scale {scale}")
    x = random_inputs(B, H, Tmax, Smax - Tmax, seed=111)
    d = upload(x)
    out = _m().mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                       torch.as_tensor(q_lens, device="cuda"),
                                       torch.as_tensor(past, device="cuda"), scale)
    _sync()
    ref = mla_prefill_varlen(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], q_lens, past, scale)
    assert_parity(to_host_f64(out), ref, f"varlen prefill scale {scale}")


@pytest.mark.parametrize("scale", [0.0, NEG])
def test_latent_decode_scales(scale):
    B, H, P = 2, 64, 1000
    log(f"case latent decode scale {scale}")
    x = latent_random_inputs(B, H, P, seed=121)
    d = upload(x)
    out = _m().mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"], P, scale)
    _sync()
    ref = mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], P, scale)
    assert_parity(to_host_f64(out), ref, f"latent decode scale {scale}")
