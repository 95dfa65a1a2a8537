"""Seeded random shapes through the prefill, decode and latent-cache decode
entry points against the fp64 oracle. The shapes come from a fixed generator,
so every run draws the same cases; they land on head counts, query counts,
cache lengths and batch sizes between the hand-picked edge cases (partial
waves, ragged tiles and splits at arbitrary offsets)."""

import numpy as np
import pytest

from oracle import mla_attention, mla_decode_latent
from seeded_inputs import WORKLOADS, latent_random_inputs, random_inputs

from _gpu_util import assert_parity, log, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = WORKLOADS["tiny_prefill"].softmax_scale


def _draw(seed, n, ranges):
    g = np.random.default_rng(seed)
    return [tuple(int(g.integers(lo, hi + 1)) for lo, hi in ranges) for _ in range(n)]


# (B, H, T, past_len)
PREFILL = _draw(2026, 8, [(1, 3), (1, 64), (1, 400), (0, 1500)])
# (B, H, past_len)
DECODE = _draw(2027, 8, [(1, 8), (1, 64), (0, 6000)])
LATENT = _draw(2028, 6, [(1, 6), (1, 64), (0, 1500)])


def _lib():
    import attention_mla_causal_amd as m
    return m


@pytest.mark.parametrize("B,H,T,P", PREFILL)
def test_prefill_random_shape(B, H, T, P):
    import torch
    log(f"case random prefill B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=B * 7 + H * 11 + T * 13 + P)
    d = upload(x)
    out = _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA)
    torch.cuda.synchronize()
    ref = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, ALPHA)
    assert_parity(to_host_f64(out), ref, f"random prefill {B},{H},{T},{P}")


@pytest.mark.parametrize("B,H,P", DECODE)
def test_decode_random_shape(B, H, P):
    import torch
    log(f"case random decode B={B} H={H} P={P}")
    x = random_inputs(B, H, 1, P, seed=B * 5 + H * 3 + P)
    d = upload(x)
    out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    _lib().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA, out=out)
    torch.cuda.synchronize()
    ref = mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, ALPHA)
    assert_parity(to_host_f64(out), ref, f"random decode {B},{H},{P}")


@pytest.mark.parametrize("B,H,P", LATENT)
def test_latent_random_shape(B, H, P):
    import torch
    log(f"case random latent B={B} H={H} P={P}")
    x = latent_random_inputs(B, H, P, seed=B * 17 + H + P)
    d = upload(x)
    out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    _lib().mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"], P, ALPHA, out=out)
    torch.cuda.synchronize()
    ref = mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], P, ALPHA)
    assert_parity(to_host_f64(out), ref, f"random latent {B},{H},{P}")
