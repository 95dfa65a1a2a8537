"""GPU parity of mla_attn_decode_latent (decode over the compressed cache)
against the fp64 oracle that decompresses keys and values, through the C ABI."""

import numpy as np
import pytest

from oracle import mla_decode_latent, mla_decode_latent_rows
from seeded_inputs import LATENT_WORKLOADS, latent_device_inputs, latent_host_inputs, latent_random_inputs

from _gpu_util import assert_parity, log, spread_pairs, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = LATENT_WORKLOADS["latent_decode_p1000"].softmax_scale


def _lib():
    import attention_mla_causal_amd as m
    return m


def _gpu(d, P, out=None, workspace=None):
    import torch
    o = _lib().mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"], P,
                                      ALPHA, out=out, workspace=workspace)
    torch.cuda.synchronize()
    return o


def _oracle(x, P):
    return mla_decode_latent(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], P, ALPHA)


def test_latent_decode_as_on_the_pages():
    wl = LATENT_WORKLOADS["latent_decode_p1000"]
    log(f"case latent_decode_p1000 B={wl.B} H={wl.H} S={wl.S}")
    x = latent_host_inputs(wl, seed=0)
    out = _gpu(upload(x), wl.past_len)
    assert_parity(to_host_f64(out), _oracle(x, wl.past_len), "latent decode p1000")


# (B, H, past_len): one key; one key short of a tile, a full tile, one past it;
# head counts that fill 1..4 waves, and ones that leave a wave part-filled
# (8 = one GPU's share of 64 heads over 8 GPUs, 1, 20, 63); several key
# splits with a ragged last tile. With more than 48 heads and few sequences x
# tiles, each attention workgroup serves one group of 16 heads (the last
# group part-filled at 63); 8 sequences take the placement that keeps a
# sequence's splits and head groups on one XCD. From five sequences on, the
# absorb stages query and output rows through LDS: 5 (the first such batch)
# and 17 (a second group of 16 holding one sequence). More sequences than
# CUs: 300 (all-heads workgroups, one split each, a part-filled last group of
# eight in the merge) and 264 x 64 heads (one head group per workgroup, 1056
# workgroups).
EDGE = [(1, 16, 0), (1, 64, 30), (2, 32, 31), (1, 48, 32), (3, 64, 777), (2, 16, 4095), (4, 64, 2000),
        (2, 8, 500), (3, 1, 40), (1, 20, 63), (1, 63, 1000), (8, 64, 1000), (1, 64, 0), (5, 64, 40),
        (17, 8, 100), (300, 8, 40), (264, 64, 31)]


@pytest.mark.parametrize("B,H,P", EDGE)
def test_latent_decode_edge_shapes(B, H, P):
    need = _lib().mla_attn_decode_latent_workspace_bytes(B, H, P + 1)
    log(f"case latent edge B={B} H={H} P={P} ws={need}")
    x = latent_random_inputs(B, H, P, seed=B * 11 + H + P)
    out = _gpu(upload(x), P)
    assert_parity(to_host_f64(out), _oracle(x, P), f"latent {B},{H},{P}")


def test_latent_workspace_garbage_and_determinism():
    import torch
    B, H, P = 2, 64, 1500
    x = latent_random_inputs(B, H, P, seed=9)
    d = upload(x)
    need = _lib().mla_attn_decode_latent_workspace_bytes(B, H, P + 1)
    log(f"case latent workspace garbage need={need}")
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    first = None
    for it in range(3):
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        _gpu(d, P, out=out, workspace=ws)
        bits = to_host_bits(out)
        if first is None:
            first = bits
            assert_parity(to_host_f64(out), _oracle(x, P), "latent workspace first call")
        assert np.array_equal(bits, first), f"call {it} differs"
        ws.fill_(0xA5)


def test_latent_batched_decode_full_size_sampled():
    """B=32, H=64, S=8192 with inputs drawn on the device; 64 (b, h) rows
    spread over the batch and heads against the oracle (which decompresses one
    head at a time)."""
    import torch
    wl = LATENT_WORKLOADS["latent_batched_decode"]
    log(f"case latent_batched_decode B={wl.B} H={wl.H} S={wl.S}")
    d = latent_device_inputs(wl, "cuda", seed=0)
    out = _gpu(d, wl.past_len)
    assert torch.isfinite(out).all().item()
    picks = sorted(spread_pairs(wl.B, wl.H, 64, seed=1))
    w = to_host_bits(d["w_kv_b"])
    got, ref = [], []
    for b, h in picks:
        xs = {"q_nope": to_host_bits(d["q_nope"][b:b + 1, h:h + 1]),
              "q_pe": to_host_bits(d["q_pe"][b:b + 1, h:h + 1]),
              "c_kv": to_host_bits(d["c_kv"][b:b + 1]),
              "k_pe": to_host_bits(d["k_pe"][b:b + 1])}
        wh = np.zeros((256, 512), dtype=np.uint16)
        wh[:] = w[256 * h:256 * h + 256]
        ref.append(mla_decode_latent_rows(xs["q_nope"], xs["q_pe"], xs["c_kv"], xs["k_pe"], wh,
                                          wl.past_len, ALPHA, [(0, 0)])[0])
        got.append(to_host_f64(out[b, h, 0]))
    assert_parity(np.stack(got), np.stack(ref), "latent batched decode sampled")


def _times(bits, k):
    """bf16 values times k (a power of two: exact)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(k)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_latent_sharp_softmax():
    """Queries scaled by 2: sharper weights, so the running maximum moves late
    and the splits' maxima differ. (Sharper still, bf16 arithmetic itself
    leaves the bar against the fp64 oracle: with the queries scaled by 8, the
    pages' own order of operations, keys and values decompressed to bf16, is
    off by 0.032 at worst on these inputs, and rounding only the absorbed
    query to bf16, as this path does, by 0.039; by 4, both sit at the bar.)"""
    B, H, P = 2, 64, 1200
    x = latent_random_inputs(B, H, P, seed=77)
    x["q_nope"] = _times(x["q_nope"], 2)
    x["q_pe"] = _times(x["q_pe"], 2)
    log(f"case latent sharp B={B} H={H} P={P}")
    out = _gpu(upload(x), P)
    assert_parity(to_host_f64(out), _oracle(x, P), "latent sharp softmax")


@pytest.mark.parametrize("B,H,P", [(3, 64, 777), (8, 64, 4095)])
def test_latent_graph_replays_with_new_inputs(B, H, P):
    """The three launches captured once and replayed after new inputs are
    copied into the captured buffers: every replay equals an eager call on the
    same inputs bit for bit, with eager work and synchronisations between
    replays (3 sequences take the one-head-group workgroups, 8 x 4096 keys the
    all-heads ones)."""
    import torch
    m = _lib()
    need = m.mla_attn_decode_latent_workspace_bytes(B, H, P + 1)
    log(f"case latent graph B={B} H={H} P={P} ws={need}")
    sets = [upload(latent_random_inputs(B, H, P, seed=300 + i)) for i in range(3)]
    d = {k: v.clone() for k, v in sets[0].items()}
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _gpu(d, P, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.mla_attn_decode_latent(d["q_nope"], d["q_pe"], d["c_kv"], d["k_pe"], d["w_kv_b"], P, ALPHA,
                                 out=out, workspace=ws)
    for i in (1, 2, 0, 1):
        for k in d:
            d[k].copy_(sets[i][k])
        g.replay()
        torch.cuda.synchronize()
        got = to_host_bits(out)
        ref = to_host_bits(_gpu(sets[i], P))
        assert np.array_equal(got, ref), f"replay with set {i} differs from the eager call"
    x = latent_random_inputs(B, H, P, seed=301)
    if B * H <= 192:
        assert_parity(to_host_f64(out), _oracle(x, P), "latent graph replay")
    else:
        picks = sorted(spread_pairs(B, H, 16, seed=2))
        ref = mla_decode_latent_rows(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_kv_b"], P, ALPHA, picks)
        assert_parity(np.stack([to_host_f64(out[b, h, 0]) for b, h in picks]), ref, "latent graph replay rows")


@pytest.mark.parametrize("B,P", [(4, 8191), (12, 4095)])
def test_latent_plan_boundary_sampled(B, P):
    """Sequences x key tiles on either side of the switch between the two
    attention plans: 4 x 8192 keys (1024 tiles: one head group per
    workgroup) and 12 x 4096 (1536: all heads, 21 splits of 196 keys rounded
    to whole tiles, so the grid stays within one workgroup per CU). Inputs
    drawn on the device, 24 (b, h) rows against the oracle."""
    import torch
    from seeded_inputs import LatentWorkload
    H = 64
    wl = LatentWorkload("boundary", B, H, P)
    log(f"case latent plan boundary B={B} H={H} S={P + 1}")
    d = latent_device_inputs(wl, "cuda", seed=B)
    out = _gpu(d, P)
    assert torch.isfinite(out).all().item()
    picks = sorted(spread_pairs(B, H, 24, seed=3))
    w = to_host_bits(d["w_kv_b"])
    x = {k: to_host_bits(d[k]) for k in ("q_nope", "q_pe", "c_kv", "k_pe")}
    ref = mla_decode_latent_rows(x["q_nope"], x["q_pe"], x["c_kv"], x["k_pe"], w, P, ALPHA, picks)
    assert_parity(np.stack([to_host_f64(out[b, h, 0]) for b, h in picks]), ref, f"latent boundary B={B}")
