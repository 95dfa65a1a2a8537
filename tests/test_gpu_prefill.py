"""GPU parity of mla_attn_prefill against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from oracle import mla_attention, mla_attention_rows
from seeded_inputs import SHARD_WORKLOADS, WORKLOADS, host_inputs, random_inputs

from _gpu_util import assert_parity, log, spread_heads, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = WORKLOADS["tiny_prefill"].softmax_scale


def _lib():
    import attention_mla_causal_amd as m
    return m


def _gpu_prefill(x, P, scale=ALPHA):
    import torch
    d = upload(x)
    out = _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, scale)
    torch.cuda.synchronize()
    return out


def _oracle(x, P, scale=ALPHA):
    return mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, scale)


def test_tiny_prefill_workload():
    wl = WORKLOADS["tiny_prefill"]
    log(f"case tiny_prefill B={wl.B} H={wl.H} T={wl.T} P={wl.past_len}")
    x = host_inputs(wl, seed=0)
    out = _gpu_prefill(x, wl.past_len, wl.softmax_scale)
    assert_parity(to_host_f64(out), _oracle(x, wl.past_len, wl.softmax_scale), "tiny_prefill")


# (B, H, T, past_len): one query; ragged tiles; several tiles with a ragged tail;
# a cache offset that is and is not a multiple of the 64-key tile; H=1 and H=64.
EDGE_SHAPES = [
    (1, 1, 1, 0),
    (1, 4, 17, 0),
    (2, 3, 127, 1),
    (1, 4, 129, 63),
    (1, 2, 130, 1000),
    (2, 1, 300, 77),
    (1, 64, 17, 0),
    (1, 2, 1, 1000),
    (1, 3, 64, 64),
    (3, 2, 257, 5),
]


@pytest.mark.parametrize("B,H,T,P", EDGE_SHAPES)
def test_edge_shapes(B, H, T, P):
    log(f"case edge B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=B * 1000 + H * 100 + T + P)
    out = _gpu_prefill(x, P)
    assert_parity(to_host_f64(out), _oracle(x, P), f"edge {B},{H},{T},{P}")


# (B, H, T, past_len) through each branch of the workgroup order, whose grid is
# a multiple of 8 (every XCD holds whole heads): tiles of uneven work (the
# causal triangle dominates) over 3, 4, 5 and 8 heads per XCD (all of them at
# once when not a multiple of four, else windows of four); near-equal tiles
# over 2 heads per XCD (head by head), 4, 8 and 12 (windows of four, one to
# three of them).
PLACEMENT_SHAPES = [
    (1, 24, 384, 0),
    (1, 32, 384, 0),
    (1, 40, 512, 0),
    (1, 64, 384, 0),
    (1, 16, 256, 1500),
    (1, 32, 256, 1500),
    (1, 64, 256, 1500),
    (2, 48, 130, 20),
]


@pytest.mark.parametrize("B,H,T,P", PLACEMENT_SHAPES)
def test_placement_branches(B, H, T, P):
    log(f"case placement B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=B * 7 + H * 5 + T * 3 + P)
    out = _gpu_prefill(x, P)
    assert_parity(to_host_f64(out), _oracle(x, P), f"placement {B},{H},{T},{P}")


@pytest.mark.parametrize("std", [2.0, 4.0])
def test_sharp_softmax(std):
    """Large logits (scaled-logit std 2 and 4): stresses the running max."""
    B, H, T, P = 1, 4, 200, 300
    log(f"case sharp std={std}")
    x = random_inputs(B, H, T, P, seed=int(std * 10), std=std)
    out = _gpu_prefill(x, P)
    assert_parity(to_host_f64(out), _oracle(x, P), f"sharp std {std}")


def test_zero_queries_give_prefix_means():
    B, H, T, P = 1, 3, 150, 70
    log("case zero queries")
    x = random_inputs(B, H, T, P, seed=4)
    x["q_nope"][:] = 0
    x["q_pe"][:] = 0
    out = to_host_f64(_gpu_prefill(x, P))
    v = np.asarray(x["v"], dtype=np.uint16)
    from oracle import bf16_bits_to_f64
    vf = bf16_bits_to_f64(v)
    want = np.cumsum(vf, axis=2)[:, :, P:, :] / (P + np.arange(T) + 1)[None, None, :, None]
    assert_parity(out, want, "zero queries")


def test_one_key_row_is_exact_and_future_keys_are_ignored():
    B, H, T = 1, 4, 200
    log("case one-key row / future keys")
    x = random_inputs(B, H, T, 0, seed=12)
    base_bits = to_host_bits(_gpu_prefill(x, 0))
    # row 0 sees only key 0: weight exactly 1, output exactly v[0] in bf16
    assert np.array_equal(base_bits[:, :, 0, :], x["v"][:, :, 0, :])
    # change every key/value after position 90: rows 0..90 must not change at all
    y = {k: v.copy() for k, v in x.items()}
    rng = np.random.default_rng(1)
    for name in ("k_nope", "k_pe", "v"):
        y[name][:, :, 91:, :] = rng.integers(0, 0x7F00, size=y[name][:, :, 91:, :].shape, dtype=np.uint16)
    new_bits = to_host_bits(_gpu_prefill(y, 0))
    assert np.array_equal(new_bits[:, :, :91], base_bits[:, :, :91])


def test_shared_rotary_key_is_read_per_batch():
    """Two batches with identical everything except k_pe must differ only via k_pe."""
    B, H, T, P = 2, 2, 40, 10
    log("case per-batch rotary key")
    x = random_inputs(B, H, T, P, seed=21)
    for name in ("q_nope", "q_pe", "k_nope", "v"):
        x[name][1] = x[name][0]
    out = to_host_f64(_gpu_prefill(x, P))
    assert_parity(out, _oracle(x, P), "per-batch k_pe")
    assert not np.allclose(out[0], out[1])


def test_deterministic_reruns():
    B, H, T, P = 1, 8, 333, 100
    log("case determinism")
    x = random_inputs(B, H, T, P, seed=2)
    a = to_host_bits(_gpu_prefill(x, P))
    b = to_host_bits(_gpu_prefill(x, P))
    assert np.array_equal(a, b)


def test_output_fully_written():
    """Every output element is written (NaN-poisoned output buffer)."""
    import torch
    B, H, T, P = 2, 3, 200, 9
    log("case poisoned output")
    x = random_inputs(B, H, T, P, seed=5)
    d = upload(x)
    out = torch.full((B, H, T, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()


def test_chunked_prefill_matches_full_prefill_suffix():
    B, H, S, P = 1, 4, 520, 333
    log("case chunked suffix")
    x = random_inputs(B, H, S, 0, seed=9)
    full = to_host_f64(_gpu_prefill(x, 0))
    y = dict(x)
    y["q_nope"] = x["q_nope"][:, :, P:].copy()
    y["q_pe"] = x["q_pe"][:, :, P:].copy()
    chunk = to_host_f64(_gpu_prefill(y, P))
    assert_parity(chunk, full[:, :, P:], "chunk vs full suffix")
    assert_parity(chunk, _oracle(y, P), "chunk vs oracle")


# (B, H, T, P): grids too small to fill the GPU, so the keys of each query
# tile split over several workgroups: several ranges, a ragged last range,
# 2..16 ranges (16, the most the merge holds per row, for the 100-query
# cases). Each query tile's visible keys are cut into the plan's number of
# near-equal ranges, so with few cached keys the first tiles see fewer key
# tiles than there are ranges and their last ranges are empty: 2 x 2560
# queries (5 ranges; tile 0 sees 4 key tiles), and 2500 queries over 60
# cached keys (a ragged last tile; tile 0 sees 6). 7 query tiles (777
# queries) give an odd count for the heavy-light pairing order.
SPLIT = [(1, 2, 256, 3840), (1, 1, 100, 5000), (2, 4, 1024, 0), (1, 3, 777, 2000), (1, 8, 129, 1023),
         (1, 1, 128, 8192), (1, 1, 100, 16000), (1, 2, 2560, 0), (1, 2, 2500, 60)]


@pytest.mark.parametrize("B,H,T,P", SPLIT)
def test_key_range_splits(B, H, T, P):
    """The split prefill against the oracle and against the unsplit kernel;
    a workspace full of NaN bits changes nothing (every partial is written)."""
    import torch
    m = _lib()
    need = m.mla_attn_prefill_workspace_bytes(B, H, T, P + T)
    log(f"case prefill split B={B} H={H} T={T} P={P} ws={need}")
    assert need > 0
    x = random_inputs(B, H, T, P, seed=B * 1000 + H * 100 + T + P)
    d = upload(x)
    args = (d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    split = m.mla_attn_prefill(*args, workspace=ws)
    whole = m.mla_attn_prefill(*args, split=False)
    fresh = m.mla_attn_prefill(*args)
    torch.cuda.synchronize()
    ref = _oracle(x, P)
    assert_parity(to_host_f64(split), ref, "split")
    assert_parity(to_host_f64(whole), ref, "unsplit")
    assert np.array_equal(to_host_bits(split), to_host_bits(fresh))
    diff = np.abs(to_host_f64(split) - to_host_f64(whole))
    assert diff.max() <= 1e-2, diff.max()


def _sample_rows(B, H, T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, H - 1, T - 1), (0, H - 1, T // 2), (B - 1, 0, min(T - 1, 127)),
            (0, 1 % H, min(T - 1, 128))}
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T))))
    return sorted(rows)


@pytest.mark.parametrize("name,std", [("causal_prefill", None), ("chunked_prefill", None),
                                      ("chunked_prefill", 2.0), ("chunked_prefill_h8", None)])
def test_full_size_workloads_sampled(name, std):
    """Full-size launch as benchmarked (and one GPU's 8-head share of the
    chunked prefill); the oracle checks sampled rows, then every query row of
    four heads spread over the head range (a head's tiles run on one XCD, in
    the order the kernel deals them)."""
    import torch
    wl = WORKLOADS[name] if name in WORKLOADS else SHARD_WORKLOADS[name]
    log(f"case full {name} std={std or wl.std} B={wl.B} H={wl.H} T={wl.T} P={wl.past_len}")
    x = host_inputs(wl, seed=0, std=std)
    out = _gpu_prefill(x, wl.past_len, wl.softmax_scale)
    rows = _sample_rows(wl.B, wl.H, wl.T, 48, seed=1)
    idx = torch.tensor([r[0] * wl.H * wl.T + r[1] * wl.T + r[2] for r in rows], device=out.device)
    got = to_host_f64(out.view(-1, 128)[idx])
    ref = mla_attention_rows(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], wl.past_len,
                             wl.softmax_scale, rows)
    assert_parity(got, ref, f"{name} sampled")
    assert torch.isfinite(out).all().item()
    for h in spread_heads(wl.H):
        ref = mla_attention(x["q_nope"][:, h:h + 1], x["q_pe"][:, h:h + 1], x["k_nope"][:, h:h + 1], x["k_pe"],
                            x["v"][:, h:h + 1], wl.past_len, wl.softmax_scale)
        assert_parity(to_host_f64(out[:, h:h + 1]), ref, f"{name} whole head {h}")


def test_split_prefill_graph_replays():
    """The key-range split path (two kernels and a workspace) captured once and
    replayed with new inputs copied in between: every replay matches the
    oracle."""
    import torch
    B, H, T, P = 1, 2, 256, 3840
    ws_bytes = _lib().mla_attn_prefill_workspace_bytes(B, H, T, P + T)
    assert ws_bytes > 0
    log(f"case split prefill graph B={B} H={H} T={T} P={P} ws={ws_bytes}")
    xs = [random_inputs(B, H, T, P, seed=70 + i) for i in range(3)]
    d = upload(xs[0])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((B, H, T, 128), dtype=torch.bfloat16, device="cuda")

    def call():
        _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA, out=out,
                                workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        for k, t in upload(x).items():
            d[k].copy_(t)
        out.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(to_host_f64(out), _oracle(x, P), f"split prefill replay {i}")


def test_empty_calls_through_the_binding():
    """Empty batches, heads or query counts are valid no-ops at every entry
    point (as torch's empty tensors): nothing is launched, shapes come back."""
    import torch
    m = _lib()
    bf = dict(dtype=torch.bfloat16, device="cuda")
    # prefill with T = 0 (S = past_len)
    q = torch.empty((1, 4, 0, 128), **bf)
    qp = torch.empty((1, 4, 0, 64), **bf)
    k = torch.zeros((1, 4, 5, 128), **bf)
    kp = torch.zeros((1, 1, 5, 64), **bf)
    out = m.mla_attn_prefill(q, qp, k, kp, k.clone(), 5, ALPHA)
    assert tuple(out.shape) == (1, 4, 0, 128)
    # decode with B = 0
    q0 = torch.empty((0, 64, 1, 128), **bf)
    out = m.mla_attn_decode(q0, torch.empty((0, 64, 1, 64), **bf), torch.empty((0, 64, 9, 128), **bf),
                            torch.empty((0, 1, 9, 64), **bf), torch.empty((0, 64, 9, 128), **bf), 8, ALPHA)
    assert tuple(out.shape) == (0, 64, 1, 128)
    # padded variable-length prefill with no query rows
    lens = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = m.mla_attn_prefill_varlen(q, qp, k, kp, k.clone(), lens, lens, ALPHA)
    assert tuple(out.shape) == (1, 4, 0, 128)
    # 2D-mask prefill with no query rows
    out = m.mla_attn_prefill_masked(q, qp, k, kp, k.clone(), torch.ones((1, 5), dtype=torch.uint8, device="cuda"),
                                    5, ALPHA)
    assert tuple(out.shape) == (1, 4, 0, 128)
    torch.cuda.synchronize()
