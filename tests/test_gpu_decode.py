"""GPU parity of mla_attn_decode against the fp64 oracle (through the C ABI)."""

import numpy as np
import pytest

from oracle import mla_attention
from seeded_inputs import SHARD_WORKLOADS, WORKLOADS, device_inputs, host_inputs, random_inputs

from _gpu_util import assert_parity, log, spread_pairs, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = WORKLOADS["decode_p1000"].softmax_scale


def _lib():
    import attention_mla_causal_amd as m
    return m


def _gpu_decode(d, P, scale=ALPHA, out=None, workspace=None):
    import torch
    if out is None:  # NaN first, so a row the kernel never writes fails the parity check
        B, H = d["q_nope"].shape[:2]
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = _lib().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, scale,
                               out=out, workspace=workspace)
    torch.cuda.synchronize()
    return o


def _oracle(x, P, scale=ALPHA):
    return mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P, scale)


def test_decode_as_on_the_pages():
    wl = WORKLOADS["decode_p1000"]
    log(f"case decode_p1000 B={wl.B} H={wl.H} P={wl.past_len}")
    x = host_inputs(wl, seed=0)
    out = _gpu_decode(upload(x), wl.past_len, wl.softmax_scale)
    assert_parity(to_host_f64(out), _oracle(x, wl.past_len, wl.softmax_scale), "decode_p1000")


# (B, H, past_len): a single key; key counts below, at and above a 64-key trip;
# many splits with a ragged last split; B*H large enough for one split.
EDGE = [(1, 1, 0), (1, 4, 62), (2, 3, 63), (1, 2, 64), (3, 5, 4095), (1, 1, 100000),
        (2, 64, 777), (8, 64, 1500)]


@pytest.mark.parametrize("B,H,P", EDGE)
def test_decode_edge_shapes(B, H, P):
    log(f"case decode edge B={B} H={H} P={P} ws={_lib().mla_attn_decode_workspace_bytes(B, H, P + 1)}")
    x = random_inputs(B, H, 1, P, seed=B * 7 + H * 3 + P)
    out = _gpu_decode(upload(x), P)
    assert_parity(to_host_f64(out), _oracle(x, P), f"decode {B},{H},{P}")


def test_decode_sharp_softmax():
    B, H, P = 1, 8, 3000
    log("case decode sharp")
    x = random_inputs(B, H, 1, P, seed=77, std=2.0)
    out = _gpu_decode(upload(x), P)
    assert_parity(to_host_f64(out), _oracle(x, P), "decode sharp")


def test_decode_equals_last_row_of_prefill():
    B, H, S = 2, 4, 700
    log("case decode == last prefill row")
    x = random_inputs(B, H, S, 0, seed=31)
    d = upload(x)
    import torch
    pre = _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], 0, ALPHA)
    dq = dict(d)
    dq["q_nope"] = d["q_nope"][:, :, -1:].contiguous()
    dq["q_pe"] = d["q_pe"][:, :, -1:].contiguous()
    dec = _gpu_decode(dq, S - 1)
    torch.cuda.synchronize()
    assert_parity(to_host_f64(dec)[:, :, 0], to_host_f64(pre)[:, :, -1], "decode vs prefill last row")
    assert_parity(to_host_f64(dec)[:, :, 0], _oracle(x, 0)[:, :, -1], "decode vs oracle")


def test_workspace_contents_do_not_matter():
    """The workspace is scratch: garbage (NaN bytes) on entry, reuse across calls."""
    import torch
    B, H, P = 1, 16, 2999
    x = random_inputs(B, H, 1, P, seed=8)
    d = upload(x)
    need = _lib().mla_attn_decode_workspace_bytes(B, H, P + 1)
    log(f"case workspace scratch need={need}")
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ref = _oracle(x, P)
    first = None
    for it in range(3):
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        _gpu_decode(d, P, out=out, workspace=ws)
        bits = to_host_bits(out)
        if first is None:
            first = bits
            assert_parity(to_host_f64(out), ref, "workspace first call")
        assert np.array_equal(bits, first), f"call {it} differs"
        ws.fill_(0xFF)


def test_back_to_back_calls_share_one_workspace():
    """Calls queued back to back on one stream reuse one workspace without
    clearing it. At this shape every split of a head runs on one XCD and the
    split kernel merges the partials itself; each call's completion flags carry
    a fresh tag, so no call may merge a partial or flag left by the previous one."""
    import torch
    B, H, P = 1, 64, 1000
    need = _lib().mla_attn_decode_workspace_bytes(B, H, P + 1)
    log(f"case back-to-back decode calls need={need}")
    xa = random_inputs(B, H, 1, P, seed=101)
    xb = random_inputs(B, H, 1, P, seed=202)
    da, db = upload(xa), upload(xb)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    outs = []
    for d in (da, db, da, db, da):
        # NaN first: a (b, h) whose splits never merge would leave it there
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        _lib().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA,
                               out=out, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    bits = [to_host_bits(o) for o in outs]
    assert_parity(to_host_f64(outs[0]), _oracle(xa, P), "first call")
    assert_parity(to_host_f64(outs[1]), _oracle(xb, P), "second call")
    assert np.array_equal(bits[0], bits[2]) and np.array_equal(bits[0], bits[4])
    assert np.array_equal(bits[1], bits[3])


@pytest.mark.parametrize("B,H,P", [(1, 64, 1000), (1, 5, 1999)])
def test_graph_replays_with_new_inputs(B, H, P):
    """A captured decode replayed after its inputs change (copied in between
    replays, outside the graph) matches an eager call every time: the graph
    repeats the captured completion tag, so the in-kernel merge must not see
    flags left by the replay before (first shape: merged in the split kernel;
    second: by the merge kernel)."""
    import torch
    log(f"case decode graph replays B={B} H={H} P={P}")
    m = _lib()
    xs = [random_inputs(B, H, 1, P, seed=300 + i) for i in range(3)]
    ds = [upload(x) for x in xs]
    d = {k: v.clone() for k, v in ds[0].items()}
    out = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(m.mla_attn_decode_workspace_bytes(B, H, P + 1), 16), dtype=torch.uint8,
                     device="cuda")

    def call():
        m.mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA,
                          out=out, workspace=ws)

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
    for i in (1, 2, 0, 1, 2):
        for k in d:
            d[k].copy_(ds[i][k])
        out.fill_(float("nan"))  # a (b, h) the replay does not merge keeps its NaN
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = to_host_bits(out).copy()
        assert np.isfinite(to_host_f64(out)).all(), f"replay with input set {i} left rows unwritten"
        fresh = torch.full_like(out, float("nan"))
        eager = to_host_bits(_gpu_decode(ds[i], P, out=fresh))
        assert np.array_equal(replayed, eager), f"replay with input set {i}"
    assert_parity(to_host_f64(out), _oracle(xs[2], P), "decode graph replay")


def test_decode_determinism():
    B, H, P = 1, 4, 1234
    log("case decode determinism")
    x = random_inputs(B, H, 1, P, seed=10)
    d = upload(x)
    a = to_host_bits(_gpu_decode(d, P))
    b = to_host_bits(_gpu_decode(d, P))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["batched_decode", "batched_decode_h8"])
def test_batched_decode_full_size_sampled(name):
    """The full batched decode (B=32, H=64, S=8192; 8.6 GB of keys and values;
    and one GPU's 8-head share of it), inputs drawn on the device; the oracle
    checks 64 (b, h) rows spread over both XCD placements of the pairs."""
    import torch
    wl = WORKLOADS[name] if name in WORKLOADS else SHARD_WORKLOADS[name]
    log(f"case batched_decode B={wl.B} H={wl.H} P={wl.past_len}")
    d = device_inputs(wl, "cuda", seed=0)
    out = _gpu_decode(d, wl.past_len, wl.softmax_scale)
    assert torch.isfinite(out).all().item()
    got, ref = [], []
    for b, h in spread_pairs(wl.B, wl.H, 64):
        xs = {
            "q_nope": to_host_bits(d["q_nope"][b:b + 1, h:h + 1]),
            "q_pe": to_host_bits(d["q_pe"][b:b + 1, h:h + 1]),
            "k_nope": to_host_bits(d["k_nope"][b:b + 1, h:h + 1]),
            "k_pe": to_host_bits(d["k_pe"][b:b + 1]),
            "v": to_host_bits(d["v"][b:b + 1, h:h + 1]),
        }
        ref.append(_oracle(xs, wl.past_len, wl.softmax_scale)[0, 0, 0])
        got.append(to_host_f64(out[b, h, 0]))
    assert_parity(np.stack(got), np.stack(ref), "batched_decode sampled")


def test_concurrent_calls_on_two_streams():
    """Two decodes (each with its own workspace) and a prefill enqueued on two
    streams at once: the library keeps no state between calls beyond the
    workspaces, so each result matches the oracle."""
    import torch
    xa = random_inputs(1, 64, 1, 1500, seed=61)
    xb = random_inputs(2, 16, 1, 700, seed=62)
    xp = random_inputs(1, 8, 200, 300, seed=63)
    da, db, dp = upload(xa), upload(xb), upload(xp)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    wa = torch.empty(max(_lib().mla_attn_decode_workspace_bytes(1, 64, 1501), 16), dtype=torch.uint8,
                     device="cuda")
    wb = torch.empty(max(_lib().mla_attn_decode_workspace_bytes(2, 16, 701), 16), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        oa = _lib().mla_attn_decode(da["q_nope"], da["q_pe"], da["k_nope"], da["k_pe"], da["v"], 1500, ALPHA,
                                    workspace=wa)
        op = _lib().mla_attn_prefill(dp["q_nope"], dp["q_pe"], dp["k_nope"], dp["k_pe"], dp["v"], 300, ALPHA)
    with torch.cuda.stream(sb):
        ob = _lib().mla_attn_decode(db["q_nope"], db["q_pe"], db["k_nope"], db["k_pe"], db["v"], 700, ALPHA,
                                    workspace=wb)
    torch.cuda.synchronize()
    log("case two streams")
    assert_parity(to_host_f64(oa), _oracle(xa, 1500), "stream a decode")
    assert_parity(to_host_f64(ob), _oracle(xb, 700), "stream b decode")
    assert_parity(to_host_f64(op), mla_attention(xp["q_nope"], xp["q_pe"], xp["k_nope"], xp["k_pe"],
                                                 xp["v"], 300, ALPHA), "stream a prefill")


def test_many_sequences_and_heads():
    """B*H = 16384 (b, h) pairs of 64 keys: a grid far larger than the GPU."""
    B, H, P = 256, 64, 63
    log(f"case decode many B={B} H={H} P={P}")
    x = random_inputs(B, H, 1, P, seed=64)
    out = _gpu_decode(upload(x), P)
    assert_parity(to_host_f64(out), _oracle(x, P), "decode many sequences")
