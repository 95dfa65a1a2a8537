"""GPU parity of mla_attn_prefill_masked and mla_attn_decode_masked (the
attention core under the caller's 2D padding mask) against the fp64 oracle,
through the C ABI."""

import numpy as np
import pytest

from oracle import mla_attention_masked
from seeded_inputs import random_inputs

from _gpu_util import assert_parity, log, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))
NAN_BF16 = np.uint16(0x7FC0)


def _lib():
    import attention_mla_causal_amd as m
    return m


def _dev_mask(mask):
    import torch
    return torch.as_tensor(np.ascontiguousarray(mask, dtype=np.uint8), device="cuda")


BIG_BF16 = np.uint16(0x46EA)   # 29952.0


def _with_nan_hidden(x, mask, v_fill=NAN_BF16):
    """Hidden keys' key rows hold NaN and their value rows v_fill: a hidden
    score that survived, or a hidden value that met a nonzero weight, would
    show. The decode clears hidden value rows, so NaN is fair there; the
    prefill's value contraction meets them with weight 0, so its inputs must
    be finite (as every input) and its tests fill them with a large value."""
    hidden = np.asarray(mask) == 0
    for b in range(hidden.shape[0]):
        x["k_nope"][b][:, hidden[b]] = NAN_BF16
        x["k_pe"][b][:, hidden[b]] = NAN_BF16
        x["v"][b][:, hidden[b]] = v_fill
    return x


def _prefill(x, mask, P):
    import torch
    d = upload(x)
    out = _lib().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                         _dev_mask(mask), P, ALPHA)
    torch.cuda.synchronize()
    return out


def _decode(x, mask, P):
    import torch
    d = upload(x)
    out = _lib().mla_attn_decode_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                        _dev_mask(mask), P, ALPHA)
    torch.cuda.synchronize()
    return out


def _oracle(x, mask, P):
    return mla_attention_masked(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], mask, P, ALPHA)


def _left_pad_mask(S, pads):
    return (np.arange(S)[None, :] >= np.asarray(pads)[:, None]).astype(np.uint8)


# (B, H, T, P, left pads per sequence): pads inside the cache, pads reaching
# into the new queries (their first rows see nothing and give 0), no pad, a
# whole sequence of padding; several query tiles with a ragged tail. The
# (batch, head) groups take each branch of the workgroup order: 12 and 4
# (not a multiple of 8: index order), 24 (a multiple of 8 but not of 32: one
# group at a time per XCD), 64 (windows of four groups per XCD).
PREFILL_LEFT = [
    (3, 4, 200, 77, [0, 40, 150]),
    (2, 2, 130, 0, [5, 130]),
    (1, 64, 33, 100, [99]),
    (3, 8, 300, 60, [0, 200, 5]),
]


@pytest.mark.parametrize("B,H,T,P,pads", PREFILL_LEFT)
def test_prefill_left_padding(B, H, T, P, pads):
    log(f"case prefill masked left B={B} H={H} T={T} P={P} pads={pads}")
    S = P + T
    mask = _left_pad_mask(S, pads)
    x = _with_nan_hidden(random_inputs(B, H, T, P, seed=B + H + T + P), mask, BIG_BF16)
    out = _prefill(x, mask, P)
    ref = _oracle(x, mask, P)
    bits = to_host_bits(out)
    for b in range(B):
        dead = max(0, pads[b] - P)          # query rows still inside the padding
        assert not np.any(bits[b, :, :dead]), b
    assert_parity(to_host_f64(out), ref, "prefill masked left")


@pytest.mark.parametrize("density", [0.9, 0.5, 0.1])
def test_prefill_random_masks(density):
    B, H, T, P = 2, 3, 150, 300
    S = P + T
    g = np.random.default_rng(int(density * 100))
    mask = (g.random((B, S)) < density).astype(np.uint8)
    mask[:, :64] = 1 if density == 0.9 else mask[:, :64]   # whole tiles kept and mixed ones
    log(f"case prefill masked random density={density} kept={int(mask.sum())}/{mask.size}")
    x = _with_nan_hidden(random_inputs(B, H, T, P, seed=5), mask, BIG_BF16)
    out = _prefill(x, mask, P)
    assert_parity(to_host_f64(out), _oracle(x, mask, P), f"prefill masked random {density}")


def test_prefill_all_ones_equals_dense():
    import torch
    B, H, T, P = 1, 8, 257, 64
    log(f"case prefill masked = dense B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=9)
    d = upload(x)
    mask = np.ones((B, P + T), dtype=np.uint8)
    out = _lib().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                         _dev_mask(mask), P, ALPHA)
    dense = _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA,
                                    split=False)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out), to_host_bits(dense))


# (B, H, S, left pads): the decode split plan with 8 splits (pads inside one
# split, covering whole splits), a fully padded sequence, B*H filling the GPU.
DECODE_LEFT = [
    (4, 64, 1001, [0, 100, 999, 1001]),
    (2, 5, 3000, [2999, 1280]),
    (8, 64, 700, [0, 1, 2, 128, 129, 300, 650, 699]),
]


@pytest.mark.parametrize("B,H,S,pads", DECODE_LEFT)
def test_decode_left_padding(B, H, S, pads):
    log(f"case decode masked left B={B} H={H} S={S} pads={pads}")
    mask = _left_pad_mask(S, pads)
    x = _with_nan_hidden(random_inputs(B, H, 1, S - 1, seed=B * 3 + S), mask)
    out = _decode(x, mask, S - 1)
    bits = to_host_bits(out)
    for b in range(B):
        if pads[b] >= S:
            assert not np.any(bits[b]), b
    assert_parity(to_host_f64(out), _oracle(x, mask, S - 1), "decode masked left")


def test_decode_random_mask_and_all_ones():
    import torch
    B, H, S = 3, 16, 2048
    g = np.random.default_rng(3)
    mask = (g.random((B, S)) < 0.3).astype(np.uint8)
    log(f"case decode masked random B={B} H={H} S={S} kept={int(mask.sum())}")
    x = _with_nan_hidden(random_inputs(B, H, 1, S - 1, seed=13), mask)
    out = _decode(x, mask, S - 1)
    assert_parity(to_host_f64(out), _oracle(x, mask, S - 1), "decode masked random")
    y = random_inputs(B, H, 1, S - 1, seed=14)
    d = upload(y)
    ones = _dev_mask(np.ones((B, S), dtype=np.uint8))
    a = _lib().mla_attn_decode_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], ones,
                                      S - 1, ALPHA)
    dense = _lib().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], S - 1, ALPHA)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(a), to_host_bits(dense))


def test_bool_mask_is_accepted():
    import torch
    B, H, T, P = 2, 2, 40, 24
    mask = _left_pad_mask(P + T, [3, 30])
    x = random_inputs(B, H, T, P, seed=21)
    d = upload(x)
    out = _lib().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                         _dev_mask(mask).bool(), P, ALPHA)
    torch.cuda.synchronize()
    assert_parity(to_host_f64(out), _oracle(x, mask, P), "prefill masked bool")


def test_full_size_workloads_sampled():
    """The benchmarked launches (left padding): a batched decode of 32
    sequences over 8192 positions and a prefill of 4 left-padded 4096-token
    prompts, 64 heads; the oracle checks sampled rows, each on its own keys,
    and for the prefill every query row of one head of each sequence."""
    import torch
    from seeded_inputs import MASKED_WORKLOADS, device_inputs, left_pad_mask, left_pads
    for name, wl in MASKED_WORKLOADS.items():
        pads = left_pads(wl, seed=0)
        mask = left_pad_mask(wl.S, pads)
        log(f"case full {name} B={wl.B} H={wl.H} T={wl.T} S={wl.S} sum(pads)={int(pads.sum())}")
        d = device_inputs(wl, "cuda", seed=0)
        m = _dev_mask(mask)
        if wl.T == 1:
            out = _lib().mla_attn_decode_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], m,
                                                wl.past_len, wl.softmax_scale)
        else:
            out = _lib().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], m,
                                                 wl.past_len, wl.softmax_scale)
        torch.cuda.synchronize()
        g = np.random.default_rng(1)
        rows = [(int(g.integers(0, wl.B)), int(g.integers(0, wl.H)), int(g.integers(0, wl.T)))
                for _ in range(24)]
        rows += [(b, 0, wl.T - 1) for b in range(wl.B)]
        if wl.T > 1:   # the first query row that sees a key, and one inside the padding
            rows += [(b, 1, int(min(pads[b], wl.T - 1))) for b in range(wl.B)]
            rows += [(b, 2, int(pads[b]) - 1) for b in range(wl.B) if pads[b] > 0]
        got, ref = [], []
        for b, h, i in rows:
            S_i = wl.past_len + i + 1           # keys 0 .. past_len + i
            sl = {k: to_host_bits(d[k][b:b + 1, h:h + 1, i:i + 1]) for k in ("q_nope", "q_pe")}
            sl.update({k: to_host_bits(d[k][b:b + 1, h:h + 1, :S_i]) for k in ("k_nope", "v")})
            sl["k_pe"] = to_host_bits(d["k_pe"][b:b + 1, :, :S_i])
            ref.append(mla_attention_masked(sl["q_nope"], sl["q_pe"], sl["k_nope"], sl["k_pe"], sl["v"],
                                            mask[b:b + 1, :S_i], S_i - 1, wl.softmax_scale)[0, 0, 0])
            got.append(to_host_f64(out[b, h, i]))
        assert_parity(np.stack(got), np.stack(ref), f"{name} sampled")
        assert torch.isfinite(out).all().item()
        if wl.T > 1:  # every query row of one head per sequence, heads spread over the range
            for b in range(wl.B):
                h = (b * 21 + 5) % wl.H
                sl = {k: to_host_bits(d[k][b:b + 1, h:h + 1]) for k in ("q_nope", "q_pe", "k_nope", "v")}
                sl["k_pe"] = to_host_bits(d["k_pe"][b:b + 1])
                ref_h = mla_attention_masked(sl["q_nope"], sl["q_pe"], sl["k_nope"], sl["k_pe"], sl["v"],
                                             mask[b:b + 1], wl.past_len, wl.softmax_scale)
                assert_parity(to_host_f64(out[b:b + 1, h:h + 1]), ref_h, f"{name} sequence {b} whole head {h}")
        del d, out
        torch.cuda.empty_cache()


def test_graph_replays_follow_the_device_mask():
    """The host never reads the mask: captured masked calls, replayed after
    the mask is rewritten in place, follow each new mask (every replay is
    checked against the oracle)."""
    import torch
    B, H, T, P = 2, 4, 64, 100
    S = P + T
    x = random_inputs(B, H, T, P, seed=41)
    xd = random_inputs(B, H, 1, S - 1, seed=42)
    d, dd = upload(x), upload(xd)
    m = _dev_mask(np.ones((B, S), dtype=np.uint8))
    out = torch.empty((B, H, T, 128), dtype=torch.bfloat16, device="cuda")
    outd = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(_lib().mla_attn_decode_varlen_workspace_bytes(B, H, S), 16), dtype=torch.uint8,
                     device="cuda")

    def calls():
        _lib().mla_attn_prefill_masked(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], m, P, ALPHA,
                                       out=out)
        _lib().mla_attn_decode_masked(dd["q_nope"], dd["q_pe"], dd["k_nope"], dd["k_pe"], dd["v"], m, S - 1,
                                      ALPHA, out=outd, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    rng = np.random.default_rng(43)
    for pads in ([0, 0], [30, 150], [120, 5]):
        mask = _left_pad_mask(S, pads)
        mask[:, -3:] = (rng.random((B, 3)) < 0.5).astype(np.uint8)   # holes near the end too
        log(f"  replay pads={pads}")
        m.copy_(_dev_mask(mask))
        out.fill_(1.0)
        outd.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_parity(to_host_f64(out), _oracle(x, mask, P), f"graph prefill pads={pads}")
        assert_parity(to_host_f64(outd), _oracle(xd, mask, S - 1), f"graph decode pads={pads}")
