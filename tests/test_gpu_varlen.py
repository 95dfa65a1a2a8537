"""GPU parity of mla_attn_decode_varlen (decode over a preallocated,
right-padded cache with a length per sequence) against the fp64 oracle,
through the C ABI."""

import numpy as np
import pytest

from oracle import mla_decode_varlen, mla_decode_varlen_rows
from seeded_inputs import (VARLEN_WORKLOADS, device_inputs, random_inputs, varlen_seq_lens)

from _gpu_util import assert_parity, log, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))
NAN_BF16 = np.uint16(0x7FC0)


def _lib():
    import attention_mla_causal_amd as m
    return m


def _cache(B, H, cap, seed, lens=None):
    """Host inputs with S = cap; rows past each length hold NaN if lens given."""
    x = random_inputs(B, H, 1, cap - 1, seed=seed)
    if lens is not None:
        for b, L in enumerate(lens):
            L = max(0, min(int(L), cap))
            for k in ("k_nope", "k_pe", "v"):
                x[k][b, :, L:] = NAN_BF16
    return x


def _gpu(d, lens, max_len, out=None, workspace=None):
    import torch
    if out is None:  # NaN first, so a row the kernel never writes fails the parity check
        B, H = d["q_nope"].shape[:2]
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    o = _lib().mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], sl,
                                      max_len, ALPHA, out=out, workspace=workspace)
    torch.cuda.synchronize()
    return o


def _oracle(x, lens):
    return mla_decode_varlen(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"],
                             np.asarray(lens), ALPHA)


def test_varlen_mixed_lengths_with_nan_padding():
    B, H, cap = 4, 64, 1024
    lens = [1001, 1, 0, 513]
    log(f"case varlen mixed B={B} H={H} cap={cap} lens={lens}")
    x = _cache(B, H, cap, 0, lens)
    out = _gpu(upload(x), lens, cap)
    got = to_host_f64(out)
    assert np.array_equal(to_host_bits(out)[2], np.zeros((H, 1, 128), dtype=np.uint16))
    assert_parity(got, _oracle(x, lens), "varlen mixed")


# (B, H, cache_len, lengths, max_seq_len): a split plan with mostly empty
# splits for the short sequence (merged inside the kernel), the merge kernel
# path (H = 5), lengths around the 128-key trip, empty sequences, lengths
# outside [0, max_seq_len] clamped on the device, and long sequences split in
# pieces of at most 1024 keys although B*H alone fills the chip.
EDGE = [
    (2, 16, 4096, [4096, 5], 4096),
    (1, 5, 2000, [1999], 2000),
    (3, 64, 300, [300, 129, 128], 300),
    (4, 8, 777, [0, 0, 1, 777], 777),
    (3, 16, 512, [600, -4, 200], 256),
    (3, 100, 3000, [3000, 1, 2049], 3000),   # long sequences split in the varlen plan; merge kernel
    (4, 64, 2500, [2500, 1025, 1024, 3], 2500),  # varlen split, merged in the split kernel
    # one split per (b, h): 64 sequences taken longest first (ties and empty
    # ones among them), and 65, past the ranking, in index order
    (64, 32, 160, [(37 * b) % 53 * 3 for b in range(64)], 160),
    (65, 32, 160, [(23 * b) % 53 * 3 for b in range(65)], 160),
]


@pytest.mark.parametrize("B,H,cap,lens,max_len", EDGE)
def test_varlen_edge_cases(B, H, cap, lens, max_len):
    log(f"case varlen edge B={B} H={H} cap={cap} lens={lens} max={max_len} "
        f"ws={_lib().mla_attn_decode_varlen_workspace_bytes(B, H, max_len)}")
    eff = [max(0, min(L, max_len)) for L in lens]
    x = _cache(B, H, cap, B * 7 + H + cap, eff)
    out = _gpu(upload(x), lens, max_len)
    assert_parity(to_host_f64(out), _oracle(x, eff), f"varlen {B},{H},{cap},{lens}")
    for b, L in enumerate(eff):
        if L == 0:
            assert not np.any(to_host_bits(out)[b])


@pytest.mark.parametrize("B,H,cap", [(2, 64, 1001), (1, 64, 1001), (3, 8, 260)])
def test_full_lengths_equal_dense_decode(B, H, cap):
    """Every sequence using the whole cache is the dense decode, bit for bit."""
    log(f"case varlen == dense B={B} H={H} S={cap}")
    x = random_inputs(B, H, 1, cap - 1, seed=cap + H)
    d = upload(x)
    a = _gpu(d, [cap] * B, cap)
    b = _lib().mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], cap - 1, ALPHA)
    assert np.array_equal(to_host_bits(a), to_host_bits(b))


def test_graph_replays_follow_the_device_lengths():
    """One captured call; the length array is rewritten between replays (eager
    copies, not part of the graph) and every replay matches an eager call."""
    import torch
    B, H, cap = 3, 16, 2048
    log(f"case varlen graph B={B} H={H} cap={cap}")
    x = random_inputs(B, H, 1, cap - 1, seed=5)
    d = upload(x)
    m = _lib()
    sl = torch.tensor([cap, 7, 1000], dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(m.mla_attn_decode_varlen_workspace_bytes(B, H, cap), 16), dtype=torch.uint8,
                     device="cuda")

    def call():
        m.mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], sl, cap,
                                 ALPHA, out=out, workspace=ws)

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
    for i, lens in enumerate(([cap, 7, 1000], [1, 2048, 0], [513, 3, 2047], [cap, 7, 1000])):
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))  # a (b, h) the replay does not merge keeps its NaN
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replayed = to_host_bits(out).copy()
        assert np.isfinite(to_host_f64(out)).all(), f"replay {i} left rows unwritten"
        eager = to_host_bits(_gpu(d, lens, cap, out=torch.full_like(out, float("nan"))))
        assert np.array_equal(replayed, eager), f"replay {i} with lengths {lens}"
        if i == 1:
            assert_parity(to_host_f64(out), _oracle(x, lens), "varlen graph replay")


def test_varlen_batched_full_size_sampled():
    """B=32, H=64, cache 8192 rows, lengths uniform in [1, 8192]; inputs drawn
    on the device; sampled (b, h) rows against the oracle."""
    import torch
    wl = VARLEN_WORKLOADS["varlen_batched_decode"]
    lens = varlen_seq_lens(wl.B, wl.cap, seed=0)
    log(f"case varlen_batched_decode B={wl.B} H={wl.H} cap={wl.cap} sum(lens)={int(lens.sum())}")
    d = device_inputs(wl.cache(), "cuda", seed=0)
    out = _gpu(d, lens, wl.cap)
    assert torch.isfinite(out).all().item()
    rng = np.random.default_rng(2)
    picks = {(0, 0), (wl.B - 1, wl.H - 1), (int(np.argmin(lens)), 5)}
    while len(picks) < 10:
        picks.add((int(rng.integers(wl.B)), int(rng.integers(wl.H))))
    picks = sorted(picks)
    got, ref = [], []
    for b, h in picks:
        L = int(lens[b])
        xs = {k: to_host_bits(d[k][b:b + 1, h:h + 1] if k != "k_pe" else d[k][b:b + 1])
              for k in ("q_nope", "q_pe", "k_nope", "k_pe", "v")}
        for k in ("k_nope", "k_pe", "v"):
            xs[k] = xs[k][:, :, :L]
        ref.append(mla_decode_varlen_rows(xs["q_nope"], xs["q_pe"], xs["k_nope"], xs["k_pe"], xs["v"],
                                          np.array([L]), ALPHA, [(0, 0)])[0])
        got.append(to_host_f64(out[b, h, 0]))
    assert_parity(np.stack(got), np.stack(ref), "varlen batched sampled")


def _random_varlen_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, H, cap = int(g.integers(1, 13)), int(g.integers(1, 65)), int(g.integers(1, 3001))
        lens = [int(v) for v in g.integers(-2, cap + 3, size=B)]  # a few outside [0, cap]: clamped
        cases.append((B, H, cap, lens))
    return cases


@pytest.mark.parametrize("B,H,cap,lens", _random_varlen_cases(8, 2029))
def test_varlen_random_shapes(B, H, cap, lens):
    """Seeded random batch sizes, head counts, cache lengths and per-sequence
    lengths (max_seq_len = cache length), rows past each length NaN."""
    log(f"case varlen random B={B} H={H} cap={cap} lens={lens}")
    eff = [max(0, min(L, cap)) for L in lens]
    x = _cache(B, H, cap, B * 13 + H * 7 + cap, eff)
    out = _gpu(upload(x), lens, cap)
    assert_parity(to_host_f64(out), _oracle(x, eff), f"varlen random {B},{H},{cap}")
    for b, L in enumerate(eff):
        if L == 0:
            assert not np.any(to_host_bits(out)[b])
