"""GPU parity of mla_attn_prefill_varlen (prefill of a right-padded batch with
a query count and a cached length per sequence) against the fp64 oracle,
through the C ABI."""

import numpy as np
import pytest

from oracle import mla_attention_rows, mla_prefill_varlen
from seeded_inputs import VARLEN_PREFILL_WORKLOADS, device_inputs, random_inputs, varlen_prefill_lens

from _gpu_util import assert_parity, log, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))
NAN_BF16 = np.uint16(0x7FC0)


def _lib():
    import attention_mla_causal_amd as m
    return m


def _inputs(B, H, Tmax, Smax, seed, q_lens=None, past_lens=None, std=1.0):
    """Host inputs of the padded shapes; with lengths given, every padded row
    (queries past T_b, keys past P_b + T_b) holds NaN, so reading one shows."""
    x = random_inputs(B, H, Tmax, Smax - Tmax, seed=seed, std=std)
    if q_lens is not None:
        for b in range(B):
            T = max(0, min(int(q_lens[b]), Tmax))
            P = max(0, min(int(past_lens[b]), Smax - T))
            for k in ("q_nope", "q_pe"):
                x[k][b, :, T:] = NAN_BF16
            for k in ("k_nope", "k_pe", "v"):
                x[k][b, :, P + T:] = NAN_BF16
    return x


def _lens(a):
    import torch
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


def _gpu(d, q_lens, past_lens, out=None):
    import torch
    o = _lib().mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                       _lens(q_lens), _lens(past_lens), ALPHA, out=out)
    torch.cuda.synchronize()
    return o


def _oracle(x, q_lens, past_lens):
    return mla_prefill_varlen(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"],
                              np.asarray(q_lens), np.asarray(past_lens), ALPHA)


def test_mixed_lengths_with_nan_padding():
    B, H, Tmax, Smax = 4, 8, 300, 1100
    tq, pp = [300, 1, 0, 129], [800, 0, 5, 971]
    log(f"case prefill varlen mixed B={B} H={H} Tmax={Tmax} Smax={Smax} q={tq} past={pp}")
    x = _inputs(B, H, Tmax, Smax, 0, tq, pp)
    out = _gpu(upload(x), tq, pp)
    bits = to_host_bits(out)
    for b in range(B):          # padded query rows are exact zeros
        assert not np.any(bits[b, :, tq[b]:]), b
    assert_parity(to_host_f64(out), _oracle(x, tq, pp), "prefill varlen mixed")


# (B, H, Tmax, Smax, q_lens, past_lens): ragged query tiles and key tiles,
# sequences with no queries, one query, a cache that is and is not a multiple
# of the 32-key tile, and lengths outside their ranges (clamped on the device:
# T_b to [0, Tmax], P_b to [0, Smax - T_b]); 24 (batch, head) groups, a
# multiple of 8 but not of 16 (one group at a time per XCD, not windows).
EDGE = [
    (2, 3, 129, 129, [129, 128], [0, 1]),
    (3, 2, 257, 600, [1, 256, 257], [599, 32, 343]),
    (2, 5, 64, 1000, [0, 64], [0, 936]),
    (1, 64, 17, 17, [17], [0]),
    (3, 4, 200, 400, [300, -3, 150], [0, 7, 9999]),
    (3, 8, 300, 700, [300, 1, 170], [400, 0, 77]),
]


@pytest.mark.parametrize("B,H,Tmax,Smax,tq,pp", EDGE)
def test_edge_cases(B, H, Tmax, Smax, tq, pp):
    log(f"case prefill varlen edge B={B} H={H} Tmax={Tmax} Smax={Smax} q={tq} past={pp}")
    eq = [max(0, min(t, Tmax)) for t in tq]
    ep = [max(0, min(p, Smax - t)) for p, t in zip(pp, eq)]
    x = _inputs(B, H, Tmax, Smax, B * 100 + H + Tmax, eq, ep)
    out = _gpu(upload(x), tq, pp)
    bits = to_host_bits(out)
    for b in range(B):
        assert not np.any(bits[b, :, eq[b]:]), b
    assert_parity(to_host_f64(out), _oracle(x, eq, ep), "prefill varlen edge")


@pytest.mark.parametrize("B", [256, 300])
def test_many_sequences(B):
    """Up to 256 sequences the workgroups rank them by work; beyond that they
    are taken in index order: both orders cover every row."""
    H, Tmax, Smax = 1, 40, 100
    g = np.random.default_rng(B)
    tq = g.integers(0, Tmax + 1, size=B)
    pp = g.integers(0, Smax - Tmax + 1, size=B)
    log(f"case prefill varlen many B={B} H={H} Tmax={Tmax} Smax={Smax}")
    x = _inputs(B, H, Tmax, Smax, B, tq, pp)
    out = _gpu(upload(x), tq, pp)
    bits = to_host_bits(out)
    for b in range(B):
        assert not np.any(bits[b, :, tq[b]:]), b
    assert_parity(to_host_f64(out), _oracle(x, tq, pp), f"prefill varlen B={B}")


@pytest.mark.parametrize("B,H,T,P", [(2, 4, 300, 77), (1, 64, 256, 1024)])
def test_full_lengths_equal_dense_prefill(B, H, T, P):
    """Every sequence at the slice sizes: bit-identical to mla_attn_prefill."""
    import torch
    log(f"case prefill varlen = dense B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=7)
    d = upload(x)
    out = _gpu(d, [T] * B, [P] * B)
    dense = _lib().mla_attn_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA,
                                    split=False)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(out), to_host_bits(dense))
    assert_parity(to_host_f64(out), _oracle(x, [T] * B, [P] * B), "prefill varlen full")


def test_graph_replays_follow_the_device_lengths():
    """The host never reads the lengths: one captured call, replayed after the
    length arrays are rewritten, follows each new set (every replay checked)."""
    import torch
    B, H, Tmax, Smax = 3, 4, 160, 700
    x = random_inputs(B, H, Tmax, Smax - Tmax, seed=11)
    d = upload(x)
    ql = _lens([160, 1, 40])
    pl = _lens([540, 0, 300])
    out = torch.empty((B, H, Tmax, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _lib().mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                       ql, pl, ALPHA, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _lib().mla_attn_prefill_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                       ql, pl, ALPHA, out=out)
    torch.cuda.synchronize()
    for tq, pp in ([[160, 1, 40], [540, 0, 300]], [[5, 160, 0], [0, 540, 9]],
                   [[100, 100, 100], [33, 600, 1]]):
        log(f"  replay q={tq} past={pp}")
        ql.copy_(_lens(tq))
        pl.copy_(_lens(pp))
        out.fill_(1.0)   # a stale row would show
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = to_host_f64(out)
        assert_parity(got, _oracle(x, tq, pp), f"graph replay q={tq}")


def _sample_rows(tq, H, n, seed):
    g = np.random.default_rng(seed)
    rows = []
    B = len(tq)
    for _ in range(n):
        b = int(g.integers(0, B))
        while tq[b] == 0:
            b = int(g.integers(0, B))
        rows.append((b, int(g.integers(0, H)), int(g.integers(0, tq[b]))))
    # always the last query of the longest sequence and the first of each
    rows.append((0, 0, int(tq[0]) - 1))
    rows += [(b, H - 1, 0) for b in range(B) if tq[b] > 0]
    return rows


def test_full_size_workload_sampled():
    """The benchmarked launch (8 chunked prefills of mixed lengths, 64 heads,
    2048 x 16384 slices); the oracle checks sampled rows of each sequence on
    its own keys only and every query row of one head per sequence, and every
    padded row must be zero."""
    import torch
    wl = VARLEN_PREFILL_WORKLOADS["varlen_prefill"]
    tq, pp = varlen_prefill_lens(wl.B, wl.max_q, wl.max_kv, seed=0)
    log(f"case full varlen_prefill B={wl.B} H={wl.H} Tmax={wl.max_q} Smax={wl.max_kv} "
        f"q={tq.tolist()} past={pp.tolist()}")
    d = device_inputs(wl.padded(), "cuda", seed=0)
    out = _gpu(d, tq, pp)
    rows = _sample_rows(tq, wl.H, 40, seed=2)
    got = np.stack([to_host_f64(out[b, h, i]) for b, h, i in rows])
    ref = np.empty_like(got)
    by_bh = {}
    for n, (b, h, i) in enumerate(rows):
        by_bh.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_bh.items():
        S = int(pp[b]) + int(tq[b])
        sl = {k: to_host_bits(d[k][b:b + 1, h:h + 1]) for k in ("q_nope", "q_pe")}
        sl.update({k: to_host_bits(d[k][b:b + 1, h:h + 1, :S]) for k in ("k_nope", "v")})
        sl["k_pe"] = to_host_bits(d["k_pe"][b:b + 1, :, :S])
        qi = [i for _, i in items]
        r = mla_attention_rows(sl["q_nope"][:, :, :int(tq[b])], sl["q_pe"][:, :, :int(tq[b])],
                               sl["k_nope"], sl["k_pe"], sl["v"], int(pp[b]), wl.softmax_scale,
                               [(0, 0, i) for i in qi])
        for k, (n, _) in enumerate(items):
            ref[n] = r[k]
    assert_parity(got, ref, "varlen_prefill sampled")
    # every query row of one head of each sequence, heads spread over the range
    for b in range(wl.B):
        h = (b * 21 + 5) % wl.H
        T_b, P_b = int(tq[b]), int(pp[b])
        sl = {k: to_host_bits(d[k][b:b + 1, h:h + 1, :T_b]) for k in ("q_nope", "q_pe")}
        sl.update({k: to_host_bits(d[k][b:b + 1, h:h + 1, :T_b + P_b]) for k in ("k_nope", "v")})
        sl["k_pe"] = to_host_bits(d["k_pe"][b:b + 1, :, :T_b + P_b])
        ref_h = mla_prefill_varlen(sl["q_nope"], sl["q_pe"], sl["k_nope"], sl["k_pe"], sl["v"], np.array([T_b]),
                                   np.array([P_b]), wl.softmax_scale)
        assert_parity(to_host_f64(out[b:b + 1, h:h + 1, :T_b]), ref_h, f"varlen_prefill sequence {b} head {h}")
    for b in range(wl.B):
        assert not torch.any(out[b, :, int(tq[b]):] != 0).item(), b
    assert torch.isfinite(out).all().item()


def _random_prefill_varlen_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, H = int(g.integers(1, 5)), int(g.integers(1, 17))
        Tmax = int(g.integers(1, 301))
        Smax = Tmax + int(g.integers(0, 1201))
        tq = [int(v) for v in g.integers(0, Tmax + 1, size=B)]
        pp = [int(g.integers(0, Smax - t + 1)) for t in tq]
        cases.append((B, H, Tmax, Smax, tq, pp))
    return cases


@pytest.mark.parametrize("B,H,Tmax,Smax,tq,pp", _random_prefill_varlen_cases(6, 2030))
def test_random_shapes(B, H, Tmax, Smax, tq, pp):
    """Seeded random padded shapes and per-sequence lengths, padded rows NaN."""
    log(f"case prefill varlen random B={B} H={H} Tmax={Tmax} Smax={Smax} q={tq} past={pp}")
    x = _inputs(B, H, Tmax, Smax, B * 31 + H + Tmax + Smax, tq, pp)
    out = _gpu(upload(x), tq, pp)
    bits = to_host_bits(out)
    for b in range(B):
        assert not np.any(bits[b, :, tq[b]:]), b
    assert_parity(to_host_f64(out), _oracle(x, tq, pp), "prefill varlen random")
