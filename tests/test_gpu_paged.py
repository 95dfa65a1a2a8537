"""GPU parity of mla_attn_decode_paged (decode over a paged cache, optionally
appending the new token) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest

from oracle import mla_decode_paged
from seeded_inputs import (PAGED_WORKLOADS, paged_device_inputs, paged_host_inputs, paged_layout,
                           varlen_seq_lens)

from _gpu_util import assert_parity, log, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))
NAN_BF16 = np.uint16(0x7FC0)
PAGE_KEYS = ("k_nope_pages", "k_pe_pages", "v_pages")


def _lib():
    import attention_mla_causal_amd as m
    return m


def _setup(lens, H, bs, seed, spare=2, nan_unowned=True):
    table, N = paged_layout(lens, bs, seed=seed, spare=spare)
    x = paged_host_inputs(len(lens), H, N, bs, seed=seed)
    if nan_unowned:  # every row no sequence owns (spare blocks, tails of last blocks) holds NaN
        owned = np.zeros((N, bs), dtype=bool)
        for b, L in enumerate(lens):
            for j in range(max(int(L), 0)):
                owned[table[b, j // bs], j % bs] = True
        x["k_nope_pages"][:, :, :][~owned[:, None, :].repeat(H, 1)] = NAN_BF16
        x["v_pages"][~owned[:, None, :].repeat(H, 1)] = NAN_BF16
        x["k_pe_pages"][~owned] = NAN_BF16
    return x, table, N


def _call(d, table, lens, max_len, append, out=None, workspace=None):
    import torch
    if out is None:  # NaN first, so a row the kernel never writes fails the parity check
        B, H = d["q_nope"].shape[:2]
        out = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    tb = torch.as_tensor(table, device="cuda")
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    new = (d["k_nope_new"], d["k_pe_new"], d["v_new"]) if append else None
    o = _lib().mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"],
                                     d["v_pages"], tb, sl, max_len, ALPHA, new=new, out=out,
                                     workspace=workspace)
    torch.cuda.synchronize()
    return o


def _oracle(x, table, lens, append):
    new = (x["k_nope_new"], x["k_pe_new"], x["v_new"]) if append else None
    return mla_decode_paged(x["q_nope"], x["q_pe"], x["k_nope_pages"], x["k_pe_pages"], x["v_pages"],
                            table, np.asarray(lens), ALPHA, new=new)


# (lengths, H, block_size): blocks of 32, 64 and 128 rows, sequences of one
# key, one block, a block plus one, empty; a small B*H so long sequences are
# split (merged inside the kernel) and an H of 5 (merged by the merge kernel).
CASES = [
    ([100, 1, 64, 0, 65], 16, 32),
    ([1001, 1, 128, 129], 64, 64),
    ([2000, 3], 16, 128),
    ([1999], 5, 64),
    ([4096, 1025, 31, 32], 8, 32),
]


@pytest.mark.parametrize("append", [False, True])
@pytest.mark.parametrize("lens,H,bs", CASES)
def test_paged_decode(lens, H, bs, append):
    seed = sum(lens) + H + bs
    x, table, N = _setup(lens, H, bs, seed)
    log(f"case paged lens={lens} H={H} bs={bs} blocks={N} append={append}")
    d = upload(x)
    max_len = max(max(lens), 1)
    out = _call(d, table, lens, max_len, append)
    ref, pages = _oracle(x, table, lens, append)
    assert_parity(to_host_f64(out), ref, f"paged {lens} H={H} bs={bs} append={append}")
    for b, L in enumerate(lens):
        if L == 0:
            assert not np.any(to_host_bits(out)[b])
    # the pages hold exactly the appended rows (or are untouched); NaN rows stay NaN bits
    for k, want in zip(PAGE_KEYS, pages):
        assert np.array_equal(to_host_bits(d[k]), want), f"{k} after the call"


def test_appended_one_key_sequence_returns_its_value():
    lens, H, bs = [1, 1, 40], 64, 32
    x, table, N = _setup(lens, H, bs, 7)
    d = upload(x)
    out = to_host_bits(_call(d, table, lens, 40, True))
    log(f"case paged append one-key lens={lens}")
    assert np.array_equal(out[0], x["v_new"][0])
    assert np.array_equal(out[1], x["v_new"][1])


def test_out_of_range_table_entries_past_the_length_are_ignored():
    lens, H, bs = [70, 5], 16, 32
    x, table, N = _setup(lens, H, bs, 8, nan_unowned=False)
    ref, _ = _oracle(x, table, lens, False)
    bad = np.concatenate([table, np.full((2, 3), 1 << 30, dtype=np.int32)], axis=1)
    bad[0, 3] = -7
    bad[1, 1:] = -1
    log(f"case paged bad table tail lens={lens}")
    out = _call(upload(x), bad, lens, 70, False)
    assert_parity(to_host_f64(out), ref, "paged bad table tail")


def test_graph_decode_loop_appends_one_token_per_replay():
    """A captured decode-with-append replayed as a decode loop: before each
    replay the lengths grow by one and new rows are written to the input
    tensors; each replay matches the oracle on the pages it started from."""
    import torch
    H, bs = 16, 32
    final = [70, 33, 3]
    steps = 3
    x, table, N = _setup(final, H, bs, 9, nan_unowned=False)
    d = upload(x)
    m = _lib()
    tb = torch.as_tensor(table, device="cuda")
    lens0 = [L - steps for L in final]
    sl = torch.as_tensor(np.asarray(lens0, dtype=np.int32), device="cuda")
    out = torch.empty((len(final), H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(m.mla_attn_decode_paged_workspace_bytes(len(final), H, max(final)), 16),
                     dtype=torch.uint8, device="cuda")

    def call():
        m.mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"],
                                d["v_pages"], tb, sl, max(final), ALPHA,
                                new=(d["k_nope_new"], d["k_pe_new"], d["v_new"]), out=out, workspace=ws)

    log(f"case paged graph decode loop final={final} steps={steps}")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()          # warm-up call appends at lens0 - 1 ...
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    rng = np.random.default_rng(10)
    for i in range(1, steps + 1):
        lens = [L0 + i for L0 in lens0]
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        host = {k: to_host_bits(d[k]) for k in d}
        for k in ("k_nope_new", "k_pe_new", "v_new", "q_nope"):
            host[k] = rng.integers(0x3C00, 0x4000, size=host[k].shape).astype(np.uint16)
            d[k].copy_(upload({k: host[k]})[k])
        out.fill_(float("nan"))  # a (b, h) the replay does not merge keeps its NaN
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, pages = _oracle(host, table, lens, True)
        assert_parity(to_host_f64(out), ref, f"graph step {i}")
        for k, want in zip(PAGE_KEYS, pages):
            assert np.array_equal(to_host_bits(d[k]), want), f"{k} after graph step {i}"


def test_paged_batched_full_size_sampled():
    """B=32, H=64, lengths uniform in [1, 8192], blocks of 64 rows in a
    shuffled layout, with append; inputs drawn on the device; sampled rows
    against the oracle and the appended slots checked."""
    import torch
    wl = PAGED_WORKLOADS["paged_batched_decode"]
    lens = varlen_seq_lens(wl.B, wl.cap, seed=0)
    table, N = paged_layout(lens, wl.block_size, seed=0)
    log(f"case paged_batched_decode B={wl.B} H={wl.H} bs={wl.block_size} blocks={N} sum={int(lens.sum())}")
    d = paged_device_inputs(wl.B, wl.H, N, wl.block_size, "cuda", seed=0)
    before_pe = d["k_pe_pages"].clone()
    out = _call(d, table, lens, wl.cap, True)
    assert torch.isfinite(out).all().item()
    rng = np.random.default_rng(3)
    picks = {(0, 0), (wl.B - 1, wl.H - 1), (int(np.argmin(lens)), 7)}
    while len(picks) < 8:
        picks.add((int(rng.integers(wl.B)), int(rng.integers(wl.H))))
    got, ref = [], []
    for b, h in sorted(picks):
        L = int(lens[b])
        nb = -(-L // wl.block_size)
        blocks = table[b, :nb]
        sub = {"q_nope": to_host_bits(d["q_nope"][b:b + 1, h:h + 1]),
               "q_pe": to_host_bits(d["q_pe"][b:b + 1, h:h + 1]),
               "k_nope_pages": to_host_bits(d["k_nope_pages"][blocks][:, h:h + 1]),
               "k_pe_pages": to_host_bits(before_pe[blocks]),
               "v_pages": to_host_bits(d["v_pages"][blocks][:, h:h + 1]),
               "k_nope_new": to_host_bits(d["k_nope_new"][b:b + 1, h:h + 1]),
               "k_pe_new": to_host_bits(d["k_pe_new"][b:b + 1]),
               "v_new": to_host_bits(d["v_new"][b:b + 1, h:h + 1])}
        # the pages already hold the appended rows; the oracle appends them again (same bits)
        r, _ = _oracle(sub, np.arange(nb, dtype=np.int32)[None], [L], True)
        ref.append(r[0, 0, 0])
        got.append(to_host_f64(out[b, h, 0]))
        blk, row = table[b, (L - 1) // wl.block_size], (L - 1) % wl.block_size
        assert np.array_equal(to_host_bits(d["k_nope_pages"][blk, h, row]), sub["k_nope_new"][0, 0, 0])
        assert np.array_equal(to_host_bits(d["k_pe_pages"][blk, row]), sub["k_pe_new"][0, 0, 0])
    assert_parity(np.stack(got), np.stack(ref), "paged batched sampled")


def _random_paged_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, H = int(g.integers(1, 7)), int(g.integers(1, 65))
        bs = 32 * int(g.integers(1, 5))
        lens = [int(v) for v in g.integers(0, 2500, size=B)]
        cases.append((lens, H, bs, bool(g.integers(0, 2))))
    return cases


@pytest.mark.parametrize("lens,H,bs,append", _random_paged_cases(6, 2031))
def test_paged_random_shapes(lens, H, bs, append):
    """Seeded random lengths, head counts and block sizes (multiples of 32),
    with and without the fused append; rows no sequence owns hold NaN."""
    seed = sum(lens) + 3 * H + bs
    x, table, N = _setup(lens, H, bs, seed)
    log(f"case paged random lens={lens} H={H} bs={bs} blocks={N} append={append}")
    d = upload(x)
    out = _call(d, table, lens, max(max(lens), 1), append)
    ref, pages = _oracle(x, table, lens, append)
    assert_parity(to_host_f64(out), ref, f"paged random {lens} H={H} bs={bs} append={append}")
    for k, want in zip(PAGE_KEYS, pages):
        assert np.array_equal(to_host_bits(d[k]), want), f"{k} after the call"
