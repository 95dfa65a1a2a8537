"""GPU parity of the rotary prologue (mla_rope_table, mla_rope_apply) against
the fp64 oracle, through the C ABI; and the prologue followed by the prefill
against the oracle's rotation followed by its attention.

Bars: the fp32 table is within 2 fp32 ulps of the fp64 cosine and sine (both
sides take the angle and its cosine and sine in fp64; only the rounding to
fp32 and the last bits of pow/sincos may differ). A rotated bf16 value is
within half a bf16 ulp of the exact rotation (2^-8 relative) plus the fp32
arithmetic and the fp32 table (2^-20 of its pair's magnitude).
"""

import numpy as np
import pytest

from oracle import KIMI_K2_ROPE, apply_rope, mla_attention, rope_cos_sin, rope_positions
from seeded_inputs import random_inputs

from _gpu_util import assert_parity, log, to_device, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))
RAMP = dict(theta=50000.0, factor=32.0, original_max_position=4096, beta_fast=32.0, beta_slow=1.0)
PLAIN = dict(theta=10000.0, factor=1.0, original_max_position=4096, beta_fast=1.0, beta_slow=1.0)


def _lib():
    import attention_mla_causal_amd as m
    return m


def _gpu_table(max_pos, cfg):
    return _lib().mla_rope_table(max_pos, cfg["theta"], cfg["factor"], cfg["original_max_position"],
                                 cfg["beta_fast"], cfg["beta_slow"])


def _check_table(tab_gpu, max_pos, cfg, what):
    t = tab_gpu.cpu().numpy().astype(np.float64)
    cos, sin = rope_cos_sin(max_pos, **cfg)
    for got, ref, name in ((t[..., 0], cos, "cos"), (t[..., 1], sin, "sin")):
        err = np.abs(got - ref)
        bound = 2.0 ** -22 * np.abs(ref) + 1e-9
        log(f"  table {what} {name}: max|err|={err.max():.3e}")
        assert np.all(err <= bound), (what, name, np.unravel_index(np.argmax(err - bound), err.shape))


def _check_rotation(got_bits, x_bits, ref, what):
    got = np.asarray(got_bits, dtype=np.float64)
    x = to_f64(x_bits)
    pair = np.repeat(np.abs(x[..., 0::2]) + np.abs(x[..., 1::2]), 2, axis=-1)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * pair + 1e-30
    log(f"  rotation {what}: max|err|={err.max():.3e} n={err.size}")
    assert np.all(err <= bound), (what, np.unravel_index(np.argmax(err - bound), err.shape))


def to_f64(bits):
    from oracle import bf16_bits_to_f64
    return bf16_bits_to_f64(np.asarray(bits))


@pytest.mark.parametrize("name,max_pos,cfg", [("released", 20000, KIMI_K2_ROPE), ("plain", 3000, PLAIN),
                                              ("ramp", 5000, RAMP), ("one", 1, KIMI_K2_ROPE)])
def test_table_matches_oracle(name, max_pos, cfg):
    log(f"case rope table {name} max_pos={max_pos}")
    _check_table(_gpu_table(max_pos, cfg), max_pos, cfg, name)


@pytest.mark.parametrize("B,H,T,P", [(2, 8, 37, 100), (1, 64, 1, 4095), (3, 5, 130, 0)])
def test_apply_matches_oracle(B, H, T, P):
    """The new queries' q_pe (H rows per position) and the new keys' shared
    k_pe (one row per position), rotated at past_len + t."""
    log(f"case rope apply B={B} H={H} T={T} P={P}")
    x = random_inputs(B, H, T, P, seed=11 + T)
    tab = _gpu_table(P + T, KIMI_K2_ROPE)
    cos, sin = rope_cos_sin(P + T, **KIMI_K2_ROPE)
    pos = rope_positions(B, T, past_len=P)
    kp_new = np.ascontiguousarray(x["k_pe"][:, :, P:])                 # the new keys' rows
    for bits, what in ((x["q_pe"], "q_pe"), (kp_new, "k_pe")):
        d = to_device(bits)
        out = _lib().mla_rope_apply(d, tab, past_len=P)
        assert out.data_ptr() == d.data_ptr()
        _check_rotation(to_host_f64(d), bits, apply_rope(to_f64(bits), pos, cos, sin), what)


def test_apply_per_sequence_positions_and_clamping():
    """past_lens give each sequence its own positions; positions read from
    them are clamped into the table (the last row), never beyond it."""
    import torch
    B, H, T, max_pos = 4, 3, 20, 10000
    x = random_inputs(B, H, T, 0, seed=21)["q_pe"]
    lens = np.array([0, 300, 9990, 5], dtype=np.int32)
    log(f"case rope apply past_lens={lens.tolist()} max_pos={max_pos}")
    tab = _gpu_table(max_pos, KIMI_K2_ROPE)
    d = to_device(x)
    _lib().mla_rope_apply(d, tab, past_lens=torch.as_tensor(lens, device="cuda"))
    cos, sin = rope_cos_sin(max_pos, **KIMI_K2_ROPE)
    pos = np.minimum(rope_positions(B, T, past_lens=lens), max_pos - 1)
    assert pos[2, -1] == max_pos - 1 and pos[2, 0] == 9990
    _check_rotation(to_host_f64(d), x, apply_rope(to_f64(x), pos, cos, sin), "past_lens")


def test_full_size_sampled():
    """The chunked prefill's new tokens: q_pe [1, 64, 2048, 64] at positions
    14336..16383 and their k_pe rows, against the oracle on sampled rows; the
    whole 16384-position table against the oracle's."""
    B, H, T, P = 1, 64, 2048, 14336
    log(f"case rope full size B={B} H={H} T={T} P={P}")
    tab = _gpu_table(P + T, KIMI_K2_ROPE)
    _check_table(tab, P + T, KIMI_K2_ROPE, "full")
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((B, H, T, 64)) * 1.0).astype(np.float32)
    bits = (np.frombuffer(x.tobytes(), dtype=np.uint32) >> 16).astype(np.uint16).reshape(x.shape)  # truncate to bf16
    d = to_device(bits)
    _lib().mla_rope_apply(d, tab, past_len=P)
    got = to_host_f64(d)
    cos, sin = rope_cos_sin(P + T, **KIMI_K2_ROPE)
    hs = rng.integers(0, H, 64)
    ts = np.concatenate([[0, T - 1], rng.integers(0, T, 62)])
    for h, t in zip(hs, ts):
        ref = apply_rope(to_f64(bits[:, h:h + 1, t:t + 1]), np.array([[P + t]]), cos, sin)
        _check_rotation(got[:, h:h + 1, t:t + 1], bits[:, h:h + 1, t:t + 1], ref, f"h={h} t={t}")


@pytest.mark.parametrize("B,H,T,P", [(1, 4, 70, 60), (2, 16, 129, 0)])
def test_prologue_then_prefill(B, H, T, P):
    """Rotate the new queries' q_pe at past_len + t and the whole k_pe at its
    positions, then attend: against the oracle's rotation and attention."""
    log(f"case rope prologue + prefill B={B} H={H} T={T} P={P}")
    S = P + T
    x = random_inputs(B, H, T, P, seed=31 + P)
    tab = _gpu_table(S, KIMI_K2_ROPE)
    dev = {k: to_device(v) for k, v in x.items()}
    m = _lib()
    m.mla_rope_apply(dev["q_pe"], tab, past_len=P)
    m.mla_rope_apply(dev["k_pe"], tab, past_len=0)
    out = m.mla_attn_prefill(dev["q_nope"], dev["q_pe"], dev["k_nope"], dev["k_pe"], dev["v"], P, ALPHA)
    cos, sin = rope_cos_sin(S, **KIMI_K2_ROPE)
    q_rot = apply_rope(to_f64(x["q_pe"]), rope_positions(B, T, past_len=P), cos, sin)
    k_rot = apply_rope(to_f64(x["k_pe"]), rope_positions(B, S), cos, sin)
    ref = mla_attention(to_f64(x["q_nope"]), q_rot, to_f64(x["k_nope"]), k_rot, to_f64(x["v"]), P, ALPHA)
    assert_parity(to_host_f64(out), ref, f"rope+prefill B={B} H={H} T={T} P={P}")


def test_graph_replays_with_new_positions():
    """A captured rotation replays with the positions and rows written into
    its inputs between replays; every replay matches an eager call."""
    import torch
    B, H, T, max_pos = 3, 8, 33, 4096
    tab = _gpu_table(max_pos, KIMI_K2_ROPE)
    m = _lib()
    x = torch.empty((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.mla_rope_apply(x, tab, past_lens=lens)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.mla_rope_apply(x, tab, past_lens=lens)
    for r in range(3):
        src = to_device(random_inputs(B, H, T, 0, seed=40 + r)["q_pe"])
        new_lens = torch.as_tensor(np.array([r * 1000, 7 + r, 4000 - T - r], dtype=np.int32), device="cuda")
        x.copy_(src)
        lens.copy_(new_lens)
        g.replay()
        torch.cuda.synchronize()
        eager = src.clone()
        m.mla_rope_apply(eager, tab, past_lens=new_lens)
        torch.cuda.synchronize()
        log(f"  replay {r}: lens={new_lens.tolist()}")
        assert np.array_equal(to_host_bits(x), to_host_bits(eager)), f"replay {r}"


def test_empty_and_errors_through_the_binding():
    import torch
    m = _lib()
    tab = _gpu_table(16, KIMI_K2_ROPE)
    x = torch.empty((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    assert m.mla_rope_apply(x, tab, past_len=16) is x                   # no rows: no-op
    y = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        m.mla_rope_apply(y, tab, past_len=13)                             # position 16 is past the table
    assert tuple(m.mla_rope_table(0).shape) == (0, 32, 2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,H,P", [(1, 64, 1000), (4, 16, 300), (32, 8, 4095)])
def test_fused_prologue_decode(B, H, P):
    """mla_attn_decode with rope_table: the raw q_pe turns at position past_len
    inside the kernel; the cache's k_pe was rotated at its positions (here by
    mla_rope_apply). Against the oracle's rotation of the query and its
    attention over the same cached keys; and close to the unfused path
    (rotation kernel, then the plain decode), which rounds the rotated query
    to bf16 first."""
    import torch
    S = P + 1
    log(f"case rope fused decode B={B} H={H} P={P}")
    x = random_inputs(B, H, 1, P, seed=50 + H)
    tab = _gpu_table(S, KIMI_K2_ROPE)
    d = {k: to_device(v) for k, v in x.items()}
    m = _lib()
    m.mla_rope_apply(d["k_pe"], tab, past_len=0)                  # the cache holds rotated keys
    k_rot_bits = to_host_bits(d["k_pe"])
    out = m.mla_attn_decode(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA, rope_table=tab)
    cos, sin = rope_cos_sin(S, **KIMI_K2_ROPE)
    q_rot = apply_rope(to_f64(x["q_pe"]), rope_positions(B, 1, past_len=P), cos, sin)
    ref = mla_attention(to_f64(x["q_nope"]), q_rot, to_f64(x["k_nope"]), to_f64(k_rot_bits), to_f64(x["v"]),
                        P, ALPHA)
    got = to_host_f64(out)
    assert_parity(got, ref, f"fused rope decode B={B} H={H} P={P}")
    q2 = d["q_pe"].clone()
    m.mla_rope_apply(q2, tab, past_len=P)
    unfused = to_host_f64(m.mla_attn_decode(d["q_nope"], q2, d["k_nope"], d["k_pe"], d["v"], P, ALPHA))
    torch.cuda.synchronize()
    assert_parity(unfused, ref, "unfused")


def test_fused_prologue_paged_append():
    """mla_attn_decode_paged with rope_table and an appended token: the query
    and the new key turn at position seq_lens[b] - 1; the slot receives the
    rotated key rounded to bf16 (within half a bf16 ulp of the exact
    rotation), and the output is the oracle's attention with the rotated query
    over the cache holding that key."""
    import torch
    from oracle import mla_decode_paged
    from seeded_inputs import paged_host_inputs, paged_layout
    lens, H, bs = [1001, 1, 64, 300], 16, 32
    table, N = paged_layout(lens, bs, seed=3, spare=1)
    x = paged_host_inputs(len(lens), H, N, bs, seed=3)
    max_len = max(lens)
    log(f"case rope fused paged append lens={lens} H={H} bs={bs}")
    tab = _gpu_table(max_len, KIMI_K2_ROPE)
    d = {k: to_device(v) for k, v in x.items()}
    tb = torch.as_tensor(table, device="cuda")
    sl = torch.as_tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    m = _lib()
    out = m.mla_attn_decode_paged(d["q_nope"], d["q_pe"], d["k_nope_pages"], d["k_pe_pages"], d["v_pages"],
                                  tb, sl, max_len, ALPHA, new=(d["k_nope_new"], d["k_pe_new"], d["v_new"]),
                                  rope_table=tab)
    torch.cuda.synchronize()
    cos, sin = rope_cos_sin(max_len, **KIMI_K2_ROPE)
    pos = np.asarray(lens, dtype=np.int64)[:, None] - 1
    pages_kp = to_host_bits(d["k_pe_pages"])
    stored = np.stack([pages_kp[table[b, (L - 1) // bs], (L - 1) % bs] for b, L in enumerate(lens)])[:, None, None]
    _check_rotation(to_f64(stored), x["k_pe_new"], apply_rope(to_f64(x["k_pe_new"]), pos, cos, sin), "new key")
    q_rot = apply_rope(to_f64(x["q_pe"]), pos, cos, sin)
    ref, _ = mla_decode_paged(x["q_nope"], q_rot, x["k_nope_pages"], x["k_pe_pages"], x["v_pages"], table,
                              np.asarray(lens), ALPHA, new=(x["k_nope_new"], stored, x["v_new"]))
    assert_parity(to_host_f64(out), ref, "fused rope paged append")


@pytest.mark.parametrize("per_seq", [False, True])
def test_apply_qk_in_one_launch_equals_two_calls(per_seq):
    """mla_rope_apply_qk (the query's and the new keys' rotary parts in one
    launch) gives the same bits as two mla_rope_apply calls."""
    import torch
    B, H, T, P = 3, 16, 45, 70
    log(f"case rope apply qk B={B} H={H} T={T} P={P} per_seq={per_seq}")
    x = random_inputs(B, H, T, P, seed=60)
    kp_new = np.ascontiguousarray(x["k_pe"][:, :, P:])
    tab = _gpu_table(400, KIMI_K2_ROPE)
    lens = torch.as_tensor(np.array([0, 200, 33], dtype=np.int32), device="cuda") if per_seq else None
    m = _lib()
    q1, k1 = to_device(x["q_pe"]), to_device(kp_new)
    m.mla_rope_apply_qk(q1, k1, tab, past_len=P, past_lens=lens)
    q2, k2 = to_device(x["q_pe"]), to_device(kp_new)
    m.mla_rope_apply(q2, tab, past_len=P, past_lens=lens)
    m.mla_rope_apply(k2, tab, past_len=P, past_lens=lens)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(q1), to_host_bits(q2))
    assert np.array_equal(to_host_bits(k1), to_host_bits(k2))
    assert not np.array_equal(to_host_bits(k1), kp_new)                 # the keys did turn


def test_fused_prologue_paged_append_graph_loop():
    """A serving loop: one paged decode step with the rotary prologue fused and
    the new token appended, captured once and replayed with the lengths
    growing by one and new token rows each time. Every replay gives the same
    bits (output and pages) as eager calls on a twin cache."""
    import torch
    from seeded_inputs import paged_host_inputs, paged_layout
    lens0, H, bs, steps = [300, 45, 1000], 16, 32, 4
    cap = [L + steps for L in lens0]
    table_np, N = paged_layout(cap, bs, seed=9, spare=1)
    x = paged_host_inputs(len(lens0), H, N, bs, seed=9)
    max_len = max(cap)
    log(f"case rope fused paged graph loop lens0={lens0} H={H} bs={bs} steps={steps}")
    m = _lib()
    tab = _gpu_table(max_len, KIMI_K2_ROPE)
    tb = torch.as_tensor(table_np, device="cuda")
    pages_g = {k: to_device(x[k]) for k in ("k_nope_pages", "k_pe_pages", "v_pages")}
    pages_e = {k: v.clone() for k, v in pages_g.items()}
    inp = {k: to_device(x[k]) for k in ("q_nope", "q_pe", "k_nope_new", "k_pe_new", "v_new")}
    sl = torch.as_tensor(np.asarray(lens0, dtype=np.int32), device="cuda")
    out_g = torch.empty((len(lens0), H, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(m.mla_attn_decode_paged_workspace_bytes(len(lens0), H, max_len), 16),
                     dtype=torch.uint8, device="cuda")

    def step(pages, out):
        return m.mla_attn_decode_paged(inp["q_nope"], inp["q_pe"], pages["k_nope_pages"], pages["k_pe_pages"],
                                       pages["v_pages"], tb, sl, max_len, ALPHA,
                                       new=(inp["k_nope_new"], inp["k_pe_new"], inp["v_new"]), out=out,
                                       workspace=ws, rope_table=tab)

    scratch = {k: v.clone() for k, v in pages_g.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(scratch, out_g)                         # warm-up outside the capture, on a scratch cache
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(pages_g, out_g)
    rng = np.random.default_rng(10)
    for r in range(steps):
        sl.copy_(torch.as_tensor(np.asarray(lens0, dtype=np.int32) + r + 1, device="cuda"))
        for k in inp:
            inp[k].copy_(torch.as_tensor(rng.standard_normal(tuple(inp[k].shape)), device="cuda").to(torch.bfloat16))
        out_g.fill_(float("nan"))  # a (b, h) the replay does not merge keeps its NaN
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out_g).all().item(), f"replay {r} left rows unwritten"
        out_e = step(pages_e, torch.full_like(out_g, float("nan")))
        torch.cuda.synchronize()
        log(f"  replay {r}: lens={sl.tolist()}")
        assert np.array_equal(to_host_bits(out_g), to_host_bits(out_e)), f"output, replay {r}"
        for k in pages_g:
            assert np.array_equal(to_host_bits(pages_g[k]), to_host_bits(pages_e[k])), f"{k}, replay {r}"


def test_fused_prologue_varlen_decode():
    """mla_attn_decode_varlen with rope_table: sequence b's query turns at
    position seq_lens[b] - 1 inside the kernel, over a right-padded cache of
    keys rotated at their positions; lengths include 0 and 1."""
    import torch
    from oracle import mla_decode_varlen
    B, H, cap = 5, 16, 700
    lens = np.array([700, 1, 0, 333, 129], dtype=np.int32)
    log(f"case rope fused varlen decode lens={lens.tolist()} H={H} cap={cap}")
    x = random_inputs(B, H, 1, cap - 1, seed=70)
    tab = _gpu_table(cap, KIMI_K2_ROPE)
    d = {k: to_device(v) for k, v in x.items()}
    m = _lib()
    m.mla_rope_apply(d["k_pe"], tab, past_len=0)                  # cache rows rotated at their positions
    k_rot_bits = to_host_bits(d["k_pe"])
    out = m.mla_attn_decode_varlen(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"],
                                   torch.as_tensor(lens, device="cuda"), cap, ALPHA, rope_table=tab)
    torch.cuda.synchronize()
    cos, sin = rope_cos_sin(cap, **KIMI_K2_ROPE)
    pos = np.maximum(lens.astype(np.int64) - 1, 0)[:, None]
    q_rot = apply_rope(to_f64(x["q_pe"]), pos, cos, sin)
    ref = mla_decode_varlen(to_f64(x["q_nope"]), q_rot, to_f64(x["k_nope"]), to_f64(k_rot_bits), to_f64(x["v"]),
                            lens, ALPHA)
    got = to_host_f64(out)
    assert not np.any(got[2])                                           # empty sequence: zero row
    assert_parity(got, ref, "fused rope varlen decode")
