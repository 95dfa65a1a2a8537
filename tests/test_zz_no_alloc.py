"""mla_attn_decode_noalloc (the decode whose scratch is a library-owned
per-device array) against mla_attn_decode with a caller's workspace, through
the C ABI: two calls in a row, the second on a smaller input, each equal bit
for bit to the workspace call and within the parity bar of the oracle."""

import numpy as np
import pytest

from oracle import mla_attention
from seeded_inputs import random_inputs

from _gpu_util import assert_parity, log, to_host_bits, to_host_f64, upload

pytestmark = pytest.mark.gpu

ALPHA = float(np.float32(192.0 ** -0.5))


def _both(B, H, P, seed):
    import torch
    import attention_mla_causal_amd as m
    x = random_inputs(B, H, 1, P, seed=seed)
    d = upload(x)
    args = (d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], P, ALPHA)
    ws = torch.full((max(m.mla_attn_decode_workspace_bytes(B, H, P + 1), 16),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    a = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    b = torch.full((B, H, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    m.mla_attn_decode(*args, out=a, workspace=ws)
    m.mla_attn_decode_noalloc(*args, out=b)
    torch.cuda.synchronize()
    return x, a, b


# (B, H, past_len): the first call splits each head's 1001 keys over 8
# workgroups merged inside the kernel (the pages' decode); the second, smaller
# one uses fewer splits and rows of the array the first left behind; the third
# splits a 5-head call whose partials a second kernel merges.
CALLS = [(1, 64, 1000, 0), (1, 16, 300, 1), (1, 5, 1999, 2)]


def test_noalloc_matches_workspace_decode_on_calls_in_a_row():
    import attention_mla_causal_amd as m
    for B, H, P, seed in CALLS:
        log(f"case noalloc decode B={B} H={H} P={P} ws={m.mla_attn_decode_workspace_bytes(B, H, P + 1)}")
        x, a, b = _both(B, H, P, seed)
        assert np.array_equal(to_host_bits(a), to_host_bits(b)), f"B={B} H={H} P={P}"
        assert_parity(to_host_f64(b), mla_attention(x["q_nope"], x["q_pe"], x["k_nope"], x["k_pe"], x["v"], P,
                                                    ALPHA), f"noalloc B={B} H={H} P={P}")


def test_noalloc_without_split_and_errors():
    import torch
    import attention_mla_causal_amd as m
    # B*H >= 256: no split, so no scratch at all
    x, a, b = _both(2, 128, 200, 3)
    assert np.array_equal(to_host_bits(a), to_host_bits(b))
    # errors are checked on the host as for mla_attn_decode
    d = upload(random_inputs(1, 4, 1, 10, seed=4))
    with pytest.raises(ValueError):
        m.mla_attn_decode_noalloc(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], 9, ALPHA)  # S = 11 keys != past_len + 1
    with pytest.raises(m.MLAError):
        m.mla_attn_decode_noalloc(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], 10, float("nan"))
    torch.cuda.synchronize()
