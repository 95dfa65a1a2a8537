"""fp64 CPU oracle for decode over the compressed (latent) key-value cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Similarities" page, section "Scale scores" (the attention module's
    __init__): the joint key-value down-projection emits a latent of
    kv_lora_rank dims plus the one shared rotary key; after the latent's
    RMSNorm, kv_b_proj (no bias) maps kv_lora_rank -> num_heads *
    (q_head_dim - qk_rope_head_dim + v_head_dim), i.e. 128 non-rotary key dims
    plus 128 value dims per head.
  * "Embedded state" page, config.json excerpt: kv_lora_rank 512, 64 heads,
    qk_nope_head_dim 128, qk_rope_head_dim 64, v_head_dim 128.
  * "Similarities" page, "Query-key similarity": the attention core itself,
    which this module does not re-implement: it decompresses the keys and
    values and calls mla_oracle.mla_attention.

Readings where the pages are silent (also listed in the design notes):
  * The forward split of kv_b_proj's output is not printed. Reading: for head
    h, output features [256h, 256h+128) are the head's non-rotary key and
    [256h+128, 256h+256) its value (the order in which the module's constants
    add up, q_head_dim - qk_rope_head_dim, then v_head_dim).
  * The latent passed in is the normalised latent (after the latent RMSNorm),
    which is what kv_b_proj consumes; the norm itself is upstream.
  * Decode only (one new query per sequence); S = past_len + 1 keys.

Parity status: pinned by tests/test_oracle_latent.py (selector weights that
reduce it to the pinned attention oracle on slices of the latent, per-head
scaling, and the absorbed evaluation order computed independently).
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import QK_NOPE_HEAD_DIM, QK_ROPE_HEAD_DIM, V_HEAD_DIM, _as_f64, mla_attention

KV_LORA_RANK = 512                              # config.json: kv_lora_rank
KV_B_PER_HEAD = QK_NOPE_HEAD_DIM + V_HEAD_DIM   # kv_b_proj output features per head (256)


def decompress_kv(c_kv, w_kv_b, num_heads: int):
    """Keys and values of every head from the normalised latent.

    c_kv [B, S, 512] (bf16 bits or floats), w_kv_b [H*256, 512] (kv_b_proj's
    weight, [out_features, in_features] as nn.Linear stores it). Returns
    k_nope [B, H, S, 128] and v [B, H, S, 128] in fp64:
    kv[b, s, :] = w_kv_b @ c_kv[b, s, :], head h owning features [256h, 256h+256).
    """
    c = _as_f64(c_kv)
    w = _as_f64(w_kv_b)
    if c.ndim != 3 or c.shape[-1] != KV_LORA_RANK:
        raise ValueError(f"latent shape {c.shape} is not [B,S,{KV_LORA_RANK}]")
    if w.shape != (num_heads * KV_B_PER_HEAD, KV_LORA_RANK):
        raise ValueError(f"kv_b_proj weight shape {w.shape} is not "
                         f"[{num_heads * KV_B_PER_HEAD},{KV_LORA_RANK}]")
    B, S, _ = c.shape
    kv = c @ w.T                                            # [B, S, H*256]
    kv = kv.reshape(B, S, num_heads, KV_B_PER_HEAD).transpose(0, 2, 1, 3)
    return kv[..., :QK_NOPE_HEAD_DIM], kv[..., QK_NOPE_HEAD_DIM:]


def mla_decode_latent(q_nope, q_pe, c_kv, k_pe, w_kv_b, past_len: int, softmax_scale: float):
    """Decode output [B, H, 1, 128] in fp64, attending over decompressed keys/values.

    q_nope [B,H,1,128], q_pe [B,H,1,64] (post-RoPE), c_kv [B,S,512] normalised
    latent, k_pe [B,1,S,64] shared rotary key (post-RoPE), w_kv_b [H*256,512],
    S = past_len + 1. The keys' non-rotary parts and the values come from
    kv_b_proj applied to the latent; the attention core is mla_attention.
    """
    qn = np.asarray(q_nope)
    if qn.ndim != 4 or qn.shape[2] != 1:
        raise ValueError(f"decode takes one query per sequence, got q_nope {qn.shape}")
    B, H = qn.shape[0], qn.shape[1]
    k_nope, v = decompress_kv(c_kv, w_kv_b, H)
    if k_nope.shape[0] != B:
        raise ValueError(f"latent batch {k_nope.shape[0]} != query batch {B}")
    return mla_attention(q_nope, q_pe, k_nope, k_pe, v, past_len, softmax_scale)


def mla_decode_latent_rows(q_nope, q_pe, c_kv, k_pe, w_kv_b, past_len: int, softmax_scale: float,
                           rows) -> np.ndarray:
    """The same definition at the requested (b, h) rows only: [len(rows), 128].

    Decompresses the keys and values of one (b, h) at a time, so large
    batches can be checked on samples.
    """
    out = np.empty((len(rows), V_HEAD_DIM), dtype=np.float64)
    w = _as_f64(w_kv_b)
    for n, (b, h) in enumerate(rows):
        c = _as_f64(c_kv[b])                                    # [S, 512]
        wk = w[h * KV_B_PER_HEAD:h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM]
        wv = w[h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM:(h + 1) * KV_B_PER_HEAD]
        k_nope = (c @ wk.T)[None, None]                         # head h's block of decompress_kv
        v = (c @ wv.T)[None, None]
        o = mla_attention(np.asarray(q_nope)[b:b + 1, h:h + 1], np.asarray(q_pe)[b:b + 1, h:h + 1],
                          k_nope, np.asarray(k_pe)[b:b + 1], v, past_len, softmax_scale)
        out[n] = o[0, 0, 0]
    return out


__all__ = ["KV_LORA_RANK", "KV_B_PER_HEAD", "decompress_kv", "mla_decode_latent",
           "mla_decode_latent_rows", "QK_ROPE_HEAD_DIM"]
