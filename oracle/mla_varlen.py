"""fp64 CPU oracle for decode over a preallocated, right-padded cache with a
length per sequence.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Causal mask" page, section "Construct causal mask": the model hands the
    caller's 2D attention mask (1 keeps a position, 0 marks padding) and the
    cached length to the 4D mask builder; with the flash-attention backend
    the 2D mask itself is passed down whenever it holds a padding entry.
  * "Similarities" page, section "Query-key similarity": the cache's update
    appends the new key and value states, and the new query then attends over
    every cached key of its sequence; the attention core itself is
    mla_oracle.mla_attention, called on each sequence's valid keys.

Readings where the pages are silent (also listed in the design notes):
  * Right padding. Sequence b owns rows [0, L_b) of its cache rows; rows
    L_b .. cap-1 are padding, i.e. the 2D mask [1]*L_b + [0]*(cap - L_b).
    The new token is the last valid key, so its query sees keys 0 .. L_b - 1
    (past_len = L_b - 1). Padding rows are never read: any bits may sit there.
  * A sequence with no valid key (L_b = 0) has an all-masked score row, for
    which the softmax is undefined (all weights exp(-inf)). Convention: its
    output is 0.
  * The cache is [B, H, cap, 128] for k_nope and v and [B, 1, cap, 64] for the
    shared rotary key, with cap >= every L_b.

Parity status: pinned by tests/test_oracle_varlen.py (padding filled with NaN
leaves every output unchanged, an explicit 2D padding mask added to the whole
cache's scores, closed forms for zero queries and one-key sequences, the
zero-length convention, batch permutation).
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import V_HEAD_DIM, mla_attention


def _check(q_nope, k_nope_cache, seq_lens):
    qn = np.asarray(q_nope)
    if qn.ndim != 4 or qn.shape[2] != 1:
        raise ValueError(f"decode takes one query per sequence, got q_nope {qn.shape}")
    B, H = qn.shape[0], qn.shape[1]
    kc = np.asarray(k_nope_cache)
    if kc.ndim != 4 or kc.shape[0] != B or kc.shape[1] != H:
        raise ValueError(f"k_nope cache {kc.shape} does not match queries {qn.shape}")
    cap = kc.shape[2]
    lens = np.asarray(seq_lens).astype(np.int64)
    if lens.shape != (B,):
        raise ValueError(f"seq_lens shape {lens.shape} is not ({B},)")
    if np.any(lens < 0) or np.any(lens > cap):
        raise ValueError(f"sequence lengths must lie in [0, {cap}], got {lens.tolist()}")
    return B, H, cap, lens


def mla_decode_varlen_rows(q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens,
                           softmax_scale: float, rows) -> np.ndarray:
    """Output rows [len(rows), 128] (fp64) for the requested (b, h) pairs."""
    B, H, cap, lens = _check(q_nope, k_nope_cache, seq_lens)
    out = np.zeros((len(rows), V_HEAD_DIM), dtype=np.float64)
    for n, (b, h) in enumerate(rows):
        L = int(lens[b])
        if L == 0:
            continue  # no valid key: output 0 by convention
        o = mla_attention(np.asarray(q_nope)[b:b + 1, h:h + 1], np.asarray(q_pe)[b:b + 1, h:h + 1],
                          np.asarray(k_nope_cache)[b:b + 1, h:h + 1, :L],
                          np.asarray(k_pe_cache)[b:b + 1, :, :L],
                          np.asarray(v_cache)[b:b + 1, h:h + 1, :L], L - 1, softmax_scale)
        out[n] = o[0, 0, 0]
    return out


def mla_decode_varlen(q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens,
                      softmax_scale: float) -> np.ndarray:
    """Decode output [B, H, 1, 128] in fp64: sequence b attends over cache rows
    [0, seq_lens[b]) of its k_nope / k_pe / v cache rows."""
    B, H, cap, lens = _check(q_nope, k_nope_cache, seq_lens)
    out = np.zeros((B, H, 1, V_HEAD_DIM), dtype=np.float64)
    for b in range(B):
        L = int(lens[b])
        if L == 0:
            continue
        out[b] = mla_attention(np.asarray(q_nope)[b:b + 1], np.asarray(q_pe)[b:b + 1],
                               np.asarray(k_nope_cache)[b:b + 1, :, :L],
                               np.asarray(k_pe_cache)[b:b + 1, :, :L],
                               np.asarray(v_cache)[b:b + 1, :, :L], L - 1, softmax_scale)[0]
    return out


__all__ = ["mla_decode_varlen", "mla_decode_varlen_rows"]
