"""fp64 CPU oracle for the attention core with the caller's 2D padding mask.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Causal mask" page, section "Construct causal mask": the caller's 2D
    attention mask (1 keeps a position, 0 pads it) is handed, with the cached
    length, to the 4D causal-mask builder, whose output the attention core adds
    to its scores.
  * "Similarities" page, section "Query-key similarity": the attention core
    (joined query and key, the one rotary key shared by every head, scale,
    mask, fp32 softmax, value mix), as in mla_oracle.

Readings where the pages are silent (also listed in the design notes):
  * The 2D mask spans every key position, cached and new: [B, S] with
    S = past_len + T, entry [b, j] for key j of sequence b.
  * The 4D builder combines the two masks: key j is visible to query i of
    sequence b iff j <= past_len + i (causal, query i at position past_len + i)
    and mask[b, j] != 0. A hidden entry of either stays hidden.
  * A query with no visible key (e.g. a left-padding position) has no defined
    softmax; its output is 0, the same convention as the variable-length calls.
  * Hidden keys are never read: the softmax and the value mix run over the
    visible keys only, so whatever a hidden row holds (NaN included) cannot
    reach the output.

Parity status: pinned by tests/test_oracle_masked.py (an all-ones mask is the
dense oracle; right padding in decode is the variable-length decode oracle;
left padding equals the unpadded sequence with a shorter cache; NaN in every
hidden row changes no bit; brute force with math.fsum on tiny random masks;
rows with no visible key are 0).
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import V_HEAD_DIM, _as_f64, _joined_query_key, _softmax_rows


def visible_keys(attn_mask, q_len: int, past_len: int) -> np.ndarray:
    """The combined 4D mask as booleans [B, T, S]: causal offset by past_len
    AND the 2D mask (nonzero keeps)."""
    m = np.asarray(attn_mask) != 0
    B, S = m.shape
    if S != past_len + q_len or past_len < 0:
        raise ValueError(f"2D mask covers {S} keys, expected past_len {past_len} + q_len {q_len}")
    i = np.arange(q_len)[:, None]
    j = np.arange(S)[None, :]
    causal = j <= past_len + i
    return causal[None, :, :] & m[:, None, :]


def mla_attention_masked(q_nope, q_pe, k_nope, k_pe, v, attn_mask, past_len: int,
                         softmax_scale: float) -> np.ndarray:
    """Attention output [B, H, T, 128] (fp64) under the causal mask and the
    caller's 2D padding mask attn_mask [B, S] (S = past_len + T).

    Shapes as mla_oracle.mla_attention. Rows with no visible key are 0.
    """
    qn, qp, kn, kp, vv = (_as_f64(x) for x in (q_nope, q_pe, k_nope, k_pe, v))
    B, H, T = qn.shape[0], qn.shape[1], qn.shape[2]
    S = kn.shape[2]
    if np.asarray(attn_mask).shape != (B, S):
        raise ValueError(f"attn_mask must be [{B}, {S}], got {np.asarray(attn_mask).shape}")
    vis = visible_keys(attn_mask, T, past_len)
    alpha = float(np.float32(softmax_scale))
    out = np.zeros((B, H, T, V_HEAD_DIM), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            query, key = _joined_query_key(qn, qp, kn, kp, b, h)
            for i in range(T):
                cols = np.nonzero(vis[b, i])[0]
                if cols.size == 0:
                    continue
                z = (query[i] @ key[cols].T) * alpha
                p = _softmax_rows(z[None, :])[0]
                out[b, h, i] = p @ vv[b, h, cols]
    return out


__all__ = ["visible_keys", "mla_attention_masked"]
