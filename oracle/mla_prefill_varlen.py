"""fp64 CPU oracle for a padded, variable-length prefill: each sequence of
the batch has its own number of new queries and of cached keys.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Causal mask" page, section "Construct causal mask": positions are
    numbered from the cached length, and the caller's 2D mask (1 keeps, 0
    pads) is handed with that length to the 4D mask builder (or passed down to
    the flash-attention backend when it holds a padding entry).
  * "Similarities" page, section "Query-key similarity": the attention core,
    mla_oracle.mla_attention, run here on each sequence's own rows.

Readings where the pages are silent (also listed in the design notes):
  * Right padding of both queries and keys: sequence b has T_b new queries
    (rows 0 .. T_b-1 of its [Tmax] query rows) and P_b cached keys; its keys
    are rows 0 .. P_b+T_b-1 of its [Smax] key rows, and query i sits at
    position P_b + i, seeing keys 0 .. P_b + i.
  * Padded query rows (i >= T_b) attend to nothing; their output is 0.
  * Padded rows are never read, whatever they hold.

Parity status: pinned by tests/test_oracle_prefill_varlen.py (an explicit 4D
mask built from the causal offset and the 2D padding mask over the whole
padded score matrix; NaN in every padded row; equal lengths reduce to the
dense oracle; zero queries give causal prefix means; batch permutation).
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import V_HEAD_DIM, mla_attention


def mla_prefill_varlen(q_nope, q_pe, k_nope, k_pe, v, q_lens, past_lens,
                       softmax_scale: float) -> np.ndarray:
    """Output [B, H, Tmax, 128] (fp64); rows past q_lens[b] are 0.

    q_nope [B,H,Tmax,128], q_pe [B,H,Tmax,64], k_nope / v [B,H,Smax,128],
    k_pe [B,1,Smax,64]; q_lens[b] + past_lens[b] <= Smax, q_lens[b] <= Tmax.
    """
    qn = np.asarray(q_nope)
    B, H, Tmax = qn.shape[0], qn.shape[1], qn.shape[2]
    Smax = np.asarray(k_nope).shape[2]
    tq = np.asarray(q_lens).astype(np.int64)
    pp = np.asarray(past_lens).astype(np.int64)
    if tq.shape != (B,) or pp.shape != (B,):
        raise ValueError("q_lens and past_lens must have one entry per sequence")
    if np.any(tq < 0) or np.any(tq > Tmax) or np.any(pp < 0) or np.any(tq + pp > Smax):
        raise ValueError(f"lengths out of range (Tmax={Tmax}, Smax={Smax}): {tq}, {pp}")
    out = np.zeros((B, H, Tmax, V_HEAD_DIM), dtype=np.float64)
    for b in range(B):
        T, P = int(tq[b]), int(pp[b])
        if T == 0:
            continue
        S = P + T
        out[b, :, :T] = mla_attention(qn[b:b + 1, :, :T], np.asarray(q_pe)[b:b + 1, :, :T],
                                      np.asarray(k_nope)[b:b + 1, :, :S], np.asarray(k_pe)[b:b + 1, :, :S],
                                      np.asarray(v)[b:b + 1, :, :S], P, softmax_scale)[0]
    return out


__all__ = ["mla_prefill_varlen"]
