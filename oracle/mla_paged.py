"""fp64 CPU oracle for decode over a paged key-value cache, with the new
token's key and value optionally appended by the call.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Similarities" page, section "Query-key similarity": the new key and
    value states go through the cache's update, which appends them to the
    sequence's cached keys and values, and the new query then attends over
    all of them; the attention core is mla_oracle.mla_attention.
  * "Causal mask" page, section "Construct causal mask": positions are
    numbered from the cached length, so the appended token is position
    L_b - 1 of a sequence that holds L_b keys after the append.

Readings where the pages are silent (also listed in the design notes):
  * The pages keep the cache as one growing tensor per layer; a paged cache
    stores the same rows in fixed-size blocks. Sequence b's key j lives in
    block block_table[b, j // block_size], row j % block_size. Blocks are laid
    out [num_blocks, H, block_size, 128] for k_nope and v, [num_blocks,
    block_size, 64] for the shared rotary key.
  * seq_lens[b] counts the keys after the append. With new rows given, row
    L_b - 1 is overwritten with them before attending; without, the cache is
    read as it is. Rows past L_b are never read; L_b = 0 gives a zero row.

Parity status: pinned by tests/test_oracle_paged.py (a contiguous block table
reduces to the pinned variable-length oracle; relabelling physical blocks
leaves outputs bit-identical; NaN in blocks and rows no sequence owns changes
nothing; appending equals writing the rows first and decoding without
append; one-key sequences return the appended value).
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import V_HEAD_DIM, _as_f64
from .mla_varlen import mla_decode_varlen


def gather_sequence(pages, block_table, b: int, L: int, block_size: int, head_axis: bool):
    """Rows 0 .. L-1 of sequence b from a paged tensor, in key order:
    [H, L, D] when the pages carry a head axis, else [L, D]."""
    rows = []
    for j in range(L):
        blk = int(block_table[b, j // block_size])
        r = j % block_size
        rows.append(pages[blk, :, r] if head_axis else pages[blk, r])
    if not rows:
        shape = (pages.shape[1], 0, pages.shape[-1]) if head_axis else (0, pages.shape[-1])
        return np.zeros(shape, dtype=pages.dtype)
    return np.stack(rows, axis=1 if head_axis else 0)


def append_rows(k_nope_pages, k_pe_pages, v_pages, block_table, seq_lens, block_size,
                k_nope_new, k_pe_new, v_new):
    """The cache after the update: copies of the pages with row L_b - 1 of
    every sequence (L_b >= 1) replaced by the new key and value."""
    kn, kp, vv = np.array(k_nope_pages), np.array(k_pe_pages), np.array(v_pages)
    for b, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        if L < 1:
            continue
        blk = int(block_table[b, (L - 1) // block_size])
        r = (L - 1) % block_size
        kn[blk, :, r] = np.asarray(k_nope_new)[b, :, 0]
        vv[blk, :, r] = np.asarray(v_new)[b, :, 0]
        kp[blk, r] = np.asarray(k_pe_new)[b, 0, 0]
    return kn, kp, vv


def mla_decode_paged(q_nope, q_pe, k_nope_pages, k_pe_pages, v_pages, block_table, seq_lens,
                     softmax_scale: float, new=None):
    """Decode output [B, H, 1, 128] (fp64) and the pages after the call.

    new: None, or (k_nope_new [B,H,1,128], k_pe_new [B,1,1,64], v_new
    [B,H,1,128]) appended at row seq_lens[b] - 1 before attending.
    Returns (out, (k_nope_pages, k_pe_pages, v_pages)).
    """
    block_table = np.asarray(block_table)
    lens = np.asarray(seq_lens).astype(np.int64)
    B, H = np.asarray(q_nope).shape[:2]
    bs = np.asarray(k_pe_pages).shape[1]
    if np.any(lens < 0) or np.any(lens > block_table.shape[1] * bs):
        raise ValueError(f"sequence lengths must lie in [0, {block_table.shape[1] * bs}]")
    kn, kp, vv = k_nope_pages, k_pe_pages, v_pages
    if new is not None:
        kn, kp, vv = append_rows(kn, kp, vv, block_table, lens, bs, *new)
    cap = max(int(lens.max()) if B else 0, 1)
    # contiguous caches [B, H, cap, .] holding each sequence's rows, then the
    # variable-length definition
    ck = np.zeros((B, H, cap, np.asarray(kn).shape[-1]), dtype=np.float64)
    cp = np.zeros((B, 1, cap, np.asarray(kp).shape[-1]), dtype=np.float64)
    cv = np.zeros((B, H, cap, V_HEAD_DIM), dtype=np.float64)
    kn64, kp64, vv64 = _as_f64(kn), _as_f64(kp), _as_f64(vv)
    for b in range(B):
        L = int(lens[b])
        ck[b, :, :L] = gather_sequence(kn64, block_table, b, L, bs, True)
        cp[b, 0, :L] = gather_sequence(kp64, block_table, b, L, bs, False)
        cv[b, :, :L] = gather_sequence(vv64, block_table, b, L, bs, True)
    out = mla_decode_varlen(q_nope, q_pe, ck, cp, cv, lens, softmax_scale)
    return out, (kn, kp, vv)


__all__ = ["gather_sequence", "append_rows", "mla_decode_paged"]
