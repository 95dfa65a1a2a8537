"""fp64 CPU oracle for the causal multi-head latent attention (MLA) core.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg call this module; the HIP library never does. It is written to
be read against the pages, not to be fast: every score, the mask and every
softmax row are materialised, one (batch, head) at a time, with no tiling, no
online softmax and no re-association beyond one library matmul per product.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Similarities" page, section "Query-key similarity" (the attention-core
    excerpt of modeling_deepseek.py): the query of each head joins its 128
    non-rotary dims and its 64 rotary dims; the key joins the head's 128
    non-rotary dims and the rotary key, which is one tensor shared by all heads;
    scores are the matmul of queries with transposed keys times
    ``softmax_scale``; the scores must have shape (B, H, T, kv_seq_len) and the
    mask (B, 1, T, kv_seq_len), else ValueError; the mask is added; softmax
    runs along the keys in fp32 (here fp64); dropout; matmul with the values.
  * "Weighted sum of values" page: the value mix, [B,64,T,S] x [B,64,S,128]
    -> [B,64,T,128].
  * "Causal mask" page, section "Construct causal mask": positions are
    numbered from the cached length P, so new query i sits at absolute
    position P+i; the 4D causal mask is built with that length.
  * "Embedded state" page, config.json excerpt: 64 heads, qk_nope_head_dim 128,
    qk_rope_head_dim 64, v_head_dim 128, attention_dropout 0.0.
  * "Similarities" page, section "Scale scores": the joint key-value
    down-projection also emits the single shared rotary key.

Readings where the pages are silent (each is listed with its reason in the
repository's design notes):
  * softmax_scale is not printed; it is an argument. It crosses the C ABI as
    a 32-bit float, so the oracle rounds it to fp32 first and then works in
    fp64, making both sides use the same scalar.
  * The body of the 4D mask builder is not printed. Reading: key j is visible
    to query i iff j <= P + i (bottom-right aligned, since query i is at
    absolute position P+i); hidden entries are -inf. Every row keeps key 0,
    so no row is ever fully hidden and exp(-inf) makes hidden weights exactly 0.
  * kv_seq_len is P + T; keys and values are [B, H, S, 128] with S = P + T.
  * Dropout is the identity (p = 0.0 and inference).
  * The real-number result is the definition: everything here is fp64 and
    no bf16 rounding of intermediate scores or weights is emulated.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (closed forms, invariants, brute force and an
independent library attention routine).
"""

from __future__ import annotations

import numpy as np

QK_NOPE_HEAD_DIM = 128  # config.json: qk_nope_head_dim
QK_ROPE_HEAD_DIM = 64   # config.json: qk_rope_head_dim
V_HEAD_DIM = 128        # config.json: v_head_dim
Q_HEAD_DIM = QK_NOPE_HEAD_DIM + QK_ROPE_HEAD_DIM  # joined query / key width


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 numbers given as their uint16 bit patterns.

    A bf16 number is the upper half of an IEEE binary32, so widening the bits
    and reinterpreting them is exact; fp32 -> fp64 is exact too.
    """
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return x.astype(np.float64, copy=False)


def causal_mask_4d(batch: int, q_len: int, past_len: int) -> np.ndarray:
    """Additive 4D causal mask, shape (B, 1, T, P+T), entries 0 or -inf.

    "Causal mask" page, section "Construct causal mask": the mask is built
    from (batch, seq_length) and the cached length. New query i is at absolute
    position P+i and may attend to every key at a position <= P+i.
    """
    kv_len = past_len + q_len
    i = np.arange(q_len)[:, None]
    j = np.arange(kv_len)[None, :]
    m = np.where(j <= past_len + i, 0.0, -np.inf)
    return np.broadcast_to(m, (batch, 1, q_len, kv_len)).copy()


def _check_inputs(qn, qp, kn, kp, v, past_len):
    if qn.ndim != 4 or qp.ndim != 4 or kn.ndim != 4 or kp.ndim != 4 or v.ndim != 4:
        raise ValueError("all inputs must be 4D")
    B, H, T, dn = qn.shape
    S = kn.shape[2]
    if dn != QK_NOPE_HEAD_DIM or qp.shape != (B, H, T, QK_ROPE_HEAD_DIM):
        raise ValueError(f"query shapes {qn.shape}, {qp.shape} do not match [B,H,T,128]/[B,H,T,64]")
    if kn.shape != (B, H, S, QK_NOPE_HEAD_DIM) or v.shape != (B, H, S, V_HEAD_DIM):
        raise ValueError(f"key/value shapes {kn.shape}, {v.shape} do not match [B,H,S,128]")
    if kp.shape != (B, 1, S, QK_ROPE_HEAD_DIM):
        raise ValueError(f"shared rotary key shape {kp.shape} is not [B,1,S,64]")
    if past_len < 0 or S != past_len + T:
        raise ValueError(f"kv_seq_len {S} != past_len {past_len} + q_len {T}")
    return B, H, T, S


def _joined_query_key(qn, qp, kn, kp, b, h):
    """Query [T,192] and key [S,192] of head h, as the attention core joins them.

    "Similarities" page, "Query-key similarity": the first 128 query dims are
    q_nope and the last 64 are q_pe; the first 128 key dims are the head's
    k_nope and the last 64 are the one rotary key shared by every head.
    """
    query = np.concatenate([qn[b, h], qp[b, h]], axis=-1)
    key = np.concatenate([kn[b, h], kp[b, 0]], axis=-1)
    return query, key


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    """Softmax along the last axis: exp(z - max) / sum(exp(z - max))."""
    zmax = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - zmax)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_probs(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float) -> np.ndarray:
    """Softmax weights [B, H, T, S] in fp64 (scores, scale, mask, softmax).

    "Similarities" page, "Query-key similarity": scores are the matmul of the
    joined queries with the transposed joined keys, times softmax_scale; the
    4D mask is added; softmax runs along the keys.
    """
    qn, qp, kn, kp, vv = (_as_f64(x) for x in (q_nope, q_pe, k_nope, k_pe, v))
    B, H, T, S = _check_inputs(qn, qp, kn, kp, vv, past_len)
    alpha = float(np.float32(softmax_scale))
    mask = causal_mask_4d(B, T, past_len)
    if mask.shape != (B, 1, T, S):
        raise ValueError(f"Attention mask should be of size {(B, 1, T, S)}, but is {mask.shape}")
    probs = np.empty((B, H, T, S), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            query, key = _joined_query_key(qn, qp, kn, kp, b, h)
            scores = (query @ key.T) * alpha
            if scores.shape != (T, S):
                raise ValueError(f"Attention weights should be of size {(T, S)}, but is {scores.shape}")
            probs[b, h] = _softmax_rows(scores + mask[b, 0])
    return probs


def mla_attention(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float) -> np.ndarray:
    """Attention output [B, H, T, 128] in fp64.

    Inputs are uint16 bf16 bit patterns (converted exactly) or float arrays:
    q_nope [B,H,T,128], q_pe [B,H,T,64], k_nope [B,H,S,128],
    k_pe [B,1,S,64] (one rotary key for all heads), v [B,H,S,128], S = P+T.
    Decode is the same call with T = 1: the pages run one code path for both.

    "Weighted sum of values" page: output = weights @ values per head. One
    (batch, head) at a time so that only one T x S matrix is alive.
    """
    qn, qp, kn, kp, vv = (_as_f64(x) for x in (q_nope, q_pe, k_nope, k_pe, v))
    B, H, T, S = _check_inputs(qn, qp, kn, kp, vv, past_len)
    alpha = float(np.float32(softmax_scale))
    mask = causal_mask_4d(1, T, past_len)[0, 0]
    out = np.empty((B, H, T, V_HEAD_DIM), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            query, key = _joined_query_key(qn, qp, kn, kp, b, h)
            scores = (query @ key.T) * alpha
            if scores.shape != (T, S):
                raise ValueError(f"Attention weights should be of size {(T, S)}, but is {scores.shape}")
            probs = _softmax_rows(scores + mask)
            out[b, h] = probs @ vv[b, h]
    return out


def mla_attention_rows(q_nope, q_pe, k_nope, k_pe, v, past_len: int, softmax_scale: float,
                       rows) -> np.ndarray:
    """The same definition evaluated only at the requested (b, h, i) rows.

    Used where the full output is too large for the CPU: each requested row
    is its query's scores against all S keys, the row of the 4D mask, the
    softmax and the value mix, exactly as in mla_attention. Inputs may be
    uint16 bf16 bits or float arrays, and may be lazily indexed arrays
    (e.g. numpy memmaps) since only rows of the requested heads are read.
    Returns [len(rows), 128].
    """
    alpha = float(np.float32(softmax_scale))
    B, H, T = q_nope.shape[0], q_nope.shape[1], q_nope.shape[2]
    S = k_nope.shape[2]
    if S != past_len + T or past_len < 0:
        raise ValueError(f"kv_seq_len {S} != past_len {past_len} + q_len {T}")
    out = np.empty((len(rows), V_HEAD_DIM), dtype=np.float64)
    by_head: dict = {}
    for n, (b, h, i) in enumerate(rows):
        if not (0 <= b < B and 0 <= h < H and 0 <= i < T):
            raise ValueError(f"row {(b, h, i)} outside [{B},{H},{T}]")
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        key = np.concatenate([_as_f64(k_nope[b, h]), _as_f64(k_pe[b, 0])], axis=-1)
        vv = _as_f64(v[b, h])
        qi = [i for _, i in items]
        query = np.concatenate([_as_f64(q_nope[b, h, qi]), _as_f64(q_pe[b, h, qi])], axis=-1)
        scores = (query @ key.T) * alpha
        j = np.arange(S)[None, :]
        mask = np.where(j <= past_len + np.asarray(qi)[:, None], 0.0, -np.inf)
        probs = _softmax_rows(scores + mask)
        res = probs @ vv
        for r, (n, _) in enumerate(items):
            out[n] = res[r]
    return out
