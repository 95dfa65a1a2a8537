"""fp64 CPU oracle for the rotary prologue: YaRN-scaled RoPE on the 64 rotary dims.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests, the smoke
check and the benchmark's CPU-baseline leg call it; the HIP library never does.

What it follows (Kimi K2 on the OpenModelAtlas pages):
  * "Similarities" page, section "Query-key similarity": before the rotary
    parts join the non-rotary ones, q_pe and k_pe are rotated with a cos/sin
    table built for kv_seq_len positions and picked by position ids; the same
    cos/sin go along with the cache update.
  * The released configuration printed on the "Embedded" and "Logits" pages
    (section on the configuration): qk_rope_head_dim 64, rope_theta 50000 and
    a "yarn" rope_scaling with factor 32, original_max_position_embeddings
    4096, beta_fast = beta_slow = 1 and mscale = mscale_all_dim = 1.

Readings where the pages are silent (they print neither the rotation nor the
YaRN formula; also listed in the design notes):
  * The rotation is RoPE as published by Su et al. (RoFormer, 2021): dims
    (2i, 2i+1) form pair i, turned by the angle pos * w_i with
    w_i = theta^(-2i/64); a pair (x, y) becomes
    (x cos a - y sin a, x sin a + y cos a).
  * The frequencies are scaled as YaRN (Peng et al., 2023) does per pair
    ("NTK-by-parts"): with wavelength lambda_i = 2 pi / w_i, the ratio
    r_i = L / lambda_i (L = original_max_position_embeddings) and the ramp
    g_i = 0 for r_i < alpha, 1 for r_i >= beta, (r_i - alpha)/(beta - alpha)
    between (alpha = beta_slow, beta = beta_fast), the pair turns at
    w_i' = g_i w_i + (1 - g_i) w_i / s, s = factor. With alpha = beta = 1 the
    ramp is a step: pairs whose wavelength is longer than L are slowed by s
    (pairs 20..31 for the released configuration), the others keep w_i.
  * YaRN's attention temperature (mscale) is not part of the table: the
    configuration gives mscale = mscale_all_dim, whose ratio is 1, and a logit
    temperature is what softmax_scale, an argument of the attention calls,
    carries.
  * New token i of sequence b sits at position past_len (or past_lens[b]) + i,
    the same positions the causal mask uses; cached keys were rotated at their
    own positions when they were appended.

Parity status: pinned by tests/test_oracle_rope.py (factor 1 is textbook RoPE,
checked against complex multiplication by exp(i pos w); the released
configuration's frequencies against the hand-derived step between pairs 19
and 20; the ramp's end points and its midpoint; hand-computed rotations of unit
vectors; position 0 is the identity; pair norms are kept; scores depend on the
relative position only; attention over rotated inputs is unchanged when every
position shifts by the same amount).
"""

import math

import numpy as np

ROPE_DIM = 64  # qk_rope_head_dim
ROPE_PAIRS = ROPE_DIM // 2

# The released configuration's rotary settings.
KIMI_K2_ROPE = dict(theta=50000.0, factor=32.0, original_max_position=4096,
                    beta_fast=1.0, beta_slow=1.0)


def yarn_inv_freq(theta=50000.0, factor=32.0, original_max_position=4096,
                  beta_fast=1.0, beta_slow=1.0, rotary_dim=ROPE_DIM) -> np.ndarray:
    """Angle per position of each pair, fp64 [rotary_dim / 2] (readings above)."""
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    w = np.power(float(theta), -2.0 * i / rotary_dim)           # RoPE frequencies
    if factor == 1.0:
        return w
    r = float(original_max_position) * w / (2.0 * math.pi)      # turns within the original length
    lo, hi = float(beta_slow), float(beta_fast)
    g = np.empty_like(r)
    for k in range(r.size):                                      # ramp, pair by pair
        if r[k] >= hi:
            g[k] = 1.0
        elif r[k] < lo:
            g[k] = 0.0
        else:
            g[k] = (r[k] - lo) / (hi - lo)
    return g * w + (1.0 - g) * w / float(factor)


def rope_cos_sin(max_pos: int, **cfg):
    """cos and sin of pos * w_i' for positions 0..max_pos-1, fp64 [max_pos, 32] each."""
    w = yarn_inv_freq(**cfg)
    ang = np.arange(int(max_pos), dtype=np.float64)[:, None] * w[None, :]
    return np.cos(ang), np.sin(ang)


def rope_positions(B: int, T: int, past_len=0, past_lens=None) -> np.ndarray:
    """Absolute position of new token i of sequence b, int64 [B, T]."""
    base = np.full(B, past_len, dtype=np.int64) if past_lens is None else np.asarray(past_lens, dtype=np.int64)
    return base[:, None] + np.arange(T, dtype=np.int64)[None, :]


def apply_rope(x: np.ndarray, positions: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate x [B, R, T, 64] (R heads, or 1 for the shared rotary key) at
    positions [B, T]; every head of a sequence uses the same positions."""
    x = np.asarray(x, dtype=np.float64)
    B, R, T, D = x.shape
    assert D == ROPE_DIM and positions.shape == (B, T)
    out = np.empty_like(x)
    for b in range(B):
        c = cos[positions[b]]                  # [T, 32]
        s = sin[positions[b]]
        ev, od = x[b, :, :, 0::2], x[b, :, :, 1::2]
        out[b, :, :, 0::2] = ev * c - od * s
        out[b, :, :, 1::2] = ev * s + od * c
    return out
