"""The latent-cache oracle's pins catch plausible mistakes (CPU only): each
case plants one mistake in a copy of oracle/mla_latent.py's source, swaps the
copy into tests/test_oracle_latent.py and runs every pin there; at least one
must fail, and the unchanged copy must pass them all."""

import pytest

import test_oracle_latent as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_latent")
NAMES = ("decompress_kv", "mla_decode_latent", "mla_decode_latent_rows")

MUTANTS = {
    "value half taken as the key": [
        ("return kv[..., :QK_NOPE_HEAD_DIM], kv[..., QK_NOPE_HEAD_DIM:]",
         "return kv[..., QK_NOPE_HEAD_DIM:], kv[..., :QK_NOPE_HEAD_DIM]"),
        ("wk = w[h * KV_B_PER_HEAD:h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM]",
         "wk = w[h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM:(h + 1) * KV_B_PER_HEAD]"),
        ("wv = w[h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM:(h + 1) * KV_B_PER_HEAD]",
         "wv = w[h * KV_B_PER_HEAD:h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM]")],
    "head blocks interleaved": [
        ("kv = kv.reshape(B, S, num_heads, KV_B_PER_HEAD).transpose(0, 2, 1, 3)",
         "kv = kv.reshape(B, S, KV_B_PER_HEAD, num_heads).transpose(0, 3, 1, 2)")],
    "rotary query dropped": [
        ("return mla_attention(q_nope, q_pe, k_nope, k_pe, v, past_len, softmax_scale)",
         "return mla_attention(q_nope, 0 * _as_f64(q_pe), k_nope, k_pe, v, past_len, softmax_scale)"),
        ("np.asarray(q_pe)[b:b + 1, h:h + 1]", "0 * _as_f64(np.asarray(q_pe)[b:b + 1, h:h + 1])")],
    "latent of another sequence": [
        ("    c = _as_f64(c_kv)\n", "    c = _as_f64(c_kv)[::-1]\n"),
        ("c = _as_f64(c_kv[b])", "c = _as_f64(c_kv[(b + 1) % len(c_kv)])")],
    "weight rows of the next head": [
        ("wk = w[h * KV_B_PER_HEAD:h * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM]",
         "hh = (h + 1) % (w.shape[0] // KV_B_PER_HEAD)\n"
         "        wk = w[hh * KV_B_PER_HEAD:hh * KV_B_PER_HEAD + QK_NOPE_HEAD_DIM]")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
