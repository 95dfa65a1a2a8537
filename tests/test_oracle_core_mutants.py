"""The core oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/mla_oracle.py's source
(loaded as a separate module; the oracle package itself is untouched), puts
the copy's functions in place of the real ones inside
tests/test_oracle_pins.py, and runs every pin there: at least one must fail.
The unchanged copy must pass them all, so the harness itself is checked too.
"""

import pytest

import test_oracle_pins as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_oracle")
NAMES = ("attention_probs", "bf16_bits_to_f64", "causal_mask_4d", "mla_attention", "mla_attention_rows")

MUTANTS = {
    "rotary term dropped": [
        ("query = np.concatenate([qn[b, h], qp[b, h]], axis=-1)",
         "query = np.concatenate([qn[b, h], 0 * qp[b, h]], axis=-1)"),
        ("_as_f64(q_pe[b, h, qi])", "0 * _as_f64(q_pe[b, h, qi])")],
    "rotary key of another batch": [
        ("key = np.concatenate([kn[b, h], kp[b, 0]], axis=-1)",
         "key = np.concatenate([kn[b, h], kp[(b + 1) % kp.shape[0], 0]], axis=-1)"),
        ("_as_f64(k_pe[b, 0])", "_as_f64(k_pe[(b + 1) % k_pe.shape[0], 0])")],
    "mask lets each query see one future key": [
        ("m = np.where(j <= past_len + i, 0.0, -np.inf)", "m = np.where(j <= past_len + i + 1, 0.0, -np.inf)"),
        ("j <= past_len + np.asarray(qi)[:, None]", "j <= past_len + np.asarray(qi)[:, None] + 1")],
    "mask without the cached length": [
        ("m = np.where(j <= past_len + i, 0.0, -np.inf)", "m = np.where(j <= i, 0.0, -np.inf)"),
        ("j <= past_len + np.asarray(qi)[:, None]", "j <= np.asarray(qi)[:, None]")],
    "scale off by 1%": [("alpha = float(np.float32(softmax_scale))",
                         "alpha = float(np.float32(softmax_scale)) * 1.01")],
    "another head's values": [("out[b, h] = probs @ vv[b, h]", "out[b, h] = probs @ vv[b, (h + 1) % H]"),
                              ("vv = _as_f64(v[b, h])", "vv = _as_f64(v[b, (h + 1) % H])")],
    "softmax normalised over the queries": [("return e / np.sum(e, axis=-1, keepdims=True)",
                                             "return e / np.sum(e, axis=-2, keepdims=True)")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
