"""The rotary pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the rotary oracle's source (loaded
as a separate module; the oracle package itself is untouched), puts the copy's
functions in place of the real ones inside tests/test_oracle_rope.py, and runs
every pin there: at least one must fail. The unchanged copy must pass them all,
so the harness itself is checked too.
"""

import pytest

import test_oracle_rope as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_rope")
NAMES = ("apply_rope", "rope_cos_sin", "rope_positions", "yarn_inv_freq", "KIMI_K2_ROPE")

MUTANTS = {
    "pairs i and i+32 instead of neighbours": [
        ("ev, od = x[b, :, :, 0::2], x[b, :, :, 1::2]", "ev, od = x[b, :, :, :32], x[b, :, :, 32:]"),
        ("out[b, :, :, 0::2] = ev * c - od * s", "out[b, :, :, :32] = ev * c - od * s"),
        ("out[b, :, :, 1::2] = ev * s + od * c", "out[b, :, :, 32:] = ev * s + od * c")],
    "rotation by minus the angle": [
        ("ev * c - od * s", "ev * c + od * s"), ("ev * s + od * c", "-ev * s + od * c")],
    "slow pairs sped up instead": [("(1.0 - g) * w / float(factor)", "(1.0 - g) * w * float(factor)")],
    "the wrong pairs slowed": [("g[k] = 1.0\n        elif r[k] < lo:\n            g[k] = 0.0",
                                "g[k] = 0.0\n        elif r[k] < lo:\n            g[k] = 1.0")],
    "positions off by one": [("+ np.arange(T, dtype=np.int64)[None, :]",
                              "+ np.arange(1, T + 1, dtype=np.int64)[None, :]")],
    "table indexed by row, not position": [("c = cos[positions[b]]", "c = cos[np.arange(T)]"),
                                           ("s = sin[positions[b]]", "s = sin[np.arange(T)]")],
    "exponent over the pair index, not the dim": [("-2.0 * i / rotary_dim", "-1.0 * i / rotary_dim")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
