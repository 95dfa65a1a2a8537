"""The 2D-mask pins catch plausible mistakes (CPU only).

As for the rotary oracle: each case plants one mistake in a copy of the
2D-mask oracle's source (loaded as a separate module; the oracle package is
untouched), puts the copy's functions in place of the real ones inside
tests/test_oracle_masked.py, and runs every pin there: at least one must fail.
The unchanged copy must pass them all.
"""

import pytest

import test_oracle_masked as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_masked")
NAMES = ("mla_attention_masked", "visible_keys")

MUTANTS = {
    "OR instead of AND of the two masks": [("causal[None, :, :] & m[:, None, :]",
                                            "causal[None, :, :] | m[:, None, :]")],
    "2D mask shifted by the cached length": [("return causal[None, :, :] & m[:, None, :]",
                                              "return causal[None, :, :] & np.roll(m, past_len, axis=1)[:, None, :]")],
    "causal bound off by one": [("causal = j <= past_len + i", "causal = j < past_len + i")],
    "empty rows give NaN, not 0": [("                if cols.size == 0:\n                    continue",
                                    "                if cols.size == 0:\n                    out[b, h, i] = np.nan\n"
                                    "                    continue")],
    "hidden value rows still reach the sum": [("out[b, h, i] = p @ vv[b, h, cols]",
                                               "out[b, h, i] = p @ vv[b, h, cols] + 0.0 * vv[b, h].sum(axis=0)")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
