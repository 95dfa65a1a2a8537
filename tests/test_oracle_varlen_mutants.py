"""The variable-length decode pins catch plausible mistakes (CPU only): each
case plants one mistake in a copy of the oracle's source, swaps the copy into
tests/test_oracle_varlen.py and runs every pin there; at least one must fail,
and the unchanged copy must pass them all."""

import pytest

import test_oracle_varlen as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_varlen")
NAMES = ("mla_decode_varlen", "mla_decode_varlen_rows")

MUTANTS = {
    "one row too many": [(":L]", ":L + 1]"), ("L - 1, softmax_scale", "L, softmax_scale")],
    "one row too few": [(":L]", ":L - 1]"), ("L - 1, softmax_scale", "L - 2, softmax_scale")],
    "another batch's rotary key": [("np.asarray(k_pe_cache)[b:b + 1, :, :L]",
                                    "np.asarray(k_pe_cache)[(b + 1) % B:(b + 1) % B + 1, :, :L]")],
    "NaN instead of 0 for an empty sequence": [
        ("        if L == 0:\n            continue\n", "        if L == 0:\n            out[b] = np.nan\n            continue\n"),
        ("            continue  # no valid key", "            out[n] = np.nan\n            continue  # no valid key")],
    "rotary term dropped": [("np.asarray(q_pe)[b:b + 1]", "0 * np.asarray(q_pe)[b:b + 1]")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
