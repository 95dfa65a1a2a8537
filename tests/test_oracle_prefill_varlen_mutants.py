"""The padded variable-length prefill oracle's pins catch plausible mistakes
(CPU only): each case plants one mistake in a copy of
oracle/mla_prefill_varlen.py's source, swaps the copy into
tests/test_oracle_prefill_varlen.py and runs every pin there; at least one
must fail, and the unchanged copy must pass them all."""

import pytest

import test_oracle_prefill_varlen as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_prefill_varlen")
NAMES = ("mla_prefill_varlen",)

MUTANTS = {
    "each query sees one future key": [("        S = P + T\n", "        S = P + T + 1\n"),
                                       ("np.asarray(v)[b:b + 1, :, :S], P, softmax_scale)",
                                        "np.asarray(v)[b:b + 1, :, :S], P + 1, softmax_scale)")],
    "cached keys dropped": [
        ("np.asarray(k_nope)[b:b + 1, :, :S], np.asarray(k_pe)[b:b + 1, :, :S],",
         "np.asarray(k_nope)[b:b + 1, :, P:S], np.asarray(k_pe)[b:b + 1, :, P:S],"),
        ("np.asarray(v)[b:b + 1, :, :S], P, softmax_scale)", "np.asarray(v)[b:b + 1, :, P:S], 0, softmax_scale)")],
    "padded rows NaN instead of 0": [("out = np.zeros((B, H, Tmax, V_HEAD_DIM), dtype=np.float64)",
                                      "out = np.full((B, H, Tmax, V_HEAD_DIM), np.nan)")],
    "another sequence's rotary key": [("np.asarray(k_pe)[b:b + 1, :, :S]",
                                       "np.asarray(k_pe)[(b + 1) % B:(b + 1) % B + 1, :, :S]")],
    "query count and cached length swapped": [("T, P = int(tq[b]), int(pp[b])", "P, T = int(tq[b]), int(pp[b])")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
