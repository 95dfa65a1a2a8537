"""The paged decode pins catch plausible mistakes (CPU only): each case plants
one mistake in a copy of the oracle's source, swaps the copy into
tests/test_oracle_paged.py and runs every pin there; at least one must fail,
and the unchanged copy must pass them all."""

import pytest

import test_oracle_paged as pins
from _mutants import load_copy, oracle_source, pin_failures, plant

SOURCE = oracle_source("mla_paged")
NAMES = ("mla_decode_paged",)

MUTANTS = {
    "logical block index used as the physical one": [("blk = int(block_table[b, j // block_size])",
                                                      "blk = int(j // block_size)")],
    "row within the block off by one": [("        r = j % block_size\n",
                                         "        r = (j + 1) % block_size\n")],
    "new token written one slot late": [("blk = int(block_table[b, (L - 1) // block_size])\n        r = (L - 1) % block_size",
                                         "blk = int(block_table[b, L // block_size])\n        r = L % block_size")],
    "new key's rotary row not written": [("        kp[blk, r] = np.asarray(k_pe_new)[b, 0, 0]\n", "")],
    "another sequence's table row": [("blk = int(block_table[b, j // block_size])",
                                      "blk = int(block_table[(b + 1) % block_table.shape[0], j // block_size])")],
}


def test_unchanged_copy_passes_every_pin():
    assert pin_failures(pins, NAMES, load_copy(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    assert pin_failures(pins, NAMES, load_copy(plant(SOURCE, MUTANTS[what]))), f"no pin caught: {what}"
