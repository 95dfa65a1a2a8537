"""The 2D-mask pins catch plausible mistakes (CPU only).

As for the rotary oracle: each case plants one mistake in a copy of the
2D-mask oracle's source (loaded as a separate module; the oracle package is
untouched), puts the copy's functions in place of the real ones inside
tests/test_oracle_masked.py, and runs every pin there: at least one must fail.
The unchanged copy must pass them all.
"""

import inspect
import os
import types

import pytest

import test_oracle_masked as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = open(os.path.join(ROOT, "oracle", "mla_masked.py")).read().replace(
    "from .mla_oracle import", "from oracle.mla_oracle import")
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


def _load(source: str) -> types.ModuleType:
    mod = types.ModuleType("mla_masked_copy")
    exec(compile(source, "mla_masked_copy", "exec"), mod.__dict__)
    return mod


def _failures(mod) -> list:
    saved = {n: getattr(pins, n) for n in NAMES}
    failed = []
    try:
        for n in NAMES:
            setattr(pins, n, getattr(mod, n))
        for name in sorted(dir(pins)):
            fn = getattr(pins, name)
            if not name.startswith("test_") or not callable(fn):
                continue
            marks = getattr(fn, "pytestmark", [])
            cases = [()]
            for mk in marks:
                if mk.name == "parametrize":
                    cases = [c if isinstance(c, tuple) else (c,) for c in mk.args[1]]
            for args in cases:
                if len(inspect.signature(fn).parameters) != len(args):
                    continue
                try:
                    fn(*args)
                except pytest.skip.Exception:
                    pass
                except Exception:  # noqa: BLE001 - any failure of a pin counts
                    failed.append(name)
    finally:
        for n, v in saved.items():
            setattr(pins, n, v)
    return failed


def test_unchanged_copy_passes_every_pin():
    assert _failures(_load(SOURCE)) == []


@pytest.mark.parametrize("what", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(what):
    src = SOURCE
    for old, new in MUTANTS[what]:
        assert old in src, (what, old)
        src = src.replace(old, new)
    assert _failures(_load(src)), f"no pin caught: {what}"
