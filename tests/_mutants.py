"""Helpers for the planted-mistake tests: load a changed copy of an oracle
module's source as a separate module (the oracle package is untouched) and
run a pin module's tests with the copy's functions swapped in."""

import inspect
import os
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def oracle_source(name: str) -> str:
    """Source of oracle/<name>.py with its package-relative imports made absolute."""
    src = open(os.path.join(ROOT, "oracle", name + ".py")).read()
    return src.replace("from .", "from oracle.")


def load_copy(source: str, name: str = "oracle_copy") -> types.ModuleType:
    mod = types.ModuleType(name)
    exec(compile(source, name, "exec"), mod.__dict__)
    return mod


def plant(source: str, edits) -> str:
    for old, new in edits:
        assert old in source, old
        source = source.replace(old, new)
    return source


def pin_failures(pins, names, mod) -> list:
    """Names of the pins (test functions of module `pins`, each parametrized
    case included) that fail with `names` taken from `mod`."""
    saved = {n: getattr(pins, n) for n in names}
    failed = []
    try:
        for n in names:
            setattr(pins, n, getattr(mod, n))
        for name in sorted(dir(pins)):
            fn = getattr(pins, name)
            if not name.startswith("test_") or not callable(fn):
                continue
            cases = [()]
            for mk in getattr(fn, "pytestmark", []):
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
