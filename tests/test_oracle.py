"""The fp64 oracle against its pins (CPU only).

The pins themselves live in ``oracle_pins.py``; this file runs each of them on
the real oracle, and runs the whole set on every planted mistake of the
oracle's mutant build to show that each mistake fails at least one pin.
"""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="session", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(0)


@pytest.mark.parametrize("mutant", sorted(P.MUTANTS), ids=lambda m: P.MUTANTS[m])
def test_pins_catch_planted_mistake(mutant):
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {mutant} ({P.MUTANTS[mutant]})"
