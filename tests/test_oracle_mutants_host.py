"""The mutation check of the oracle's pins still works (CPU): a planted slip
is caught and a change that computes the same thing is not. The full set of
planted slips runs by hand with ``python tests/oracle_mutants.py``."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle_mutants as om  # noqa: E402


def test_a_planted_slip_fails_a_pin():
    f, old, new = next(m for m in om.MUTANTS if "0x8000" in m[2])   # bf16 rounding half up
    status, info = om.run_one(f, old, new)
    assert status == "KILLED", info


def test_an_equivalent_change_passes_the_pins():
    f, old, new, _ = om.EQUIVALENT[0]
    status, info = om.run_one(f, old, new)
    assert status == "SURVIVED", info


def test_every_planted_slip_applies_once():
    for f, old, new in om.MUTANTS:
        src = open(os.path.join(om.ROOT, "oracle", f), encoding="utf-8").read()
        assert src.count(old) == 1, (f, old)
