"""The CPU oracle against its pins (library routines, closed forms, invariants,
hand-derived fixtures). CPU only."""

import pytest

import oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)


def test_prefill_non_causal_vs_sdpa():
    P.pin_prefill_vs_sdpa(O, seed=21, causal=False)
