"""The oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os

import pytest

import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_shuffle_golden_offsets(orc):
    with open(os.path.join(GOLDEN, "shuffle_offsets.json")) as f:
        P.pin_shuffle_golden(orc, json.load(f))
