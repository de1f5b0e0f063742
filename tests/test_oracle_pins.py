"""The CPU oracle against its pins (formats, hand-worked fixtures, exact
rational arithmetic, full sorts, the dense softmax, closed forms and
invariants).  CPU only."""
import pytest

import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins as P  # noqa: E402


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
