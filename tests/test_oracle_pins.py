"""The oracle against the pages' worked examples, library routines, closed forms and invariants."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL, ids=[c.__name__ for c in pins.ALL])
def test_pin(check):
    check()
