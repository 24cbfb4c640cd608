"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

from tests import oracle_checks as OC


@pytest.mark.parametrize("check", OC.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
