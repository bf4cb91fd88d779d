"""The oracle against its pins (CPU only): see oracle_checks.py for what each
check compares against."""
import pytest

import oracle
import oracle_checks
import oracle_checks_f32


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)


@pytest.mark.parametrize("check", oracle_checks_f32.F32_CHECKS, ids=lambda c: c.__name__)
def test_pin_f32(orc, check):
    check(orc)
