"""The comparison rules between the HIP path and the oracle (tests/checker.py) against the cases that pin them."""
import pytest

from tests import checker
from tests.checker_cases import ALL_CASES


@pytest.mark.parametrize("case", ALL_CASES, ids=[c.__name__ for c in ALL_CASES])
def test_checker_case(case):
    case(checker)
