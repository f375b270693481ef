"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_more_seeds(seed):
    pins.check_brute_force(seed=seed, n_cases=12)
