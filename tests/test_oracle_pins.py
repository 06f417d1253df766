"""The CPU oracle against what the pages and the mathematics fix (see oracle_pins.py)."""
import pytest

from oracle import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("name", pins.GOLDEN_FILES)
def test_golden(orc, name):
    pins.check_golden(orc, name)


def test_bruteforce_all_small_count_matrices(orc):
    # N, E in {1,2,3}, entries in {0,1,2}: 21,297 matrices (all-zero ones included).
    assert pins.check_bruteforce(orc, 3, 3, (0, 1, 2)) == 21297


def test_identity_single_rank_or_expert(orc):
    pins.check_identity(orc)


def test_uniform_counts_block_transpose(orc):
    pins.check_block_transpose(orc)


def test_pages_examples(orc):
    pins.check_pages_examples(orc)


def test_random_invariants(orc):
    pins.check_random_invariants(orc)


def test_errors_write_nothing(orc):
    pins.check_errors(orc)


def test_empty_inputs(orc):
    pins.check_empty(orc)


@pytest.mark.parametrize("name", pins.GOLDEN_FILES)
def test_inverse_golden(orc, name):
    pins.check_inverse_golden(orc, name)


def test_inverse_bruteforce_all_small_count_matrices(orc):
    assert pins.check_inverse_bruteforce(orc, 3, 3, (0, 1, 2)) == 21297


def test_roundtrip(orc):
    pins.check_roundtrip(orc)


def test_inverse_errors_write_nothing(orc):
    pins.check_inverse_errors(orc)
