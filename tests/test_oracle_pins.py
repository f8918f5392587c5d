"""The CPU oracle against its pins (closed forms, library conversions, exact
sums, invariants, and the independent Fraction formulation)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def test_default_build_is_not_a_mutant(o):
    assert o.mutant == 0


def test_golden_closed_forms(o):
    pins.pin_golden(o)


def test_every_code_pair(o):
    pins.pin_code_pairs(o)


def test_unbounded_bits_give_exact_sum(o):
    pins.pin_unbounded_bits_exact(o)


def test_no_truncation_bruteforce(o):
    pins.pin_no_truncation_bruteforce(o)


def test_zero_rules(o):
    pins.pin_zero_rules(o)


def test_sign_symmetry(o):
    pins.pin_sign_symmetry(o)


def test_power_of_two_scaling(o):
    pins.pin_power_of_two_scaling(o)


def test_block_permutation(o):
    pins.pin_block_permutation(o)


def test_split_invariants(o):
    pins.pin_split_invariants(o)


def test_epilogue_random(o):
    pins.pin_epilogue_random(o)


def test_spec_cross_check(o):
    pins.pin_spec_cross_check(o)


def test_accumulator_only_path(o):
    pins.pin_c_only(o)


def test_incoming_accumulator_composes_chains(o):
    pins.pin_c_composition(o)


def test_infinities_follow_ieee(o):
    pins.pin_infinities_ieee(o)


def test_nonfinite_incoming_accumulators_follow_ieee(o):
    pins.pin_c_nonfinite_ieee(o)


def test_spec_cross_check_per_profile_and_mode(o):
    pins.pin_spec_cross_check_profiles(o)
