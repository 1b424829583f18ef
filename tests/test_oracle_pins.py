"""The oracle against the pages' printed examples, brute force, exhaustive
subsets, special cases, invariants, draw frequencies and an independent
Philox4x32-10 implementation (rocRAND's engine, built for the host)."""
import shutil

import pytest

import oracle_pins as P


def test_worked_examples(oracle_lib):
    P.check_worked_examples(oracle_lib.default())


def test_order_counterexample(oracle_lib):
    P.check_order_counterexample(oracle_lib.default())


def test_special_cases(oracle_lib):
    P.check_special_cases(oracle_lib.default())


def test_bruteforce_protocol(oracle_lib):
    rows, boundary = P.check_bruteforce_protocol(oracle_lib.default())
    # The page compared 8,970 sampled rows; about 3/4 of 12,000 rows are not greedy.
    assert rows > 8000
    assert boundary < 2000


def test_bruteforce_with_topk_minp(oracle_lib):
    rows, _ = P.check_bruteforce_protocol(oracle_lib.default(), batches=1500, seed=4321, extras=True)
    assert rows > 4000


def test_exhaustive_subsets(oracle_lib):
    P.check_exhaustive_subsets(oracle_lib.default())


def test_invariants(oracle_lib):
    P.check_invariants(oracle_lib.default())


def test_large_rows(oracle_lib):
    P.check_large_rows(oracle_lib.default())


def test_race_frequencies(oracle_lib):
    P.check_race_frequencies(oracle_lib.default())


def test_race_chisquare(oracle_lib):
    P.check_race_chisquare(oracle_lib.default())


def test_race_reproducible(oracle_lib):
    P.check_race_reproducible(oracle_lib.default())


def test_logprobs(oracle_lib):
    P.check_logprobs(oracle_lib)


def test_row_seeds(oracle_lib):
    P.check_row_seeds(oracle_lib)


def test_exp1(oracle_lib):
    P.check_exp1(oracle_lib.default())


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available to build rocRAND's engine")
def test_philox_matches_rocrand(oracle_lib, tmp_path_factory):
    tuples = P.philox_tuples()
    words = P.rocrand_words(tuples, str(tmp_path_factory.mktemp("rocrand")))
    P.check_philox_against(oracle_lib.default(), tuples, words)


def test_rejection_pages(oracle_lib):
    P.check_rejection_pages(oracle_lib.default())


def test_rejection_law(oracle_lib):
    P.check_rejection_law(oracle_lib.default())


def test_rejection_is_the_race(oracle_lib):
    P.check_rejection_is_the_race(oracle_lib.default())


def test_spec_law(oracle_lib):
    P.check_spec_law(oracle_lib.default())


def test_spec_special(oracle_lib):
    P.check_spec_special(oracle_lib.default())


def test_preprocess_values(oracle_lib):
    P.check_preprocess_values(oracle_lib.default())


def test_preprocess_identity_and_invariants(oracle_lib):
    P.check_preprocess_identity_and_invariants(oracle_lib.default())


def test_chain_order(oracle_lib):
    P.check_chain_order(oracle_lib.default())
