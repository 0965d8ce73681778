"""Pins of the intervention-control supports and of the retained mass (CPU only).

SizeMatched and MassMatched (the WISE paper, App. B, intervention controls) are
checked against brute-force enumeration of every subset on small rows, and
against the invariants that fix them: SizeMatched keeps exactly K_q blocks with
at least the reference mass; MassMatched keeps no more blocks than the
reference and at least its mass; a reference that is itself a sorted prefix is
reproduced exactly.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from oracle.wise_oracle import MASS_MATCH_SLACK

RNG = np.random.default_rng(77)


def _best_subset(m, size=None, threshold=None):
    """Brute force: among subsets of the given size (or, for a threshold, of the
    smallest size reaching it) the one of largest mass, ties to the
    lexicographically lowest sorted index tuple."""
    n = len(m)
    sizes = [size] if size is not None else range(1, n + 1)
    for k in sizes:
        cands = [(sum(m[i] for i in c), c) for c in itertools.combinations(range(n), k)]
        if threshold is not None:
            cands = [x for x in cands if x[0] >= threshold]
        if cands:
            top = max(t for t, _ in cands)
            return np.array(min(c for t, c in cands if t == top))
    return np.arange(n)


@pytest.mark.parametrize("n", [1, 3, 6, 9])
def test_size_matched_is_the_heaviest_subset_of_that_size(n):
    for _ in range(12):
        m = RNG.dirichlet(np.full(n, 0.6))
        for k in range(1, n + 1):
            assert np.array_equal(O.size_matched_support(m, k), _best_subset(m, size=k)), (m, k)


def test_size_matched_ties_and_bounds():
    m = np.array([0.25, 0.25, 0.25, 0.25])
    assert O.size_matched_support(m, 2).tolist() == [0, 1]
    assert O.size_matched_support(m, 0).tolist() == []
    assert O.size_matched_support(m, 9).tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("n", [2, 5, 8])
def test_mass_matched_is_the_smallest_heaviest_subset_reaching_the_reference_mass(n):
    for _ in range(12):
        m = RNG.dirichlet(np.full(n, 0.6))
        ref = RNG.choice(n, size=RNG.integers(1, n + 1), replace=False)
        mref = float(sum(m[b] for b in ref))
        got = O.mass_matched_support(m, ref)
        assert np.array_equal(got, _best_subset(m, threshold=mref - MASS_MATCH_SLACK)), (m, ref)
        assert len(got) <= len(ref)
        assert m[got].sum() >= mref - MASS_MATCH_SLACK


def test_mass_matched_reproduces_a_prefix_reference():
    for n in (4, 16, 64):
        m = RNG.dirichlet(np.full(n, 0.3))
        for k in (1, n // 2, n):
            ref = O.sorted_order(m)[:k]
            assert np.array_equal(O.mass_matched_support(m, ref), np.sort(ref))


def test_mass_matched_empty_reference_keeps_one_block():
    m = np.array([0.1, 0.7, 0.2])
    assert O.mass_matched_support(m, []).tolist() == [1]


def test_size_matched_keeps_at_least_the_reference_mass():
    for _ in range(50):
        n = int(RNG.integers(2, 40))
        m = RNG.dirichlet(np.full(n, 0.5))
        ref = RNG.choice(n, size=RNG.integers(1, n + 1), replace=False)
        got = O.size_matched_support(m, len(ref))
        assert len(got) == len(ref) and m[got].sum() >= m[ref].sum() - 1e-15


def test_static95_is_the_single_step_support():
    m = RNG.dirichlet(np.full(12, 0.4))
    assert np.array_equal(O.select_support(m, 0.95), O.union_supports([[O.select_support(m, 0.95)]])[0])


def test_retained_mass_definition():
    m = np.array([0.5, 0.3, 0.2])
    assert O.retained_mass(m, [0, 2]) == pytest.approx(0.7, abs=1e-15)
    assert O.retained_mass(m, []) == 0.0
    # the cumulative-eta support keeps at least eta
    for _ in range(30):
        m = RNG.dirichlet(np.full(20, 0.5))
        assert O.retained_mass(m, O.select_support(m, 0.9)) >= 0.9 - 1e-12


def _size_matched_ascending(m, k):          # mutant: lightest blocks first
    return np.sort(np.argsort(m, kind="stable")[:k])


def _mass_matched_strict(m, ref):           # mutant: ">" instead of ">="
    order = O.sorted_order(m)
    mref = sum(m[b] for b in order if b in set(ref))
    c = np.cumsum(np.asarray(m, dtype=np.float64)[order])
    hit = np.nonzero(c > mref + 1e-12)[0]
    return np.sort(order[:(hit[0] + 1) if hit.size else len(m)])


def test_variant_mutants_are_caught():
    m = np.array([0.1, 0.4, 0.3, 0.2])
    assert not np.array_equal(_size_matched_ascending(m, 2), _best_subset(m, size=2))
    ref = O.sorted_order(m)[:2]
    assert not np.array_equal(_mass_matched_strict(m, ref), np.sort(ref))
