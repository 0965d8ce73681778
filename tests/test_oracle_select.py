"""Pins of the oracle's cumulative-eta selection, temporal union and CSR
(the WISE paper §3 attention support, §5.1 block support, App. B temporal union
and sparse-kernel schedule) (CPU only).

Pinned by brute-force enumeration of every subset on small rows, invariants
(retained mass >= eta, minimality, eta = 1 keeps all, eta-monotonicity as a
property test), the zero-drift union, and hand-built examples.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

RNG = np.random.default_rng(7)


def _brute(masses, eta):
    """All subsets: minimum cardinality reaching eta, then maximum mass, then the
    lexicographically smallest index tuple."""
    nb = len(masses)
    best = None
    for size in range(1, nb + 1):
        cands = []
        for comb in itertools.combinations(range(nb), size):
            tot = sum(masses[i] for i in comb)
            if tot >= eta:
                cands.append((tot, comb))
        if cands:
            top = max(t for t, _ in cands)
            best = min(c for t, c in cands if t == top)
            break
    return np.array(best if best is not None else range(nb))


@pytest.mark.parametrize("nb", [1, 2, 3, 5, 8, 10])
@pytest.mark.parametrize("eta", [0.3, 0.5, 0.9, 0.95, 0.99])
def test_brute_force_random_masses(nb, eta):
    for _ in range(5):
        m = RNG.dirichlet(np.full(nb, 0.7))
        sel = O.select_support(m, eta)
        bf = _brute(list(m), eta)
        assert len(sel) == len(bf)
        # masses distinct with probability one: the sets must coincide
        np.testing.assert_array_equal(sel, np.sort(bf))


def test_brute_force_exact_ties_prefer_lower_index():
    # dyadic masses sum exactly in float64, so ties are exact
    cases = [
        ([0.25, 0.25, 0.5], 0.7),
        ([0.125] * 8, 0.5),
        ([0.0625, 0.25, 0.0625, 0.25, 0.125, 0.25], 0.6),
        ([0.5, 0.125, 0.125, 0.125, 0.125], 0.75),
        ([1 / 16] * 4 + [3 / 16] * 4, 0.8),
    ]
    for m, eta in cases:
        sel = O.select_support(np.array(m), eta)
        np.testing.assert_array_equal(sel, _brute(m, eta))


def test_invariants_on_real_attention_rows():
    n, d = 512, 32
    q = RNG.standard_normal((n, d)) * 2.5
    k = RNG.standard_normal((n, d)) * 2.5
    r = O.block_mass(q, k, 32)
    for eta in (0.5, 0.9, 0.95, 0.99):
        for qb, sup in enumerate(O.step_supports(r, eta)):
            row = r[qb, :qb + 1]
            assert O.retained_mass(row, sup) >= eta - 1e-12
            srt = np.sort(row)[::-1]
            assert srt[:len(sup) - 1].sum() < eta        # minimal: one block fewer misses eta
            assert np.all(sup <= qb) and np.all(np.diff(sup) > 0)
            # the kept blocks are the heaviest ones
            if len(sup) < qb + 1:
                out = np.setdiff1d(np.arange(qb + 1), sup)
                assert row[sup].min() >= row[out].max()


def test_eta_one_keeps_everything_and_q0_keeps_block0():
    m = RNG.dirichlet(np.ones(9))
    np.testing.assert_array_equal(O.select_support(m, 1.0), np.arange(9))
    np.testing.assert_array_equal(O.select_support(np.array([1.0]), 0.95), [0])


def test_unreachable_eta_keeps_everything():
    # rounded masses that sum below eta: no prefix reaches it, so every block is kept
    m = np.array([0.3, 0.3, 0.3])
    np.testing.assert_array_equal(O.select_support(m, 0.95), [0, 1, 2])


@settings(max_examples=200, deadline=None)
@given(st.lists(st.floats(0.001, 1.0), min_size=1, max_size=40),
       st.floats(0.01, 1.0), st.floats(0.01, 1.0))
def test_eta_monotone(raw, e1, e2):
    m = np.array(raw) / np.sum(raw)
    lo, hi = min(e1, e2), max(e1, e2)
    a, b = set(O.select_support(m, lo)), set(O.select_support(m, hi))
    assert a <= b


def test_union_properties_and_zero_drift():
    n, d = 256, 16
    base_q = RNG.standard_normal((n, d)) * 2
    base_k = RNG.standard_normal((n, d)) * 2
    steps = []
    masses = []
    for t in range(4):
        q = base_q + 0.3 * RNG.standard_normal((n, d))
        k = base_k + 0.3 * RNG.standard_normal((n, d))
        r = O.block_mass(q, k, 32)
        masses.append(r)
        steps.append(O.step_supports(r, 0.9))
    uni = O.union_supports(steps)
    for qb in range(n // 32):
        u = set(uni[qb].tolist())
        for t in range(4):
            assert set(steps[t][qb].tolist()) <= u
            assert O.retained_mass(masses[t][qb, :qb + 1], uni[qb]) >= 0.9 - 1e-12
        assert len(u) >= max(len(steps[t][qb]) for t in range(4))
        assert np.all(np.diff(uni[qb]) > 0)
    # zero drift: identical steps, union equals each step's set
    same = O.step_supports(O.block_mass(base_q, base_k, 32), 0.9)
    for qb, s in enumerate(O.union_supports([same] * 4)):
        np.testing.assert_array_equal(s, same[qb])


def test_build_csr_hand_example():
    rp, ci = O.build_csr([np.array([0]), np.array([0, 1]), np.array([], dtype=int), np.array([1, 2])])
    np.testing.assert_array_equal(rp, [0, 1, 3, 3, 5])
    np.testing.assert_array_equal(ci, [0, 0, 1, 1, 2])


def test_boundary_flags():
    # cumulative boundary: c after the two heaviest blocks is 0.95 + 5e-5, within 1e-4 of eta
    m = np.array([0.6, 0.35005, 0.04995])
    fc, ft = O.boundary_flags(m, 0.95)
    assert fc[2] and not fc[0]          # block 2's inclusion depends on c_1 vs eta
    assert not fc[1]
    # ranking near-tie across the cut
    m = np.array([0.5, 0.2500004, 0.2499996])
    fc, ft = O.boundary_flags(m, 0.7)
    sel = O.select_support(m, 0.7)
    np.testing.assert_array_equal(sel, [0, 1])
    assert ft[1] and ft[2] and not ft[0]
    # a clean row has no flags
    fc, ft = O.boundary_flags(np.array([0.7, 0.2, 0.1]), 0.85)
    assert not fc.any() and not ft.any()


def test_density_and_pairs():
    nq = 4
    rows = [np.arange(q + 1) for q in range(nq)]
    assert O.block_density(rows, nq) == 1.0
    assert O.scheduled_pairs(rows, nq) == 32 * 32 * 6 + 528 * 4
    half = [np.array([0]), np.array([1]), np.array([0, 2]), np.array([3])]
    assert O.block_density(half, nq) == 5 / 10
    assert O.scheduled_pairs(half, nq) == 528 * 4 + 1024
