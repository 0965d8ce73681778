"""Pins of the oracle's block mass, the WISE paper §5.1 (Eq. 5) (CPU only).

Pinned by: the closed form of uniform attention computed with exact rational
arithmetic, a brute-force double sum over an explicitly materialised attention
matrix written as loops, and normalisation / causality invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(99)


def _uniform_closed_form(n, block):
    """r_qb for A_ij = 1/(i+1) (j <= i): (1/B) sum_{i in I_q} |{j in I_b : j <= i}| / (i+1)."""
    nq = n // block
    r = np.zeros((nq, nq))
    for qb in range(nq):
        for b in range(qb + 1):
            acc = Fraction(0)
            for i in range(qb * block, (qb + 1) * block):
                cnt = max(0, min((b + 1) * block - 1, i) - b * block + 1)
                acc += Fraction(cnt, i + 1)
            r[qb, b] = float(acc / block)
    return r


@pytest.mark.parametrize("n,block", [(128, 32), (96, 16), (256, 32)])
def test_uniform_attention_closed_form(n, block):
    d = 8
    r = O.block_mass(np.zeros((n, d)), RNG.standard_normal((n, d)), block=block)
    np.testing.assert_allclose(r, _uniform_closed_form(n, block), rtol=0, atol=1e-14)


def test_uniform_closed_form_spot_values():
    # n = 64, B = 32: query block 1 holds rows 32..63.  Block 0 contributes 32/(i+1)
    # per row; block 1 contributes (i-31)/(i+1).
    r = O.block_mass(np.zeros((64, 4)), RNG.standard_normal((64, 4)), block=32)
    r10 = sum(32.0 / (i + 1) for i in range(32, 64)) / 32
    r11 = sum((i - 31.0) / (i + 1) for i in range(32, 64)) / 32
    assert r[0, 0] == 1.0 and r[0, 1] == 0.0
    assert abs(r[1, 0] - r10) < 1e-15 and abs(r[1, 1] - r11) < 1e-15


def test_brute_force_double_sum():
    n, d, block = 96, 16, 32
    q = RNG.standard_normal((n, d)) * 2
    k = RNG.standard_normal((n, d)) * 2
    # materialise A with explicit loops
    a = np.zeros((n, n))
    for i in range(n):
        logits = [float(q[i] @ k[j]) / np.sqrt(d) for j in range(i + 1)]
        m = max(logits)
        w = [np.exp(x - m) for x in logits]
        tot = sum(w)
        for j in range(i + 1):
            a[i, j] = w[j] / tot
    nq = n // block
    expect = np.zeros((nq, nq))
    for qb in range(nq):
        for b in range(nq):
            s = 0.0
            for i in range(qb * block, (qb + 1) * block):
                for j in range(b * block, (b + 1) * block):
                    s += a[i, j]
            expect[qb, b] = s / block
    np.testing.assert_allclose(O.block_mass(q, k, block), expect, rtol=1e-12, atol=1e-15)


def test_rows_sum_to_one_and_causal_zero():
    n, d = 1024, 64
    q = RNG.standard_normal((n, d)) * 3
    k = RNG.standard_normal((n, d)) * 3
    r = O.block_mass(q, k, 32)
    np.testing.assert_allclose(r.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(r[np.triu_indices(r.shape[0], 1)] == 0.0)
    assert np.all(r >= 0.0)


def test_sum_of_block_mass_matches_attention_columns():
    # Summing r over query blocks equals the column sums of A grouped by blocks / B.
    n, d, block = 160, 8, 32
    q, k = RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    a = O.attention_probs(q, k)
    r = O.block_mass(q, k, block)
    col = a.reshape(n // block, block, n // block, block).sum(axis=(1, 3)) / block
    np.testing.assert_allclose(r, col, rtol=1e-12, atol=1e-15)


def test_rejects_ragged_length():
    with pytest.raises(ValueError):
        O.block_mass(np.zeros((33, 4)), np.zeros((33, 4)), 32)


def test_query_block_subset_equals_slice():
    n, d = 640, 16
    q, k = RNG.standard_normal((n, d)) * 2, RNG.standard_normal((n, d)) * 2
    r = O.block_mass(q, k, 32)
    np.testing.assert_allclose(O.block_mass(q, k, 32, qblocks=(5, 19)), r[5:19], rtol=1e-13, atol=1e-15)
