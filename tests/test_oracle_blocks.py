"""Pins of the block-size study's oracle pieces (CPU only; the WISE paper, App. B,
Table 8): block masses at B = 64 / 128 are the (32/B)-scaled sums of the 32-token
masses they cover and the 32-token masses the halved sums of the 16-token ones
(Eq. 5 is linear in A), and attention under a B-level support equals attention
under its expansion to the 32-token grid."""
import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(31)


@pytest.mark.parametrize("block", [64, 128])
def test_block_mass_aggregates(block):
    n, d = 512, 16
    q, k = RNG.standard_normal((n, d)) * 1.5, RNG.standard_normal((n, d)) * 1.5
    r32 = O.block_mass(q, k, block=32)
    rb = O.block_mass(q, k, block=block)
    f = block // 32
    nb = n // block
    agg = r32.reshape(nb, f, nb, f).sum(axis=(1, 3)) / f
    np.testing.assert_allclose(rb, agg, rtol=0, atol=1e-13)
    np.testing.assert_allclose(rb.sum(axis=1), 1.0, atol=1e-12)


def test_block16_masses_aggregate_to_block32():
    n, d = 256, 16
    q, k = RNG.standard_normal((n, d)) * 1.5, RNG.standard_normal((n, d)) * 1.5
    r16 = O.block_mass(q, k, block=16)
    r32 = O.block_mass(q, k, block=32)
    nb = n // 32
    np.testing.assert_allclose(r16.reshape(nb, 2, nb, 2).sum(axis=(1, 3)) / 2, r32, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r16.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(r16[np.triu_indices(n // 16, 1)] == 0.0)
    # a 16-token diagonal block averages over its 16 queries the causal prefix
    # of the block: query j of the block sees keys 0..j of it
    a = O.attention_probs(q, k)
    for qb in range(n // 16):
        blk = a[16 * qb:16 * qb + 16, 16 * qb:16 * qb + 16]
        assert abs(r16[qb, qb] - np.tril(blk).sum() / 16) < 1e-13


def test_block16_support_matches_masked_softmax():
    """Attention under a 16-token support is the softmax over exactly the keys of
    the scheduled 16-token blocks (brute force)."""
    n, d = 128, 8
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    nb = n // 16
    sup = [np.sort(RNG.choice(qb + 1, size=RNG.integers(1, qb + 2), replace=False)) for qb in range(nb)]
    o, lse = O.sparse_attention(q, k, v, sup, block=16)
    s = q @ k.T / np.sqrt(d)
    for i in range(n):
        keys = [j for j in range(i + 1) if (j // 16) in set(sup[i // 16].tolist())]
        if not keys:
            assert np.all(o[i] == 0) and np.isneginf(lse[i])
            continue
        w = np.exp(s[i, keys] - s[i, keys].max())
        np.testing.assert_allclose(o[i], (w / w.sum()) @ v[keys], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("block", [64, 128])
def test_sparse_attention_equals_its_expansion(block):
    n, d = 512, 16
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    nb = n // block
    sup = [np.sort(RNG.choice(qb + 1, size=RNG.integers(1, qb + 2), replace=False)) for qb in range(nb)]
    for qb in range(nb):                      # keep the diagonal block so no row is left empty
        sup[qb] = np.union1d(sup[qb], [qb])
    ob, lb = O.sparse_attention(q, k, v, sup, block=block)
    rows = O.expand_supports(sup, n // 32, block)
    o32, l32 = O.sparse_attention(q, k, v, rows, block=32)
    np.testing.assert_allclose(o32, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l32, lb, rtol=1e-12, atol=1e-12)


def test_expand_supports_causality_and_coverage():
    rows = O.expand_supports([np.array([0]), np.array([0, 1])], 4, 64)
    assert [r.tolist() for r in rows] == [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3]]
    rows = O.expand_supports([np.array([1])], 4, 128)      # an inadmissible block admits no key
    assert [r.tolist() for r in rows] == [[], [], [], []]
    rows = O.expand_supports([np.array([0])], 4, 128)
    assert [r.tolist() for r in rows] == [[0], [0, 1], [0, 1, 2], [0, 1, 2, 3]]
