"""Pins of the oracle's full and sparse causal attention (CPU only).

Pinned against things other than the oracle itself: torch's scaled-dot-product
attention in float64 (a library routine), closed forms (uniform attention),
invariants (constant values, a dominant key, rows summing to one) and the
pages' own validation method, "explicit exact masked attention"
(the WISE paper, App. B, sparse-kernel implementation).
"""
import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(1234)


def _qkv(n, d, scale=1.0):
    return (RNG.standard_normal((n, d)) * scale, RNG.standard_normal((n, d)) * scale,
            RNG.standard_normal((n, d)))


def _sdpa(q, k, v, mask=None, causal=False):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None, None],
        is_causal=causal)
    return out[0, 0].numpy()


@pytest.mark.parametrize("n,d", [(1, 8), (7, 16), (64, 64), (96, 128), (700, 32)])
def test_full_matches_torch_sdpa_fp64(n, d):
    q, k, v = _qkv(n, d, 2.0)
    o, _ = O.causal_attention(q, k, v)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=1e-11, atol=1e-12)


def test_lse_matches_torch_logsumexp():
    n, d = 130, 32
    q, k, _ = _qkv(n, d, 3.0)
    _, lse = O.causal_attention(q, k, np.zeros((n, d)))
    logits = torch.from_numpy(q @ k.T / np.sqrt(d))
    logits = logits.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -float("inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).numpy(), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_prefix_mean_closed_form():
    # Q = 0 makes every admissible logit equal: A_ij = 1/(i+1) for j <= i, so
    # O_i is the running mean of v_0..v_i and lse_i = log(i+1).
    n, d = 200, 16
    v = RNG.standard_normal((n, d))
    o, lse = O.causal_attention(np.zeros((n, d)), RNG.standard_normal((n, d)), v)
    expect = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-13)


def test_constant_values_give_constant_output():
    n, d = 150, 24
    q, k, _ = _qkv(n, d, 2.0)
    c = RNG.standard_normal(d)
    o, _ = O.causal_attention(q, k, np.tile(c, (n, 1)))
    np.testing.assert_allclose(o, np.tile(c, (n, 1)), rtol=1e-12, atol=1e-12)


def test_dominant_key_is_selected():
    # One key aligned with every query with a huge logit wins all rows at or after it.
    n, d, target = 64, 32, 10
    q, k, v = _qkv(n, d, 0.1)
    u = RNG.standard_normal(d)
    u /= np.linalg.norm(u)
    q = q + 60.0 * u
    k[target] = 60.0 * u
    o, _ = O.causal_attention(q, k, v)
    np.testing.assert_allclose(o[target:], np.tile(v[target], (n - target, 1)), atol=1e-9)


def test_probabilities_are_causal_and_normalised():
    n, d = 100, 8
    q, k, _ = _qkv(n, d, 2.0)
    a = O.attention_probs(q, k)
    assert np.all(a[np.triu_indices(n, 1)] == 0.0)
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    # rows computed in two chunks agree with the whole
    np.testing.assert_array_equal(O.attention_probs(q, k, rows=(40, 70)), a[40:70])


def test_custom_scale_matches_sdpa():
    n, d = 50, 16
    q, k, v = _qkv(n, d)
    o, _ = O.causal_attention(q, k, v, scale=0.37)
    t = lambda x: torch.from_numpy(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.37)
    np.testing.assert_allclose(o, ref[0, 0].numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- sparse (§5.2)

def _explicit_mask(n, block, supports):
    keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for b in supports[i // block]:
            for j in range(b * block, min((b + 1) * block, i + 1)):
                keep[i, j] = True
    return keep


@pytest.mark.parametrize("n,block,d", [(64, 32, 16), (256, 32, 64), (96, 16, 8)])
def test_sparse_matches_sdpa_with_explicit_boolean_mask(n, block, d):
    q, k, v = _qkv(n, d, 1.5)
    nq = n // block
    supports = []
    for qb in range(nq):
        pick = RNG.random(qb + 1) < 0.5
        pick[RNG.integers(0, qb + 1)] = True          # never empty
        supports.append(np.nonzero(pick)[0])
    o, _ = O.sparse_attention(q, k, v, supports, block=block)
    ref = _sdpa(q, k, v, mask=_explicit_mask(n, block, supports))
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-12)


def test_sparse_with_every_block_equals_full():
    n, d, block = 224, 32, 32
    q, k, v = _qkv(n, d, 2.0)
    full_o, full_lse = O.causal_attention(q, k, v)
    sup = [np.arange(qb + 1) for qb in range(n // block)]
    o, lse = O.sparse_attention(q, k, v, sup, block=block)
    np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, full_lse, rtol=1e-12, atol=1e-12)
    # eta = 1 supports are every admissible block
    r = O.block_mass(q, k, block)
    assert all(np.array_equal(s, np.arange(qb + 1)) for qb, s in enumerate(O.step_supports(r, 1.0)))


def test_sparse_renormalises_instead_of_truncating():
    # Keeping only block 0 for query block 1: the rows equal attention over keys 0..31 alone.
    n, d, block = 64, 8, 32
    q, k, v = _qkv(n, d, 2.0)
    o, lse = O.sparse_attention(q, k, v, [np.array([0]), np.array([0])], block=block)
    for i in range(32, 64):
        s = q[i] @ k[:32].T / np.sqrt(d)
        p = np.exp(s - s.max())
        np.testing.assert_allclose(o[i], p @ v[:32] / p.sum(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[i], s.max() + np.log(p.sum()), rtol=1e-13)
    # rows 0..31 (block 0, diagonal) are unchanged full attention
    full_o, _ = O.causal_attention(q[:32], k[:32], v[:32])
    np.testing.assert_allclose(o[:32], full_o, rtol=1e-12, atol=1e-13)


def test_sparse_constant_values_and_ignored_entries():
    n, d, block = 128, 16, 32
    q, k, _ = _qkv(n, d, 2.0)
    c = RNG.standard_normal(d)
    sup = [np.array([0]), np.array([1, 3]), np.array([0, 2, 7, -1]), np.array([3])]
    o, _ = O.sparse_attention(q, k, np.tile(c, (n, 1)), sup, block=block)
    np.testing.assert_allclose(o, np.tile(c, (n, 1)), rtol=1e-12, atol=1e-12)
    # b > q and out-of-range entries carry no admissible key: same as dropping them
    o1, _ = O.sparse_attention(q, k, RNG.standard_normal((n, d)), sup, block=block)
    clean = [np.array([0]), np.array([1]), np.array([0, 2]), np.array([3])]
    v2 = RNG.standard_normal((n, d))
    a, _ = O.sparse_attention(q, k, v2, sup, block=block)
    b, _ = O.sparse_attention(q, k, v2, clean, block=block)
    np.testing.assert_array_equal(a, b)


def test_sparse_empty_support_convention():
    n, d = 64, 8
    q, k, v = _qkv(n, d)
    o, lse = O.sparse_attention(q, k, v, [np.array([], dtype=int), np.array([1])], block=32)
    assert np.all(o[:32] == 0.0) and np.all(np.isneginf(lse[:32]))
    assert np.all(np.isfinite(o[32:]))


def test_row_subsets_equal_slices_of_the_whole():
    n, d, block = 320, 16, 32
    q, k, v = _qkv(n, d, 2.0)
    o, lse = O.causal_attention(q, k, v)
    o2, lse2 = O.causal_attention(q, k, v, rows=(64, 200))
    # equal up to BLAS blocking order
    np.testing.assert_allclose(o2, o[64:200], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse[64:200], rtol=1e-13, atol=1e-14)
    sup = [np.nonzero(RNG.random(qb + 1) < 0.6)[0] for qb in range(n // block)]
    sup = [s if s.size else np.array([qb]) for qb, s in enumerate(sup)]
    so, sl = O.sparse_attention(q, k, v, sup, block=block)
    so2, sl2 = O.sparse_attention(q, k, v, sup, block=block, qblocks=(3, 7))
    np.testing.assert_allclose(so2, so[96:224], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sl2, sl[96:224], rtol=1e-13, atol=1e-14)
