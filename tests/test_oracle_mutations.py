"""The oracle's pins catch plausible mistakes (CPU only).

Each test plants one mistake in a copy of an oracle function -- a dropped term,
a wrong sign or index, a transposed operand, an off-by-one mask, a flipped
comparison or tie rule -- and checks that the pin it should trip rejects the
mutant while the real oracle passes the same pin.
"""
import itertools

import numpy as np
import torch

import oracle as O

RNG = np.random.default_rng(2024)


# ----------------------------------------------------------------- pins as checks

def pin_attention(fn):
    """torch SDPA (float64, causal) on random inputs of a few shapes."""
    for n, d in ((37, 16), (96, 64)):
        q, k, v = (RNG.standard_normal((n, d)) * 2 for _ in range(3))
        t = lambda x: torch.from_numpy(x)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)[0, 0].numpy()
        if not np.allclose(fn(q, k, v)[0], ref, rtol=1e-10, atol=1e-12):
            return False
    return True


def pin_mass(fn):
    """Uniform-attention closed form and rows summing to one."""
    n, block = 128, 32
    r = fn(np.zeros((n, 8)), RNG.standard_normal((n, 8)), block)
    for qb in range(n // block):
        for b in range(qb + 1):
            exp = sum(max(0, min((b + 1) * block - 1, i) - b * block + 1) / (i + 1)
                      for i in range(qb * block, (qb + 1) * block)) / block
            if abs(r[qb, b] - exp) > 1e-13:
                return False
    q = RNG.standard_normal((160, 8)) * 2
    k = RNG.standard_normal((160, 8)) * 2
    return np.allclose(fn(q, k, 32).sum(axis=1), 1.0, atol=1e-12)


def pin_select(fn):
    """Brute-force enumeration, including exact dyadic ties."""
    cases = [(RNG.dirichlet(np.full(nb, 0.7)), eta) for nb in (3, 6, 9) for eta in (0.5, 0.9, 0.95)]
    cases += [(np.array([0.25, 0.25, 0.5]), 0.7), (np.array([0.125] * 8), 0.5), (np.array([0.5, 0.25, 0.25]), 0.75)]
    for m, eta in cases:
        best = None
        for size in range(1, len(m) + 1):
            cands = [(sum(m[i] for i in c), c) for c in itertools.combinations(range(len(m)), size)
                     if sum(m[i] for i in c) >= eta]
            if cands:
                top = max(t for t, _ in cands)
                best = min(c for t, c in cands if t == top)
                break
        if not np.array_equal(np.sort(fn(m, eta)), np.array(best)):
            return False
    return True


def pin_sparse(fn):
    """SDPA with an explicit boolean mask (explicit exact masked attention)."""
    n, d, block = 96, 16, 32
    q, k, v = (RNG.standard_normal((n, d)) * 1.5 for _ in range(3))
    sup = [np.array([0]), np.array([1]), np.array([0, 2])]
    keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for b in sup[i // block]:
            keep[i, b * block:min((b + 1) * block, i + 1)] = True
    t = lambda x: torch.from_numpy(x)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=t(keep))[0, 0].numpy()
    return np.allclose(fn(q, k, v, sup, block)[0], ref, rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- mutants

def _softmax_rows(logits):
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return p / p.sum(axis=1, keepdims=True)


def att_mask_off_by_one(q, k, v):          # j < i instead of j <= i (row 0 made valid)
    n, d = q.shape
    lg = q @ k.T / np.sqrt(d)
    lg[np.arange(n)[None, :] >= np.arange(n)[:, None]] = -np.inf
    lg[0, 0] = 0.0
    return _softmax_rows(lg) @ v, None


def att_no_scale(q, k, v):                 # dropped 1/sqrt(d)
    n, d = q.shape
    lg = q @ k.T
    lg[np.triu_indices(n, 1)] = -np.inf
    return _softmax_rows(lg) @ v, None


def att_transposed(q, k, v):               # K Q^T instead of Q K^T
    n, d = q.shape
    lg = k @ q.T / np.sqrt(d)
    lg[np.triu_indices(n, 1)] = -np.inf
    return _softmax_rows(lg) @ v, None


def mass_divide_by_n(q, k, block):         # mean over all keys' rows instead of |I_q|
    return O.block_mass(q, k, block) * block / q.shape[0]


def mass_transposed(q, k, block):          # r_bq instead of r_qb
    return O.block_mass(q, k, block).T


def mass_strict_causal(q, k, block):       # diagonal block loses the j == i key
    n = q.shape[0]
    a = O.attention_probs(q, k)
    a[np.arange(n), np.arange(n)] = 0.0
    nq = n // block
    return a.reshape(nq, block, nq, block).sum(axis=(1, 3)) / block


def sel_strict(m, eta):                    # "> eta" instead of ">= eta"
    order = O.sorted_order(m)
    c = np.cumsum(m[order])
    hit = np.nonzero(c > eta)[0]
    return np.sort(order[:(hit[0] + 1) if hit.size else len(m)])


def sel_high_index_ties(m, eta):           # ties to the higher index
    order = np.lexsort((-np.arange(len(m)), -m))
    c = np.cumsum(m[order])
    hit = np.nonzero(c >= eta)[0]
    return np.sort(order[:(hit[0] + 1) if hit.size else len(m)])


def sel_ascending(m, eta):                 # sorted ascending (lightest first)
    order = np.argsort(m, kind="stable")
    c = np.cumsum(m[order])
    hit = np.nonzero(c >= eta)[0]
    return np.sort(order[:(hit[0] + 1) if hit.size else len(m)])


def sel_one_short(m, eta):                 # k* - 1 blocks
    s = O.select_support(m, eta)
    order = O.sorted_order(m)
    return np.sort(order[:max(1, len(s) - 1)])


def sparse_truncated(q, k, v, supports, block):   # truncates the full softmax instead of renormalising
    n, d = q.shape
    a = O.attention_probs(q, k)
    keep = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for b in supports[i // block]:
            keep[i, b * block:min((b + 1) * block, i + 1)] = True
    return (a * keep) @ v, None


def sparse_ignores_support(q, k, v, supports, block):
    return O.causal_attention(q, k, v)


# ----------------------------------------------------------------- tests

def test_real_oracle_passes_every_pin():
    assert pin_attention(O.causal_attention)
    assert pin_mass(O.block_mass)
    assert pin_select(O.select_support)
    assert pin_sparse(lambda q, k, v, s, b: O.sparse_attention(q, k, v, s, block=b))


def test_attention_mutants_are_caught():
    for bad in (att_mask_off_by_one, att_no_scale, att_transposed):
        assert not pin_attention(bad), bad.__name__


def test_mass_mutants_are_caught():
    for bad in (mass_divide_by_n, mass_transposed, mass_strict_causal):
        assert not pin_mass(bad), bad.__name__


def test_selection_mutants_are_caught():
    for bad in (sel_strict, sel_high_index_ties, sel_ascending, sel_one_short):
        assert not pin_select(bad), bad.__name__


def test_sparse_mutants_are_caught():
    for bad in (sparse_truncated, sparse_ignores_support):
        assert not pin_sparse(bad), bad.__name__
