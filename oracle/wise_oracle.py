"""Plain, slow, fp64 CPU oracle for the WISE working-set attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library; it reads the same seeded input arrays and
nothing else.

Source of every definition: Wan & Chen, "Attention Routing Stabilizes Early:
Working-Set Inference for Recurrent-Depth Language Models" (arXiv 2609.27373),
cited below as "the WISE paper" with the section or equation a step follows.

Every function works on ONE attention head with plain numpy in float64; the
inputs are the exact values the GPU reads (bf16 or fp32), upcast to float64.

Readings taken where the paper is silent:
  * recurrent steps are numbered from 1; the union covers steps 9..12;
  * block mass averages over all B rows of a query block, so the masses of one
    query block sum to 1 (the diagonal block counts only its causal keys);
  * the cumulative-mass comparison is ">= eta"; equal masses are ordered by the
    lower block index; eta >= 1, or a cumulative sum that never reaches eta in
    floating point, selects every admissible block;
  * no block is forced into a support: selection is by mass alone.

Parity of every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, library routines (torch SDPA in float64), invariants and
brute-force enumeration; no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 512  # rows of the attention matrix materialised at a time


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scale(d: int, scale) -> float:
    # The WISE paper, §3 (recurrent attention): logits are divided by sqrt(d_h).
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def causal_attention(q, k, v, scale=None, rows=None):
    """Full causal attention of one head.

    The WISE paper, §3 "Recurrent attention": A = softmax(Q K^T / sqrt(d_h) + M),
    O = A V, with M the causal mask (key j is admissible for query i iff j <= i).
    Written as the two-pass stable softmax: m_i = max_j s_ij, p_ij = exp(s_ij - m_i),
    l_i = sum_j p_ij, O_i = sum_j p_ij v_j / l_i, lse_i = m_i + log l_i.

    q, k, v: [n, d].  rows: optional (r0, r1) query-row range (default all rows).
    Returns (O [r1 - r0, d], lse [r1 - r0]) in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    lo, hi = (0, n) if rows is None else rows
    s = _scale(d, scale)
    out = np.empty((hi - lo, v.shape[1]))
    lse = np.empty(hi - lo)
    for r0 in range(lo, hi, _ROW_CHUNK):
        r1 = min(hi, r0 + _ROW_CHUNK)
        logits = (q[r0:r1] @ k.T) * s
        ri = np.arange(r0, r1)[:, None]
        cj = np.arange(n)[None, :]
        logits[cj > ri] = -np.inf
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        l = p.sum(axis=1, keepdims=True)
        out[r0 - lo:r1 - lo] = (p @ v) / l
        lse[r0 - lo:r1 - lo] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def attention_probs(q, k, scale=None, rows=None):
    """Rows of the causal attention matrix A (the WISE paper, §3), float64.

    rows: optional (r0, r1) range; default all n rows.  Returns [r1 - r0, n].
    """
    q, k = _f64(q), _f64(k)
    n, d = q.shape
    r0, r1 = (0, n) if rows is None else rows
    logits = (q[r0:r1] @ k.T) * _scale(d, scale)
    ri = np.arange(r0, r1)[:, None]
    cj = np.arange(n)[None, :]
    logits[cj > ri] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return p / p.sum(axis=1, keepdims=True)


def block_mass(q, k, block=32, scale=None, qblocks=None):
    """Block-level attention mass of one head, the WISE paper §5.1 (Eq. 5).

    r_qb = (1/|I_q|) * sum_{i in I_q} sum_{j in I_b} A_ij, where I_q are the B rows
    of query block q and I_b the B keys of key block b.  A_ij = 0 for j > i, so
    r_qb = 0 for b > q.  qblocks: optional (q0, q1) query-block range.
    Returns r [q1 - q0, nq] in float64 (all nq query blocks by default).
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    if n % block:
        raise ValueError("sequence length must be a multiple of the block size")
    nq = n // block
    q0, q1 = (0, nq) if qblocks is None else qblocks
    r = np.zeros((q1 - q0, nq))
    rows_per_chunk = max(block, (_ROW_CHUNK // block) * block)
    for r0 in range(q0 * block, q1 * block, rows_per_chunk):
        r1 = min(q1 * block, r0 + rows_per_chunk)
        a = attention_probs(q, k, scale, rows=(r0, r1))        # [rows, n]
        per_key_block = a.reshape(r1 - r0, nq, block).sum(axis=2)  # sum over j in I_b
        per_query_block = per_key_block.reshape((r1 - r0) // block, block, nq).sum(axis=1)
        r[r0 // block - q0:r1 // block - q0] = per_query_block / block  # mean over i in I_q
    return r


def sorted_order(masses):
    """Order of admissible blocks by (mass descending, block index ascending).

    Ties between equal masses go to the lower block index.  np.lexsort sorts by
    its last key first, so the primary key is -mass and the secondary the index.
    """
    masses = _f64(masses)
    idx = np.arange(masses.shape[0])
    return np.lexsort((idx, -masses))


def select_support(masses, eta):
    """Cumulative-eta block support of one (head, query block, step).

    The support of the WISE paper, §3 -- the fewest admissible blocks whose
    masses add up to eta or more -- taken over the block masses of §5.1.  Such a
    minimal set is always a prefix of the blocks ordered by decreasing mass, so
    sort, form the float64 running sum c_k, and keep the first
    k* = min{k : c_k >= eta} blocks.

    masses: the q+1 admissible block masses r_q0 .. r_qq.
    Returns the selected block indices, ascending.
    """
    masses = _f64(masses)
    nb = masses.shape[0]
    if eta >= 1.0:
        return np.arange(nb)
    order = sorted_order(masses)
    c = np.cumsum(masses[order])
    reached = np.nonzero(c >= eta)[0]
    kstar = nb if reached.size == 0 else int(reached[0]) + 1
    return np.sort(order[:kstar])


def size_matched_support(masses, k):
    """SizeMatched control of the WISE paper (App. B, intervention controls):
    TopK(a_q, K_q), the K_q blocks of largest mass, equal masses to the lower
    block index (the same order as the cumulative support).

    masses: the q+1 admissible block masses of one step (step 1 in the paper);
    k: K_q, the size of the WISE working set of the same query block.
    Returns the selected block indices, ascending.
    """
    order = sorted_order(masses)
    return np.sort(order[:max(0, min(int(k), order.shape[0]))])


MASS_MATCH_SLACK = 1e-9


def mass_matched_support(masses, reference, slack=MASS_MATCH_SLACK):
    """MassMatched control of the WISE paper (App. B, intervention controls).

    The paper defines the mass the WISE working set W_q keeps at step 1,
    m_q = sum over j in W_q of a_{q,j}; the control is read here as the
    cumulative support of the same step at threshold m_q: the smallest prefix
    of the blocks sorted by mass whose running sum reaches m_q (at least one
    block).  m_q is summed over W_q's blocks taken in that sorted order, and the
    prefixes are compared with m_q - slack, so that a working set which is
    itself a sorted prefix is matched exactly whatever the rounding of the two
    fp64 sums.

    masses: the q+1 admissible block masses of one step; reference: W_q.
    Returns the selected block indices, ascending.
    """
    masses = _f64(masses)
    order = sorted_order(masses)
    ref = set(int(b) for b in np.asarray(reference).tolist() if 0 <= int(b) < masses.shape[0])
    m = 0.0
    for b in order:
        if int(b) in ref:
            m += masses[b]
    c = np.cumsum(masses[order])
    reached = np.nonzero(c >= m - slack)[0]
    kstar = order.shape[0] if reached.size == 0 else int(reached[0]) + 1
    return np.sort(order[:max(1, kstar)])


def step_supports(r, eta):
    """Per-query-block supports of one head at one step: list of index arrays."""
    nq = r.shape[0]
    return [select_support(r[q, :q + 1], eta) for q in range(nq)]


def union_supports(per_step):
    """Temporal union of supports, the WISE paper App. B (WISE configuration):
    B_q = union over t = t_d-3 .. t_d of B_q^(t, eta), i.e. steps 9..12.

    per_step: list over steps of lists over query blocks of index arrays.
    Returns a list over query blocks of ascending index arrays.
    """
    nq = len(per_step[0])
    out = []
    for q in range(nq):
        acc = set()
        for sup in per_step:
            acc.update(int(b) for b in sup[q])
        out.append(np.array(sorted(acc), dtype=np.int64))
    return out


def expand_supports(supports, nq, block, tile=32):
    """Supports selected at block size ``block`` (a multiple of ``tile``) as
    per-``tile`` rows: tile query block q lists every tile key block k <= q whose
    ``block``-sized key block is selected for q's ``block``-sized query block --
    the keys the reuse mask of §5.2 admits at that block size, on the tile grid
    (the WISE paper, App. B, block-size study).

    supports: list over block-sized query blocks of index arrays; nq: tile-sized
    query blocks.  Returns a list over tile query blocks of ascending arrays.
    """
    f = block // tile
    out = []
    for q in range(nq):
        sel = set(int(b) for b in supports[q // f])
        out.append(np.array([k for k in range(q + 1) if k // f in sel], dtype=np.int64))
    return out


def build_csr(supports):
    """CSR schedule of the WISE paper, App. B (sparse-kernel implementation): row
    offsets plus the active key-block indices of every (head, query block) row.

    supports: list over rows (row = head * nq + q) of ascending index arrays.
    Returns (row_ptr [rows + 1], col_idx [nnz]) as int64 arrays.
    """
    counts = np.array([len(s) for s in supports], dtype=np.int64)
    row_ptr = np.zeros(len(supports) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate([np.asarray(s, dtype=np.int64) for s in supports]) \
        if supports else np.zeros(0, dtype=np.int64)
    return row_ptr, col_idx


def sparse_attention(q, k, v, supports, block=32, scale=None, qblocks=None):
    """Late-step attention restricted to a frozen block support.

    The WISE paper, §5.2: R_ij = 0 if b(j) is in B_q(i), -inf otherwise, added to
    the logits before the softmax together with the causal mask M.  The softmax
    therefore renormalises over the kept keys; it is not a truncated full softmax.

    supports: list over query blocks of block-index arrays (entries b > q have no
    admissible key and change nothing).  A row left with no admissible key (only
    possible for an empty support) gets O = 0 and lse = -inf.  qblocks: optional
    (q0, q1) query-block range; supports is still indexed by absolute query block.
    Returns (O [rows, d], lse [rows]) in float64 for the rows of those blocks.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    nq = n // block
    q0, q1 = (0, nq) if qblocks is None else qblocks
    s = _scale(d, scale)
    out = np.zeros(((q1 - q0) * block, v.shape[1]))
    lse = np.full((q1 - q0) * block, -np.inf)
    key_block = np.arange(n) // block
    for qb in range(q0, q1):
        r0, r1 = qb * block, (qb + 1) * block
        o0, o1 = r0 - q0 * block, r1 - q0 * block
        allowed_block = np.zeros(nq, dtype=bool)
        sup = np.asarray(supports[qb], dtype=np.int64)
        sup = sup[(sup >= 0) & (sup < nq)]
        allowed_block[sup] = True
        logits = (q[r0:r1] @ k.T) * s
        rows = np.arange(r0, r1)[:, None]
        keep = (np.arange(n)[None, :] <= rows) & allowed_block[key_block][None, :]
        logits[~keep] = -np.inf
        live = keep.any(axis=1)
        if not live.any():
            continue
        lg = logits[live]
        m = lg.max(axis=1, keepdims=True)
        p = np.exp(lg - m)
        l = p.sum(axis=1, keepdims=True)
        out[o0:o1][live] = (p @ v) / l
        lse[o0:o1][live] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def boundary_flags(masses, eta, cum_tol=1e-4, tie_tol=1e-6):
    """Blocks whose inclusion in the cumulative-eta support is numerically fragile.

    Follows the nondegeneracy margin of the WISE paper, §6.1 (the minimum margin to
    the ranking and cumulative-mass boundaries).  In sorted order, the block at rank
    s is included iff c_{s-1} < eta (c_{-1} = 0).  It is flagged when
      (i)  |c_{s-1} - eta| <= cum_tol  (the cumulative-mass boundary), or
      (ii) its mass is within tie_tol of a block on the other side of the cut (a
           ranking near-tie).
    Returns (flag_cum, flag_tie): boolean arrays over block indices 0..q.
    """
    masses = _f64(masses)
    nb = masses.shape[0]
    flag_cum = np.zeros(nb, dtype=bool)
    flag_tie = np.zeros(nb, dtype=bool)
    if eta >= 1.0:
        return flag_cum, flag_tie
    order = sorted_order(masses)
    c = np.cumsum(masses[order])
    before = np.concatenate(([0.0], c[:-1]))
    flag_cum[order[np.abs(before - eta) <= cum_tol]] = True
    chosen = select_support(masses, eta)
    inside = np.zeros(nb, dtype=bool)
    inside[chosen] = True
    if inside.all() or not inside.any():
        return flag_cum, flag_tie
    lo_in = masses[inside].min()
    hi_out = masses[~inside].max()
    flag_tie[inside & (masses - hi_out <= tie_tol)] = True
    flag_tie[~inside & (lo_in - masses <= tie_tol)] = True
    return flag_cum, flag_tie


def retained_mass(masses_row, support):
    """Fraction of the block mass of one query block that falls inside a support
    (the WISE paper, App. B "retained future attention mass", per query block)."""
    masses_row = _f64(masses_row)
    sup = np.asarray(support, dtype=np.int64)
    return float(masses_row[sup].sum()) if sup.size else 0.0


def block_density(supports_rows, nq):
    """Fraction of admissible query-key blocks kept (the WISE paper, App. B
    "block density").  supports_rows: list over (head, q) rows, row = h*nq + q."""
    kept = 0
    admissible = 0
    for row, sup in enumerate(supports_rows):
        qb = row % nq
        sup = np.asarray(sup)
        kept += int(np.count_nonzero(sup <= qb))
        admissible += qb + 1
    return kept / admissible if admissible else 0.0


def scheduled_pairs(supports_rows, nq, block=32):
    """Admissible (query, key) pairs visited by the sparse step: B*B for every kept
    block b < q and B*(B+1)/2 for the diagonal block b = q."""
    total = 0
    for row, sup in enumerate(supports_rows):
        qb = row % nq
        for b in np.asarray(sup):
            if b < qb:
                total += block * block
            elif b == qb:
                total += block * (block + 1) // 2
    return total
