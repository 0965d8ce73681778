"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Workloads tiny / 1k / 2k are compared element by element on every head; the
inputs are the seeded synthetic recurrent-step tensors of
block_sparse_attention_wise_amd.synthetic, read identically by both sides.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_wise_amd.synthetic import WORKLOADS, Generator
from parity_helpers import (assert_attn_close, assert_lse_close, assert_mass_close, compare_supports,
                            csr_rows, f64, flagged_row_bound, note, oracle_union_row, record, schedule_from_rows,
                            step_pair)

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = ["tiny", "1k", "2k", "d96", "gqa"]   # d96: head_dim 96; gqa: 8 query / 2 key-value heads


def _wise():
    from block_sparse_attention_wise_amd import wise
    return wise


_GEN = {}


def _gen(name):
    if name not in _GEN:
        _GEN[name] = Generator(WORKLOADS[name])
    return _GEN[name]


@pytest.mark.parametrize("name", SMALL)
def test_dense_attention(name):
    wise, w = _wise(), WORKLOADS[name]
    (q, k, v), dev = step_pair(_gen(name), 1)
    note(f"dense {name}")
    o, lse = wise.dense_attn(*dev, want_lse=True)
    torch.cuda.synchronize()
    for h in range(w.heads):
        ro, rl = O.causal_attention(f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group]))
        assert_attn_close(f64(o[0, h]), ro, w.dtype, f"{name} head {h} O")
        assert_lse_close(f64(lse[0, h]), rl, w.dtype, f"{name} head {h}")


@pytest.mark.parametrize("epilogue", ["one-pass", "sweep"])
@pytest.mark.parametrize("name", SMALL)
def test_discovery_attention_and_block_mass(name, epilogue):
    """Both block-mass epilogues (stored block log-sum-exps, or a second sweep
    over the keys) against the oracle's Eq. 5."""
    wise, w = _wise(), WORKLOADS[name]
    (q, k, v), dev = step_pair(_gen(name), 9)
    note(f"mass {name} {epilogue}")
    o, lse, mass = wise.full_attn_mass(*dev, want_lse=True, want_mass=True,
                                       workspace=None if epilogue == "one-pass" else False)
    torch.cuda.synchronize()
    for h in range(w.heads):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group])
        ro, rl = O.causal_attention(qh, kh, vh)
        assert_attn_close(f64(o[0, h]), ro, w.dtype, f"{name} head {h} O")
        assert_lse_close(f64(lse[0, h]), rl, w.dtype, f"{name} head {h}")
        assert_mass_close(f64(mass[h]), O.block_mass(qh, kh), w.dtype, f"{name} head {h}")


def _oracle_masses(name, steps=(9, 10, 11, 12)):
    w, g = WORKLOADS[name], _gen(name)
    out = np.zeros((len(steps), w.heads, w.nq, w.nq))
    for si, t in enumerate(steps):
        q, k, _ = g.step_torch(t)
        for h in range(w.heads):
            out[si, h] = O.block_mass(f64(q[0, h]), f64(k[0, h // w.group]))
    return out


@pytest.mark.parametrize("name", SMALL)
def test_build_support_on_fed_masses_is_exact(name):
    """Both sides select from the same fp32 masses (upcast to fp64): supports must
    agree exactly (flags only at summation-order level, 1e-12)."""
    wise, w = _wise(), WORKLOADS[name]
    m32 = _oracle_masses(name).astype(np.float32)
    eta = w.etas[0]
    note(f"build_support fed {name}")
    sched = wise.build_support(torch.from_numpy(m32).to(DEV), eta)
    torch.cuda.synchronize()
    gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
    assert int(sched.nnz.item()) == int(sched.row_ptr[-1].item())
    ref_rows, flags = [], []
    for h in range(w.heads):
        for qb in range(w.nq):
            sup, fl = oracle_union_row([m32[s, h, qb, :qb + 1].astype(np.float64) for s in range(4)], eta,
                                       cum_tol=1e-12, tie_tol=0.0)
            ref_rows.append(sup)
            flags.append(fl)
    bad, flagged = compare_supports(gpu_rows, ref_rows, flags)
    assert not bad, f"{len(bad)} rows differ, first {bad[:3]}"
    assert flagged == 0


@pytest.mark.parametrize("name,t", [("tiny", 2), ("1k", 1), ("1k", 2), ("1k", 3), ("1k", 4), ("1k", 7)])
def test_rolling_window_supports(name, t):
    """The rolling working set of the WISE paper (App. C.2), W^(t) = union of the
    supports of steps max(1, t - 3) .. t: the builder over that window's masses
    (1, 2, 3 or 4 steps) against the oracle's union over the same steps, both
    selecting from the same fp32 masses (exact; flags at summation order only)."""
    wise, w = _wise(), WORKLOADS[name]
    window = tuple(range(max(1, t - 3), t + 1))
    m32 = _oracle_masses(name, steps=window).astype(np.float32)
    eta = w.etas[0]
    note(f"rolling window {name} t={t} steps {window}")
    sched = wise.build_support(torch.from_numpy(m32).to(DEV), eta)
    torch.cuda.synchronize()
    gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
    ref_rows, flags = [], []
    for h in range(w.heads):
        per_step = [O.step_supports(m32[s, h].astype(np.float64), eta) for s in range(len(window))]
        union = O.union_supports(per_step)
        for qb in range(w.nq):
            _, fl = oracle_union_row([m32[s, h, qb, :qb + 1].astype(np.float64) for s in range(len(window))], eta,
                                     cum_tol=1e-12, tie_tol=0.0)
            ref_rows.append(union[qb])
            flags.append(fl)
    bad, flagged = compare_supports(gpu_rows, ref_rows, flags)
    assert not bad, f"{len(bad)} rows differ, first {bad[:3]}"
    assert flagged == 0
    record(f"rolling window {name} t={t} ({len(window)} steps)", rows=len(ref_rows), flagged_blocks=flagged)


def test_build_support_exact_ties_and_eta_edges():
    """Exact ties (dyadic masses) go to the lower block index; eta = 1 keeps all."""
    wise = _wise()
    rng = np.random.default_rng(5)
    bh, nq = 3, 40
    m = np.zeros((4, bh, nq, nq), dtype=np.float32)
    for s in range(4):
        for r in range(bh):
            for qb in range(nq):
                raw = rng.integers(1, 4, size=qb + 1).astype(np.float64)
                m[s, r, qb, :qb + 1] = raw / 2 ** np.ceil(np.log2(raw.sum()))  # dyadic, ties frequent
    for eta in (0.3, 0.5, 0.75, 0.9, 1.0):
        note(f"build_support ties eta={eta}")
        sched = wise.build_support(torch.from_numpy(m).to(DEV), eta)
        gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
        for r in range(bh):
            for qb in range(nq):
                sup, _ = oracle_union_row([m[s, r, qb, :qb + 1].astype(np.float64) for s in range(4)], eta,
                                          cum_tol=0.0, tie_tol=0.0)
                np.testing.assert_array_equal(gpu_rows[r * nq + qb], sup)


@pytest.mark.parametrize("name", SMALL)
def test_sparse_attention_on_oracle_schedule(name):
    wise, w = _wise(), WORKLOADS[name]
    masses = _oracle_masses(name)
    eta = w.etas[0]
    rows = []
    for h in range(w.heads):
        per_step = [O.step_supports(masses[s, h], eta) for s in range(4)]
        rows += O.union_supports(per_step)
    sched = schedule_from_rows(rows, DEV)
    for t in (13, 32):
        (q, k, v), dev = step_pair(_gen(name), t)
        note(f"sparse {name} step {t}")
        o, lse = wise.sparse_attn(*dev, sched, want_lse=True)
        torch.cuda.synchronize()
        for h in range(w.heads):
            ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group]),
                                        rows[h * w.nq:(h + 1) * w.nq])
            assert_attn_close(f64(o[0, h]), ro, w.dtype, f"{name} step {t} head {h} O")
            assert_lse_close(f64(lse[0, h]), rl, w.dtype, f"{name} step {t} head {h}")


@pytest.mark.parametrize("name", SMALL)
def test_end_to_end_trajectory(name):
    """GPU masses -> GPU schedule vs the oracle's, then GPU sparse steps vs oracle.

    Supports must match the oracle's exactly outside boundary-flagged blocks, and
    at most 1% of the rows (at least 2) may differ in flagged blocks.  Every
    row's output is compared with the oracle's sparse attention over the GPU's
    own schedule (for the rows whose support matches, that is the oracle's)."""
    wise, w = _wise(), WORKLOADS[name]
    eta = w.etas[0]
    g = _gen(name)
    mass = torch.empty((4, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        note(f"e2e {name} discovery step {t}")
        wise.full_attn_mass(q, k, v, mass=mass[si])
    sched = wise.build_support(mass, eta)
    torch.cuda.synchronize()
    gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
    masses = _oracle_masses(name)
    ref_rows, flags = [], []
    for h in range(w.heads):
        for qb in range(w.nq):
            sup, fl = oracle_union_row([masses[s, h, qb, :qb + 1] for s in range(4)], eta)
            ref_rows.append(sup)
            flags.append(fl)
    flagged_rows = []
    bad, flagged = compare_supports(gpu_rows, ref_rows, flags, flagged_rows)
    note(f"e2e {name}: flagged mismatching rows {len(flagged_rows)}, blocks {flagged}")
    assert not bad, f"{len(bad)} rows differ outside flagged blocks, first {bad[:3]}"
    assert len(flagged_rows) <= flagged_row_bound(len(ref_rows)), f"{len(flagged_rows)} flagged rows"
    (q, k, v), dev = step_pair(g, 20)
    note(f"e2e {name} sparse step 20")
    o, lse = wise.sparse_attn(*dev, sched, want_lse=True)
    torch.cuda.synchronize()
    worst_abs = worst_tol = 0.0
    for h in range(w.heads):
        ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group]),
                                    gpu_rows[h * w.nq:(h + 1) * w.nq])
        ea, er = assert_attn_close(f64(o[0, h]), ro, w.dtype, f"{name} head {h} O")
        assert_lse_close(f64(lse[0, h]), rl, w.dtype, f"{name} head {h}")
        worst_abs, worst_tol = max(worst_abs, ea), max(worst_tol, er)
    record(f"trajectory {name} (eta {eta}, step 20, all rows)", rows=len(ref_rows),
           flagged_rows=len(flagged_rows), flagged_blocks=flagged, max_abs=worst_abs, tol_used=worst_tol)


@pytest.mark.parametrize("name", ["tiny", "1k"])
def test_eta_one_sparse_equals_dense(name):
    wise, w = _wise(), WORKLOADS[name]
    g = _gen(name)
    mass = torch.empty((4, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        wise.full_attn_mass(q, k, v, mass=mass[si])
    note(f"eta=1 {name}")
    sched = wise.build_support(mass, 1.0)
    assert int(sched.nnz.item()) == w.heads * w.nq * (w.nq + 1) // 2
    (q, k, v), dev = step_pair(g, 13)
    os_, ls = wise.sparse_attn(*dev, sched, want_lse=True)
    od, ld = wise.dense_attn(*dev, want_lse=True)
    torch.cuda.synchronize()
    # same blocks in the same order; only instruction scheduling may differ
    assert_attn_close(f64(os_), f64(od), w.dtype, "sparse(eta=1) vs dense")
    assert float((ls - ld).abs().max()) <= 1e-5
    for h in range(w.heads):
        ro, _ = O.causal_attention(f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group]))
        assert_attn_close(f64(os_[0, h]), ro, w.dtype, "sparse(eta=1) vs oracle full")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("batch,heads,kv,n", [(1, 1, 1, 32), (2, 3, 3, 96), (1, 2, 2, 160), (2, 4, 2, 96),
                                               (1, 6, 1, 64), (1, 11, 11, 64), (2, 13, 1, 96)])
def test_shapes_batch_and_head_dim(dtype, d, batch, heads, kv, n):
    wise = _wise()
    rng = np.random.default_rng(batch * 100 + heads * 10 + n + d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mk = lambda hh, s: torch.from_numpy(rng.standard_normal((batch, hh, n, d)).astype(np.float32) * s).to(tdt)
    q, k, v = mk(heads, 1.5), mk(kv, 1.5), mk(kv, 1.0)
    grp = heads // kv
    nq = n // 32
    note(f"shapes {dtype} d={d} b={batch} h={heads} kv={kv} n={n}")
    o, lse, mass = wise.full_attn_mass(q.to(DEV), k.to(DEV), v.to(DEV), want_lse=True, want_mass=True)
    rows = []
    for bb in range(batch):
        for h in range(heads):
            rows += [np.nonzero(rng.random(qb + 1) < 0.6)[0] for qb in range(nq)]
    rows = [r if r.size else np.array([0]) for r in rows]
    sched = schedule_from_rows(rows, DEV)
    so, sl = wise.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), sched, want_lse=True)
    torch.cuda.synchronize()
    for bb in range(batch):
        for h in range(heads):
            qh, kh, vh = f64(q[bb, h]), f64(k[bb, h // grp]), f64(v[bb, h // grp])
            ro, rl = O.causal_attention(qh, kh, vh)
            assert_attn_close(f64(o[bb, h]), ro, dtype, "dense O")
            assert_lse_close(f64(lse[bb, h]), rl, dtype, "dense")
            assert_mass_close(f64(mass[bb * heads + h]), O.block_mass(qh, kh), dtype, "mass")
            r0 = (bb * heads + h) * nq
            ro, rl = O.sparse_attention(qh, kh, vh, rows[r0:r0 + nq])
            assert_attn_close(f64(so[bb, h]), ro, dtype, "sparse O")
            assert_lse_close(f64(sl[bb, h]), rl, dtype, "sparse")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sparse_ignores_invalid_entries_and_handles_empty_rows(dtype):
    wise = _wise()
    rng = np.random.default_rng(11)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n, d, nq = 128, 128, 4
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 1, n, d)).astype(np.float32)).to(tdt) for _ in range(3))
    # row 0 empty; row 1 lists b > q and negative; row 2 unsorted with an out-of-range id;
    # row 3 lists each of its blocks twice (a block listed twice counts once)
    rp = np.array([0, 0, 4, 8, 12], dtype=np.int32)
    ci = np.array([3, 1, -5, 0, 2, 99, 0, 7, 0, 3, 3, 0], dtype=np.int32)
    sched = wise.Schedule(torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV),
                          torch.tensor([12], dtype=torch.int32, device=DEV), 1, nq)
    note(f"sparse invalid entries {dtype}")
    o = torch.full((1, 1, n, d), float("nan"), dtype=tdt, device=DEV)
    lse = torch.full((1, 1, n), float("nan"), dtype=torch.float32, device=DEV)
    wise.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), sched, out=o, lse=lse)
    torch.cuda.synchronize()
    clean = [np.array([], dtype=np.int64), np.array([0, 1]), np.array([0, 2]), np.array([0, 3])]
    ro, rl = O.sparse_attention(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), clean)
    assert_attn_close(f64(o[0, 0]), ro, dtype, "O")
    assert_lse_close(f64(lse[0, 0]), rl, dtype, "lse")
    assert torch.all(o[0, 0, :32] == 0)


def test_sparse_col_capacity_bounds_reads():
    """Offsets past col_capacity are clamped: the row sees only readable entries."""
    wise = _wise()
    rng = np.random.default_rng(12)
    n, d = 64, 128
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 1, n, d)).astype(np.float32)).to(torch.bfloat16)
               for _ in range(3))
    rp = torch.tensor([0, 1, 1000], dtype=torch.int32, device=DEV)
    ci = torch.tensor([0, 1, 0], dtype=torch.int32, device=DEV)   # capacity 3 < 1000
    sched = wise.Schedule(rp, ci, torch.tensor([3], dtype=torch.int32, device=DEV), 1, 2)
    note("sparse col capacity")
    o, lse = wise.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), sched, want_lse=True)
    torch.cuda.synchronize()
    ro, rl = O.sparse_attention(f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0]), [np.array([0]), np.array([1, 0])])
    assert_attn_close(f64(o[0, 0]), ro, "bf16", "O")


def test_deterministic_and_poison_overwritten():
    wise, w = _wise(), WORKLOADS["1k"]
    g = _gen("1k")
    q, k, v = g.step_torch(9, DEV)
    outs = []
    for rep in range(2):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, w.heads, w.seqlen), float("nan"), device=DEV)
        mass = torch.full((w.heads, w.nq, w.nq), float("nan"), device=DEV)
        note(f"determinism rep {rep}")
        wise.full_attn_mass(q, k, v, out=o, lse=lse, mass=mass)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all() and torch.isfinite(mass).all()
        outs.append((o.clone(), lse.clone(), mass.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    m4 = torch.stack([outs[0][2]] * 4)
    s1 = wise.build_support(m4, 0.95)
    s2 = wise.build_support(m4, 0.95)
    torch.cuda.synchronize()
    assert torch.equal(s1.row_ptr, s2.row_ptr)
    nnz = int(s1.nnz.item())
    assert torch.equal(s1.col_idx[:nnz], s2.col_idx[:nnz])


def test_uniform_attention_closed_form_on_gpu():
    """Q = 0 gives uniform causal attention: masses equal the rational closed form
    and every admissible block ties in score, exercising the tie-break path."""
    wise = _wise()
    n, d = 256, 128
    rng = np.random.default_rng(3)
    q = torch.zeros((1, 1, n, d), dtype=torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((1, 1, n, d)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, 1, n, d)).astype(np.float32)).to(torch.bfloat16)
    note("uniform closed form")
    o, lse, mass = wise.full_attn_mass(q.to(DEV), k.to(DEV), v.to(DEV), want_lse=True, want_mass=True)
    torch.cuda.synchronize()
    vv = f64(v[0, 0])
    expect = np.cumsum(vv, axis=0) / np.arange(1, n + 1)[:, None]
    assert_attn_close(f64(o[0, 0]), expect, "bf16", "uniform O")
    np.testing.assert_allclose(f64(lse[0, 0]), np.log(np.arange(1, n + 1)), atol=1e-5)
    assert_mass_close(f64(mass[0]), O.block_mass(np.zeros((n, d)), f64(k[0, 0])), "bf16", "uniform mass")


def _expected_units(counts, nq, nnz, slots, row_ptr_h, col_idx):
    """The work units of wise_build_support, on the host, for one head: unit
    length L = max(4, m, min(ceil(nnz / slots), 3 m)), m = ceil(head blocks / nq)
    the head's mean row length; a row of n > L
    blocks splits in P = 2 parts (n <= 2 L) or 4; units of 4-part rows, then
    2-part rows, then whole rows, each by ceil(n / P) descending, then row, then
    part; each as (row << 8) | (part << 4) | (P - 1), the part's CSR entries
    [e0, e1) (part p of n entries: n p / P .. n (p + 1) / P) and its first block."""
    mean = -(-sum(counts) // nq)
    length = max(4, mean, min(-(-nnz // slots), 3 * mean))
    units = []
    for r, n in enumerate(counts):
        parts = 1 if n <= length else (2 if n <= 2 * length else 4)
        ul = -(-n // parts)
        cls = {4: 0, 2: 1, 1: 2}[parts]
        units += [(cls, -ul, r, p, parts) for p in range(parts)]
    units.sort()
    out = []
    for _, _, r, p, parts in units:
        n = counts[r]
        e0, e1 = row_ptr_h[r] + n * p // parts, row_ptr_h[r] + n * (p + 1) // parts
        out.append([(r << 8) | (p << 4) | (parts - 1), e0, e1, int(col_idx[e0]) if e1 > e0 else -1])
    return out


@pytest.mark.parametrize("bh,nq,eta", [(3, 37, 0.9), (2, 8, 0.5), (1, 130, 0.95), (2, 5, 1.0), (1, 300, 0.99),
                                       (2, 64, 0.9), (11, 16, 0.9), (1, 1100, 0.95)])
def test_work_units_split_long_rows(bh, nq, eta):
    """The schedule's work units: per head a count, then its rows (longer rows
    split in parts of their CSR entries) longest first -- the rule written out on
    the host, bitonic-sorted on the GPU up to 2 nq units.  Sparse attention
    through the units (split rows merged from their parts) gives the oracle's
    values, and the same values as without units up to summation order."""
    wise = _wise()
    rng = np.random.default_rng(bh * 1000 + nq)
    m = np.zeros((4, bh, nq, nq), dtype=np.float32)
    for s in range(4):
        for r in range(bh):
            for qb in range(nq):
                m[s, r, qb, :qb + 1] = rng.dirichlet(np.full(qb + 1, 0.4))
    note(f"work units bh={bh} nq={nq} eta={eta}")
    sched = wise.build_support(torch.from_numpy(m).to(DEV), eta)
    torch.cuda.synchronize()
    base = (bh + 3) // 4 * 4
    assert sched.plan is not None and sched.plan.numel() == base + bh * 4 * nq * 4
    plan = sched.plan.cpu().numpy()
    rp_host = sched.row_ptr.cpu().numpy()
    ci_host = sched.col_idx.cpu().numpy()
    gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
    ref_rows, flags = [], []
    for r in range(bh):
        for qb in range(nq):
            sup, fl = oracle_union_row([m[s, r, qb, :qb + 1].astype(np.float64) for s in range(4)], eta)
            ref_rows.append(sup)
            flags.append(fl)
    bad, _ = compare_supports(gpu_rows, ref_rows, flags)
    assert not bad
    slots = torch.cuda.get_device_properties(0).multi_processor_count * 8
    nnz = int(sched.nnz.item())
    split = 0
    for h in range(bh):
        counts = [len(gpu_rows[h * nq + q]) for q in range(nq)]
        want = _expected_units(counts, nq, nnz, slots, rp_host[h * nq:(h + 1) * nq], ci_host)
        got = plan[base + h * 4 * nq * 4:base + (h + 1) * 4 * nq * 4].reshape(4 * nq, 4)
        assert int(plan[h]) == len(want) <= 4 * nq, f"head {h}: unit count"
        assert got[:len(want)].tolist() == want, f"head {h}: units"
        assert np.all(got[len(want):] == -1)
        split += sum(1 for u in want if (u[0] & 15) > 0)
    # cover the split path: a schedule whose units include split rows ...
    n, d = 32 * nq, 128
    if nq > 300:
        return
    q, k, v = (torch.from_numpy(rng.standard_normal((1, bh, n, d)).astype(np.float32)).to(torch.bfloat16)
               for _ in range(3))
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    op, lp = wise.sparse_attn(dq, dk, dv, sched, want_lse=True)
    csr_only = wise.Schedule(sched.row_ptr, sched.col_idx, sched.nnz, bh, nq)
    oc, lc = wise.sparse_attn(dq, dk, dv, csr_only, want_lse=True)
    # ... and the same schedule with every row forced into 4 parts (hand-made units,
    # one workgroup per row; rows with fewer than 4 blocks leave parts empty:
    # log-sum-exp -inf, weight 0)
    forced = np.full(base + bh * 4 * nq * 4, -1, dtype=np.int32)
    for h in range(bh):
        forced[h] = 4 * nq
        us = []
        for qb in range(nq):
            r0, n_ = int(rp_host[h * nq + qb]), int(rp_host[h * nq + qb + 1] - rp_host[h * nq + qb])
            for p in range(4):
                e0, e1 = r0 + n_ * p // 4, r0 + n_ * (p + 1) // 4
                # the first block as the builder writes it (parts 0, 3), left out (part 1: the
                # kernel finds it from the CSR) or wrong (part 2: the kernel drops that copy)
                fb = int(ci_host[e0]) if e1 > e0 else -1
                us.append([(qb << 8) | (p << 4) | 3, e0, e1, {1: -1, 2: qb}.get(p, fb)])
        forced[base + h * 4 * nq * 4:base + (h + 1) * 4 * nq * 4] = np.array(us, dtype=np.int32).ravel()
    rows_forced = set(range(nq))
    fsched = wise.Schedule(sched.row_ptr, sched.col_idx, sched.nnz, bh, nq, plan=torch.from_numpy(forced).to(DEV))
    of, lf = wise.sparse_attn(dq, dk, dv, fsched, want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(f64(op), f64(oc), "bf16", "units vs CSR O")
    assert float((lp - lc).abs().max()) <= 1e-5
    for h in range(bh):
        rows_h = ref_rows[h * nq:(h + 1) * nq]
        ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), rows_h)
        keep = np.zeros(n, dtype=bool)
        kf = np.zeros(n, dtype=bool)
        for qb in range(nq):
            if set(gpu_rows[h * nq + qb].tolist()) == set(rows_h[qb].tolist()):
                keep[32 * qb:32 * qb + 32] = True
                kf[32 * qb:32 * qb + 32] = qb in rows_forced
        assert_attn_close(f64(op[0, h])[keep], ro[keep], "bf16", f"units head {h} O")
        assert_lse_close(f64(lp[0, h])[keep], rl[keep], "bf16", f"units head {h}")
        assert_attn_close(f64(of[0, h])[kf], ro[kf], "bf16", f"4-part rows head {h} O")
        assert_lse_close(f64(lf[0, h])[kf], rl[kf], "bf16", f"4-part rows head {h}")
    record(f"work units bh={bh} nq={nq} eta={eta}", rows=bh * nq, split_parts=split)


def test_high_dynamic_range_logits():
    """Logits spread over more than 60 (natural-log units) and a dominant key
    whose logit lifts the running maximum by tens of units in the middle of the
    rows: dense attention, both block-mass epilogues and sparse attention (with
    the schedule's row order) against the oracle (the GPU counterpart of the oracle's
    dominant-key pin)."""
    wise = _wise()
    rng = np.random.default_rng(77)
    n, d, heads, nq = 1024, 128, 2, 32
    s = np.sqrt(20.0)                       # q.k / sqrt(d) has standard deviation s^2 = 20
    q = rng.standard_normal((1, heads, n, d)) * s
    k = rng.standard_normal((1, heads, n, d)) * s
    v = rng.standard_normal((1, heads, n, d))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q[:, :, 480:] += 40.0 * u               # queries 480.. share a direction ...
    k[:, :, 500] += 40.0 * u                # ... that key 500 carries: about +140 for rows >= 500
    q, k, v = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v))
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    note("high dynamic range: dense, masses, sparse")
    o, lse = wise.dense_attn(dq, dk, dv, want_lse=True)
    _, _, m1 = wise.full_attn_mass(dq, dk, dv, want_mass=True)
    _, _, m2 = wise.full_attn_mass(dq, dk, dv, want_mass=True, workspace=False)
    sched = wise.build_support(m1.unsqueeze(0).contiguous(), 0.95)
    os_, ls_ = wise.sparse_attn(dq, dk, dv, sched, want_lse=True)
    torch.cuda.synchronize()
    rows = csr_rows(sched.row_ptr, sched.col_idx)
    worst = [0.0, 0.0]
    for h in range(heads):
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        logits = (qh @ kh.T) / np.sqrt(d)
        causal = np.tril(np.ones((n, n), dtype=bool))
        span = logits[causal].max() - logits[causal].min()
        assert span > 60 and logits[600, 500] - np.delete(logits[600, :601], 500).max() > 20
        ro, rl = O.causal_attention(qh, kh, vh)
        ea, er = assert_attn_close(f64(o[0, h]), ro, "bf16", f"hdr dense head {h} O")
        assert_lse_close(f64(lse[0, h]), rl, "bf16", f"hdr dense head {h}")
        rm = O.block_mass(qh, kh)
        assert_mass_close(f64(m1[h]), rm, "bf16", f"hdr one-pass mass head {h}")
        assert_mass_close(f64(m2[h]), rm, "bf16", f"hdr sweep mass head {h}")
        so, sl = O.sparse_attention(qh, kh, vh, rows[h * nq:(h + 1) * nq])
        es, rs = assert_attn_close(f64(os_[0, h]), so, "bf16", f"hdr sparse head {h} O")
        assert_lse_close(f64(ls_[0, h]), sl, "bf16", f"hdr sparse head {h}")
        worst = [max(worst[0], ea, es), max(worst[1], er, rs)]
    record("high dynamic range (logit span > 60, dominant key)", rows=heads * nq, max_abs=worst[0],
           tol_used=worst[1])


def test_maximum_context_schedule_units_and_sparse_rows():
    """The longest context the bf16 path takes: 4096 query blocks (n = 131072, one
    head, d = 64), masses fed for two discovery steps.  Sampled rows on both of
    the selection kernel's paths (rows of up to 1024 blocks sorted by one
    wavefront per step, longer rows by the whole workgroup, keys up to 4096 per
    row) match the oracle outside boundary-flagged blocks; the work units follow
    the host rule (4 nq unit slots, the unit sort's largest LDS buffer); sparse
    attention of sampled query blocks, through the units, matches the oracle
    over the GPU's own rows."""
    wise = _wise()
    nq, d, steps, eta = 4096, 64, 2, 0.9
    n = 32 * nq
    rng = np.random.default_rng(131072)
    m = np.zeros((steps, 1, nq, nq), dtype=np.float32)
    for s in range(steps):
        g = np.tril(rng.gamma(0.4, size=(nq, nq)))  # Dirichlet(0.4) rows over blocks 0..q
        m[s, 0] = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
        del g
    note(f"maximum context: build nq={nq}")
    sched = wise.build_support(torch.from_numpy(m).to(DEV), eta)
    torch.cuda.synchronize()
    rp_host = sched.row_ptr.cpu().numpy()
    ci_host = sched.col_idx.cpu().numpy()
    nnz = int(sched.nnz.item())
    assert nnz == int(rp_host[-1])
    gpu_rows = [np.sort(ci_host[rp_host[r]:rp_host[r + 1]]) for r in range(nq)]
    sample = [0, 1, 511, 1022, 1023, 1024, 1025, 2047, 2048, 3001, 4094, 4095]
    flagged_rows = 0
    for qb in sample:
        sup, flags = oracle_union_row([m[s, 0, qb, :qb + 1].astype(np.float64) for s in range(steps)], eta)
        diff = set(gpu_rows[qb].tolist()) ^ set(sup.tolist())
        assert diff <= flags, f"row {qb}: unflagged mismatch {sorted(diff - flags)[:8]}"
        flagged_rows += int(bool(diff))
    assert flagged_rows <= flagged_row_bound(len(sample))
    # work units: the host rule over the GPU's own rows
    base = 4
    plan = sched.plan.cpu().numpy()
    slots = torch.cuda.get_device_properties(0).multi_processor_count * 8
    want = _expected_units([len(r) for r in gpu_rows], nq, nnz, slots, rp_host[:nq], ci_host)
    got = plan[base:base + 4 * nq * 4].reshape(4 * nq, 4)
    assert int(plan[0]) == len(want) <= 4 * nq
    assert got[:len(want)].tolist() == want
    assert np.all(got[len(want):] == -1)
    # sparse attention through the units, sampled query blocks against the oracle
    tg = torch.Generator().manual_seed(4096)
    q, k, v = (torch.randn((1, 1, n, d), generator=tg).to(torch.bfloat16) for _ in range(3))
    note(f"maximum context: sparse attention n={n}")
    o, lse = wise.sparse_attn(q.to(DEV), k.to(DEV), v.to(DEV), sched, want_lse=True)
    torch.cuda.synchronize()
    qh, kh, vh = f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0])
    worst_abs = worst_tol = 0.0
    for qb in sample:
        rows = [np.array([0])] * nq
        rows[qb] = gpu_rows[qb]
        ro, rl = O.sparse_attention(qh, kh, vh, rows, qblocks=(qb, qb + 1))
        sl = slice(32 * qb, 32 * qb + 32)
        ea, er = assert_attn_close(f64(o[0, 0, sl]), ro, "bf16", f"maximum context block {qb} O")
        assert_lse_close(f64(lse[0, 0, sl]), rl, "bf16", f"maximum context block {qb}")
        worst_abs, worst_tol = max(worst_abs, ea), max(worst_tol, er)
    split = sum(1 for u in want if (u[0] & 15) > 0)
    record(f"maximum context nq={nq} (n {n}, eta {eta}, {steps} steps)", rows=len(sample), nnz=nnz,
           split_parts=split, flagged_rows=flagged_rows, max_abs=worst_abs, tol_used=worst_tol)


def test_sparse_repeated_launches_and_graph_replays():
    """The bf16 sparse kernel with work units, launched back to back and replayed
    from a captured graph (with other work between the replays), gives outputs
    bit-identical to its first launch, and agrees with the CSR walk over the same
    schedule."""
    wise, w = _wise(), WORKLOADS["2k"]
    g = _gen("2k")
    mass = torch.empty((4, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        wise.full_attn_mass(q, k, v, mass=mass[si])
    sched = wise.build_support(mass, 0.95)
    q, k, v = g.step_torch(13, DEV)
    ref, ref_lse = wise.sparse_attn(q, k, v, sched, want_lse=True)
    ref, ref_lse = ref.clone(), ref_lse.clone()
    o = torch.empty_like(q)
    lse = torch.empty_like(ref_lse)
    for rep in range(3):
        note(f"repeated sparse launch {rep}")
        o.fill_(float("nan"))
        wise.sparse_attn(q, k, v, sched, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_lse)
    note("sparse graph capture")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            wise.sparse_attn(q, k, v, sched, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        note(f"sparse graph replay {rep}")
        o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref) and torch.equal(lse, ref_lse)
        wise.dense_attn(q, k, v)  # other work between the replays
        torch.cuda.synchronize()
    csr_only = wise.Schedule(sched.row_ptr, sched.col_idx, sched.nnz, w.heads, w.nq)
    oc, lc = wise.sparse_attn(q, k, v, csr_only, want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(f64(ref), f64(oc), "bf16", "units vs CSR O")
    assert float((ref_lse - lc).abs().max()) <= 1e-5
    record("sparse repeated launches (2k, 3 launches, 3 graph replays)", rows=w.heads * w.nq)


@pytest.mark.parametrize("name", ["2k", "huginn4k"])
def test_sparse_bundle_order_does_not_change_results(name):
    """Order independence of the work-unit sparse kernel: the builder's units,
    with the bundles of every head reversed, and shuffled, run the same units on
    other workgroups in another order (a permuted grid), and must give outputs
    and log-sum-exps bit-identical to the builder's order.  Every output row is
    written by one wavefront (a split row merged inside its bundle in a fixed
    order), so nothing may depend on which workgroup runs it or when."""
    wise, w = _wise(), WORKLOADS[name]
    g = _gen(name)
    bh, nq = w.batch * w.heads, w.nq
    mass = torch.empty((4, bh, nq, nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        wise.full_attn_mass(q, k, v, mass=mass[si])
    sched = wise.build_support(mass, w.etas[0])
    q, k, v = g.step_torch(17, DEV)
    ref, ref_lse = wise.sparse_attn(q, k, v, sched, want_lse=True)
    torch.cuda.synchronize()
    plan = sched.plan.cpu().numpy()
    base = (bh + 3) // 4 * 4
    cap = 4 * nq
    rng = np.random.default_rng(7)
    split_bundles = 0
    for order in ("reversed", "shuffled"):
        perm = plan.copy()
        for h in range(bh):
            units = int(plan[h])
            nb = (units + 3) // 4
            slots = plan[base + h * cap * 4:base + (h + 1) * cap * 4].reshape(cap, 4)
            bundles = slots[:4 * nb].reshape(nb, 4, 4)
            split_bundles += int(np.sum(np.any((bundles[:, :, 0] >= 0) & ((bundles[:, :, 0] & 15) > 0), axis=1)))
            idx = np.arange(nb)[::-1] if order == "reversed" else rng.permutation(nb)
            out = np.full((cap, 4), -1, dtype=np.int32)
            out[:4 * nb] = bundles[idx].reshape(4 * nb, 4)
            # the count covers every slot of the last bundle: unused slots hold -1 units
            perm[h] = 4 * nb
            perm[base + h * cap * 4:base + (h + 1) * cap * 4] = out.ravel()
        note(f"bundle order {order} ({name})")
        psched = wise.Schedule(sched.row_ptr, sched.col_idx, sched.nnz, bh, nq, plan=torch.from_numpy(perm).to(DEV))
        o = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        wise.sparse_attn(q, k, v, psched, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"{order}: outputs differ"
        assert torch.equal(lse, ref_lse), f"{order}: log-sum-exps differ"
    assert split_bundles > 0  # the permutation moved split rows too
    record(f"sparse bundle order ({name}: reversed, shuffled)", rows=bh * nq, split_bundles=split_bundles // 2)
