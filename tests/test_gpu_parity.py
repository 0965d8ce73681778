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
                            csr_rows, f64, note, oracle_union_row, schedule_from_rows, step_pair)

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
    """GPU masses -> GPU schedule vs the oracle's, then GPU sparse steps vs oracle."""
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
    bad, flagged = compare_supports(gpu_rows, ref_rows, flags)
    note(f"e2e {name}: flagged mismatching blocks {flagged}")
    assert not bad, f"{len(bad)} rows differ outside flagged blocks, first {bad[:3]}"
    same = [r for r in range(len(ref_rows)) if np.array_equal(gpu_rows[r], ref_rows[r])]
    (q, k, v), dev = step_pair(g, 20)
    note(f"e2e {name} sparse step 20")
    o, lse = wise.sparse_attn(*dev, sched, want_lse=True)
    torch.cuda.synchronize()
    for h in range(w.heads):
        ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group]),
                                    ref_rows[h * w.nq:(h + 1) * w.nq])
        keep = np.zeros(w.seqlen, dtype=bool)
        for r in same:
            if r // w.nq == h:
                keep[(r % w.nq) * 32:(r % w.nq + 1) * 32] = True
        assert_attn_close(f64(o[0, h])[keep], ro[keep], w.dtype, f"{name} head {h} O")
        assert_lse_close(f64(lse[0, h])[keep], rl[keep], w.dtype, f"{name} head {h}")


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
    # row 0 empty; row 1 lists b > q and negative; row 2 unsorted with an out-of-range id; row 3 normal
    rp = np.array([0, 0, 4, 8, 10], dtype=np.int32)
    ci = np.array([3, 1, -5, 0, 2, 99, 0, 7, 0, 3], dtype=np.int32)
    sched = wise.Schedule(torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV),
                          torch.tensor([10], dtype=torch.int32, device=DEV), 1, nq)
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


def _decode_plan(plan, bh, nq, rows_per_group=4):
    """plan (host int32) -> {group: (rows, [(block, membership), ...])} in plan order:
    entry counts plan[0..G), the slot stride plan[G] = nq, four row indices per
    group from plan[G + 1], group g's entries in its slot plan[5 G + 1 + g nq ..],
    with G = bh (ceil(nq / 4) + ceil(nq / 16))."""
    gh = (nq + rows_per_group - 1) // rows_per_group + (nq + 15) // 16
    groups = bh * gh
    cnt = plan[:groups]
    assert int(plan[groups]) == nq and np.all(cnt >= 0) and np.all(cnt <= nq)
    rows = plan[groups + 1:groups + 1 + rows_per_group * groups].reshape(groups, rows_per_group)
    ent = plan[groups + 1 + rows_per_group * groups:]
    out = {}
    for g in range(groups):
        r = [int(x) for x in rows[g]]
        valid = [x for x in r if x >= 0]
        assert r == valid + [-1] * (rows_per_group - len(valid)), f"group {g} rows {r}"
        out[g] = (valid, [(int(e) >> 8, int(e) & 255) for e in ent[g * nq:g * nq + cnt[g]]])
    return out, gh


def _expected_groups(rows_h, nq, gh, max_count, head_dim=0):
    """The grouping rule of wise_build_support's plan, on the host: a head's rows
    longest first (ties: lower index first), packed up to 4 to a group, a group
    closed early when the next row would raise its cost 9 ceil(u / 4) + 4 m (u
    union blocks, m longest row) above 5/4 (9/10 for head_dim 64) of the cost of
    the longest row alone, while the rows left still fit in the groups left."""
    cost = lambda u, m: 9 * ((u + 3) // 4) + 4 * m
    num, den = (9, 10) if head_dim == 64 else (5, 4)
    cap = cost(max_count, max_count) * num // den
    order = sorted(range(nq), key=lambda q: (-len(rows_h[q]), q))
    groups, cur, uni, tot, mx = [], [], set(), 0, 0
    for k, q in enumerate(order):
        c = len(rows_h[q])
        close = len(cur) == 4
        if (not close and cur and cost(tot + c, max(mx, c)) > cap
                and len(groups) + 1 + (nq - k + 3) // 4 <= gh):
            close = cost(len(uni | rows_h[q]), max(mx, c)) > cap
        if close:
            groups.append(cur)
            cur, uni, tot, mx = [], set(), 0, 0
        cur.append(q)
        uni |= rows_h[q]
        tot += c
        mx = max(mx, c)
    groups.append(cur)
    return groups


@pytest.mark.parametrize("bh,nq,eta,hd", [(3, 37, 0.9, 0), (2, 8, 0.5, 128), (1, 130, 0.95, 64), (2, 5, 1.0, 96),
                                          (1, 300, 0.99, 0), (2, 64, 0.9, 64), (11, 16, 0.9, 96)])
def test_execution_plan_lists_each_union_block_once(bh, nq, eta, hd):
    """The plan deals each head's query blocks to groups of at most 4, every block
    once, in order of scheduled block count (longest first, lower index first);
    each group lists exactly the union of its rows' key blocks, each once, with the
    membership bits of the oracle's supports; the sparse kernel gives the same rows
    through the plan as through the CSR."""
    wise = _wise()
    rng = np.random.default_rng(bh * 1000 + nq)
    m = np.zeros((4, bh, nq, nq), dtype=np.float32)
    for s in range(4):
        for r in range(bh):
            for qb in range(nq):
                m[s, r, qb, :qb + 1] = rng.dirichlet(np.full(qb + 1, 0.4))
    note(f"plan bh={bh} nq={nq} eta={eta} plan_head_dim={hd}")
    sched = wise.build_support(torch.from_numpy(m).to(DEV), eta, plan_head_dim=hd)
    torch.cuda.synchronize()
    assert sched.plan is not None
    plan = sched.plan.cpu().numpy()
    gpu_rows = csr_rows(sched.row_ptr, sched.col_idx)
    ref_rows, flags = [], []
    for r in range(bh):
        for qb in range(nq):
            sup, fl = oracle_union_row([m[s, r, qb, :qb + 1].astype(np.float64) for s in range(4)], eta)
            ref_rows.append(sup)
            flags.append(fl)
    bad, _ = compare_supports(gpu_rows, ref_rows, flags)
    assert not bad
    groups, gh = _decode_plan(plan, bh, nq)
    max_count = max(len(r) for r in gpu_rows)
    for h in range(bh):
        rows_h = [set(gpu_rows[h * nq + q].tolist()) for q in range(nq)]
        want_groups = _expected_groups(rows_h, nq, gh, max_count, hd)
        got_groups = [groups[h * gh + j][0] for j in range(gh) if groups[h * gh + j][0]]
        assert got_groups == want_groups, f"head {h}: groups {got_groups} != {want_groups}"
        dealt = [q for j in range(gh) for q in groups[h * gh + j][0]]
        assert sorted(dealt) == list(range(nq)), f"head {h}: rows dealt {dealt}"
        counts = [len(gpu_rows[h * nq + q]) for q in dealt]
        assert [(-c, q) for c, q in zip(counts, dealt)] == sorted((-c, q) for c, q in zip(counts, dealt)), \
            f"head {h}: rows not in count order"
        seen_empty = False
        for j in range(gh):
            if not groups[h * gh + j][0]:
                seen_empty = True
            else:
                assert not seen_empty, f"head {h}: a group after an empty one"
    for g, (rows_g, ents) in groups.items():
        h = g // gh
        blocks = [b for b, _ in ents]
        assert len(blocks) == len(set(blocks)), f"group {g} lists a block twice"
        want = {}
        for w_, q in enumerate(rows_g):
            for b in gpu_rows[h * nq + q].tolist():
                want[b] = want.get(b, 0) | (1 << w_)
        assert dict(ents) == want, f"group {g}"
        for w_, q in enumerate(rows_g):
            r = h * nq + q
            if set(gpu_rows[r].tolist()) == set(ref_rows[r].tolist()):
                assert {b for b, mm in ents if (mm >> w_) & 1} == set(ref_rows[r].tolist())
    # sparse attention through the plan vs through the CSR rows vs the oracle
    n, d = 32 * nq, 128
    q, k, v = (torch.from_numpy(rng.standard_normal((1, bh, n, d)).astype(np.float32)).to(torch.bfloat16)
               for _ in range(3))
    dq, dk, dv = q.to(DEV), k.to(DEV), v.to(DEV)
    op, lp = wise.sparse_attn(dq, dk, dv, sched, want_lse=True)
    csr_only = wise.Schedule(sched.row_ptr, sched.col_idx, sched.nnz, bh, nq)
    oc, lc = wise.sparse_attn(dq, dk, dv, csr_only, want_lse=True)
    torch.cuda.synchronize()
    assert_attn_close(f64(op), f64(oc), "bf16", "plan vs CSR O")
    assert float((lp - lc).abs().max()) <= 1e-5
    for h in range(bh):
        rows_h = ref_rows[h * nq:(h + 1) * nq]
        ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), rows_h)
        keep = np.zeros(n, dtype=bool)
        for qb in range(nq):
            if set(gpu_rows[h * nq + qb].tolist()) == set(rows_h[qb].tolist()):
                keep[32 * qb:32 * qb + 32] = True
        assert_attn_close(f64(op[0, h])[keep], ro[keep], "bf16", f"plan head {h} O")
        assert_lse_close(f64(lp[0, h])[keep], rl[keep], "bf16", f"plan head {h}")
