"""GPU parity of the intervention-control schedules and the retained-mass
diagnostic (the WISE paper, App. B: Static-95, SizeMatched, MassMatched,
retained future mass), through the C ABI.

Both sides read the same fp32 block masses (the oracle's step-1 masses rounded
to fp32) and the same reference working set (the oracle's union of steps
9..12), so the supports must agree exactly; the only tolerated differences are
blocks whose inclusion test lies within summation-order rounding of the
threshold (flagged at 1e-12 / 1e-10).  An end-to-end case builds the controls
from GPU masses and compares them with the oracle's under the usual flags.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_wise_amd.synthetic import WORKLOADS, Generator
from parity_helpers import (assert_attn_close, assert_lse_close, csr_rows, f64, note, oracle_union_row,
                            schedule_from_rows, step_pair)

pytestmark = pytest.mark.gpu
DEV = "cuda"
_GEN, _MASS = {}, {}


def _wise():
    from block_sparse_attention_wise_amd import wise
    return wise


def _gen(name):
    if name not in _GEN:
        _GEN[name] = Generator(WORKLOADS[name])
    return _GEN[name]


def _masses(name, step):
    """Oracle block masses of every head at one step (float64)."""
    key = (name, step)
    if key not in _MASS:
        w = WORKLOADS[name]
        q, k, _ = _gen(name).step_torch(step)
        _MASS[key] = np.stack([O.block_mass(f64(q[0, h]), f64(k[0, h])) for h in range(w.heads)])
    return _MASS[key]


def _reference_rows(name, eta):
    w = WORKLOADS[name]
    rows = []
    for h in range(w.heads):
        per = [O.step_supports(_masses(name, t)[h], eta) for t in (9, 10, 11, 12)]
        rows += O.union_supports(per)
    return rows


def _flags(masses, thr, tol):
    fc, _ = O.boundary_flags(masses, thr, cum_tol=tol, tie_tol=0.0)
    return set(int(b) for b in np.nonzero(fc)[0])


@pytest.mark.parametrize("name", ["tiny", "1k", "2k"])
def test_controls_on_fed_masses(name):
    wise, w = _wise(), WORKLOADS[name]
    eta = w.etas[0]
    m1 = _masses(name, 1).astype(np.float32)                 # [heads][nq][nq]
    ref_rows = _reference_rows(name, eta)
    ref = schedule_from_rows(ref_rows, DEV)
    dm = torch.from_numpy(np.ascontiguousarray(m1)).to(DEV)
    note(f"controls fed {name}")
    got = {kind: csr_rows(*(lambda s: (s.row_ptr, s.col_idx))(wise.build_support_variant(kind, dm, eta=eta,
                                                                                         reference=ref)))
           for kind in ("static", "size_matched", "mass_matched")}
    torch.cuda.synchronize()
    flagged = 0
    for h in range(w.heads):
        for qb in range(w.nq):
            r = h * w.nq + qb
            row = m1[h, qb, :qb + 1].astype(np.float64)
            want = O.select_support(row, eta)
            diff = set(got["static"][r].tolist()) ^ set(want.tolist())
            assert diff <= _flags(row, eta, 1e-12), f"static {name} row {r}: {diff}"
            want = O.size_matched_support(row, len(ref_rows[r]))
            np.testing.assert_array_equal(got["size_matched"][r], want, err_msg=f"size_matched {name} row {r}")
            want = O.mass_matched_support(row, ref_rows[r])
            mref = sum(row[b] for b in O.sorted_order(row) if b in set(ref_rows[r].tolist()))
            diff = set(got["mass_matched"][r].tolist()) ^ set(want.tolist())
            assert diff <= _flags(row, mref - O.wise_oracle.MASS_MATCH_SLACK, 1e-10), \
                f"mass_matched {name} row {r}: {diff}"
            flagged += len(diff)
    note(f"controls {name}: flagged differences {flagged}")


def test_controls_edge_cases():
    """Prefix references are reproduced exactly by MassMatched; empty and
    duplicated reference rows; SizeMatched on exact ties."""
    wise = _wise()
    rng = np.random.default_rng(9)
    bh, nq = 2, 24
    m = np.zeros((bh, nq, nq), dtype=np.float32)
    for r in range(bh):
        for qb in range(nq):
            raw = rng.integers(1, 4, size=qb + 1).astype(np.float64)
            m[r, qb, :qb + 1] = raw / 2 ** np.ceil(np.log2(raw.sum()))     # dyadic masses, many ties
    rows = []
    for r in range(bh):
        for qb in range(nq):
            row = m[r, qb, :qb + 1].astype(np.float64)
            k = qb % 5
            pref = O.sorted_order(row)[:k]                   # a sorted prefix (empty for k = 0)
            rows.append(np.concatenate([pref, pref]).astype(np.int64))   # listed twice
    ref = schedule_from_rows(rows, DEV)
    dm = torch.from_numpy(m).to(DEV)
    note("controls edge cases")
    sm = csr_rows(*(lambda s: (s.row_ptr, s.col_idx))(wise.build_support_variant("size_matched", dm, reference=ref)))
    mm = csr_rows(*(lambda s: (s.row_ptr, s.col_idx))(wise.build_support_variant("mass_matched", dm, reference=ref)))
    for r in range(bh):
        for qb in range(nq):
            i = r * nq + qb
            row = m[r, qb, :qb + 1].astype(np.float64)
            k = len(set(rows[i].tolist()))
            np.testing.assert_array_equal(sm[i], O.size_matched_support(row, k))
            np.testing.assert_array_equal(mm[i], O.mass_matched_support(row, rows[i]))
            if k:
                np.testing.assert_array_equal(mm[i], np.sort(np.unique(rows[i])))


@pytest.mark.parametrize("name", ["1k", "2k"])
def test_retained_mass_on_fed_masses(name):
    wise, w = _wise(), WORKLOADS[name]
    eta = w.etas[0]
    ref_rows = _reference_rows(name, eta)
    ref = schedule_from_rows(ref_rows, DEV)
    for t in (13, 32):
        mt = _masses(name, t).astype(np.float32)
        note(f"retained mass {name} step {t}")
        got = wise.retained_mass(torch.from_numpy(np.ascontiguousarray(mt)).to(DEV), ref).cpu().numpy()
        want = np.array([O.retained_mass(mt[h, qb, :qb + 1], ref_rows[h * w.nq + qb])
                         for h in range(w.heads) for qb in range(w.nq)])
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)
        note(f"{name} step {t}: mean retained future mass {want.mean():.4f}, min {want.min():.4f}")


def test_end_to_end_controls_from_gpu_masses():
    """1k: step-1 and steps 9..12 masses from the GPU, controls built on the GPU,
    compared with the oracle's controls from oracle masses (flags as in the
    schedule tests), then a sparse step over the SizeMatched schedule."""
    wise, w = _wise(), WORKLOADS["1k"]
    eta = w.etas[0]
    g = _gen("1k")
    mass = torch.empty((5, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((1, 9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        wise.full_attn_mass(q, k, v, mass=mass[si])
    note("e2e controls 1k")
    sched = wise.build_support(mass[1:].contiguous(), eta)
    size = wise.build_support_variant("size_matched", mass[0].contiguous(), reference=sched)
    torch.cuda.synchronize()
    wise_rows = csr_rows(sched.row_ptr, sched.col_idx)
    size_rows = csr_rows(size.row_ptr, size.col_idx)
    m1 = _masses("1k", 1)
    for h in range(w.heads):
        for qb in range(w.nq):
            r = h * w.nq + qb
            row = m1[h, qb, :qb + 1]
            sup_ref, fl_ref = oracle_union_row([_masses("1k", t)[h, qb, :qb + 1] for t in (9, 10, 11, 12)], eta)
            if set(wise_rows[r].tolist()) ^ set(sup_ref.tolist()):
                continue                                     # flagged working-set difference: skip the row
            want = O.size_matched_support(row, len(sup_ref))
            if not np.array_equal(size_rows[r], want):
                _, ft = O.boundary_flags(row, 1.0, cum_tol=0.0, tie_tol=1e-6)
                assert set(size_rows[r].tolist()) ^ set(want.tolist()) <= set(np.nonzero(ft)[0].tolist())
    (q, k, v), dev = step_pair(g, 20)
    o, lse = wise.sparse_attn(*dev, size, want_lse=True)
    torch.cuda.synchronize()
    for h in range(w.heads):
        rows = size_rows[h * w.nq:(h + 1) * w.nq]
        ro, rl = O.sparse_attention(f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), rows)
        assert_attn_close(f64(o[0, h]), ro, w.dtype, f"size-matched head {h} O")
        assert_lse_close(f64(lse[0, h]), rl, w.dtype, f"size-matched head {h}")
