"""GPU parity of schedules selected at block sizes 64 and 128 (the WISE paper,
App. B, block-size study), through the C ABI.

Fed masses: both sides start from the same fp32 32-token masses; the oracle
aggregates them in fp64 to the block size, rounds to fp32 as the schedule
builder stores them (both sides take the selection decision on the same fp32
values), selects, unions and expands to the 32-token grid; rows must match
exactly (flags only at 1e-12).  End to end: GPU masses and schedule against
the oracle's block-level masses and supports (usual flags), then the sparse
step against the oracle's attention at that block size.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_wise_amd.synthetic import WORKLOADS, Generator
from parity_helpers import assert_attn_close, assert_lse_close, csr_rows, f64, note, step_pair

pytestmark = pytest.mark.gpu
DEV = "cuda"
_GEN, _M = {}, {}


def _wise():
    from block_sparse_attention_wise_amd import wise
    return wise


def _gen(name):
    if name not in _GEN:
        _GEN[name] = Generator(WORKLOADS[name])
    return _GEN[name]


def _masses(name, block):
    key = (name, block)
    if key not in _M:
        w, g = WORKLOADS[name], _gen(name)
        out = []
        for t in (9, 10, 11, 12):
            q, k, _ = g.step_torch(t)
            out.append(np.stack([O.block_mass(f64(q[0, h]), f64(k[0, h // w.group]), block=block)
                                 for h in range(w.heads)]))
        _M[key] = np.stack(out)
    return _M[key]


@pytest.mark.parametrize("name", ["1k", "2k", "gqa"])
@pytest.mark.parametrize("block", [64, 128])
def test_blocked_schedule_on_fed_masses(name, block):
    wise, w = _wise(), WORKLOADS[name]
    eta = w.etas[0]
    f = block // 32
    m32 = _masses(name, 32).astype(np.float32)                  # [4][heads][nq][nq]
    nq, nb = w.nq, w.nq // f
    agg = (m32.astype(np.float64).reshape(4, w.heads, nb, f, nb, f).sum(axis=(3, 5)) / f).astype(np.float32)
    note(f"blocked fed {name} B={block}")
    sched = wise.build_support(torch.from_numpy(m32).to(DEV), eta, block=block)
    torch.cuda.synchronize()
    rows = csr_rows(sched.row_ptr, sched.col_idx)
    assert int(sched.nnz.item()) == int(sched.row_ptr[-1].item())
    for h in range(w.heads):
        sup_b, flags_b = [], []
        for qb in range(nb):
            per = [agg[s, h, qb, :qb + 1].astype(np.float64) for s in range(4)]
            sup_b.append(O.union_supports([[O.select_support(m, eta)] for m in per])[0])
            fl = set()
            for m in per:
                fc, _ = O.boundary_flags(m, eta, cum_tol=1e-12, tie_tol=0.0)
                fl |= set(int(b) for b in np.nonzero(fc)[0])
            flags_b.append(fl)
        want = O.expand_supports(sup_b, nq, block)
        for q in range(nq):
            diff = set(rows[h * nq + q].tolist()) ^ set(want[q].tolist())
            assert {k // f for k in diff} <= flags_b[q // f], f"{name} B={block} head {h} row {q}: {diff}"


@pytest.mark.parametrize("block", [64, 128])
def test_blocked_end_to_end(block):
    wise, w = _wise(), WORKLOADS["1k"]
    eta = w.etas[0]
    f = block // 32
    g = _gen("1k")
    mass = torch.empty((4, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    for si, t in enumerate((9, 10, 11, 12)):
        q, k, v = g.step_torch(t, DEV)
        wise.full_attn_mass(q, k, v, mass=mass[si])
    note(f"blocked e2e B={block}")
    sched = wise.build_support(mass, eta, block=block)
    torch.cuda.synchronize()
    rows = csr_rows(sched.row_ptr, sched.col_idx)
    mb = _masses("1k", block)
    nb = w.nq // f
    (qs, ks, vs), dev = step_pair(g, 20)
    o, lse = wise.sparse_attn(*dev, sched, want_lse=True)
    torch.cuda.synchronize()
    for h in range(w.heads):
        sup_b, flags_b = [], []
        for qb in range(nb):
            per = [mb[s, h, qb, :qb + 1] for s in range(4)]
            sup_b.append(O.union_supports([[O.select_support(m, eta)] for m in per])[0])
            fl = set()
            for m in per:
                fc, ft = O.boundary_flags(m, eta)
                fl |= set(int(b) for b in np.nonzero(fc | ft)[0])
            flags_b.append(fl)
        want = O.expand_supports(sup_b, w.nq, block)
        same = np.zeros(w.seqlen, dtype=bool)
        for q in range(w.nq):
            diff = set(rows[h * w.nq + q].tolist()) ^ set(want[q].tolist())
            assert {k // f for k in diff} <= flags_b[q // f], f"B={block} head {h} row {q}: {diff}"
            if not diff:
                same[32 * q:32 * q + 32] = True
        ro, rl = O.sparse_attention(f64(qs[0, h]), f64(ks[0, h]), f64(vs[0, h]), sup_b, block=block)
        assert_attn_close(f64(o[0, h])[same], ro[same], w.dtype, f"B={block} head {h} O")
        assert_lse_close(f64(lse[0, h])[same], rl[same], w.dtype, f"B={block} head {h}")
