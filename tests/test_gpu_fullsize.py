"""GPU parity at the full workload sizes (4k headline, 16k stress), in the launch
configuration bench.py times: every head runs on the GPU, and sampled heads and
query blocks are compared with the fp64 oracle computed one by one."""
import numpy as np
import pytest
import torch

import oracle as O
from block_sparse_attention_wise_amd.synthetic import WORKLOADS, Generator
from parity_helpers import (assert_attn_close, assert_lse_close, assert_mass_close, csr_rows, f64,
                            flagged_row_bound, note, oracle_union_row, record, step_pair)

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "4k": dict(heads=[0, 11, 22, 31], qblocks=None),                       # every query block of 4 heads
    "16k": dict(heads=[0, 31], qblocks=[0, 1, 2, 77, 255, 256, 400, 510, 511]),
    # the pages' geometries: Huginn (55 heads, d = 96), Recurrent-Llama (32 query / 8 kv heads, d = 64)
    "huginn4k": dict(heads=[0, 27, 54], qblocks=[0, 1, 5, 63, 64, 100, 126, 127]),
    # one Huginn step, 4 layers x 55 heads: a head of each layer
    "huginn4k_step": dict(heads=[0, 70, 150, 219], qblocks=[0, 1, 5, 63, 64, 100, 126, 127]),
    "llama4k": dict(heads=[0, 3, 4, 31], qblocks=[0, 1, 5, 63, 64, 100, 126, 127]),
}
FULL = ["4k", "16k", "huginn4k", "huginn4k_step", "llama4k"]


def _run_gpu(name):
    from block_sparse_attention_wise_amd import wise
    w = WORKLOADS[name]
    g = Generator(w)
    mass = torch.empty((4, w.heads, w.nq, w.nq), dtype=torch.float32, device=DEV)
    host = {}
    for si, t in enumerate((9, 10, 11, 12)):
        hq, dq = step_pair(g, t)
        note(f"{name} discovery step {t}")
        wise.full_attn_mass(*dq, mass=mass[si])
        host[t] = hq[:2]
        del dq
    return wise, w, g, mass, host


@pytest.mark.parametrize("name", FULL)
def test_fullsize_schedule_and_sparse_attention(name):
    wise, w, g, mass, host = _run_gpu(name)
    case = CASES[name]
    qbs = case["qblocks"] if case["qblocks"] is not None else list(range(w.nq))
    torch.cuda.synchronize()
    gm = mass.cpu().numpy()
    # oracle masses of the sampled rows, compared with the GPU's
    orc = {}
    for h in case["heads"]:
        for t in (9, 10, 11, 12):
            qh, kh = f64(host[t][0][0, h]), f64(host[t][1][0, h // w.group])
            for qb in qbs:
                r = O.block_mass(qh, kh, qblocks=(qb, qb + 1))[0]
                orc[(h, t, qb)] = r
                assert_mass_close(gm[t - 9, h, qb], r, w.dtype, f"{name} head {h} step {t} block {qb}")
    (q13, k13, v13), dev13 = step_pair(g, 13)
    for eta in w.etas:
        note(f"{name} build eta={eta}")
        sched = wise.build_support(mass, eta)
        note(f"{name} sparse eta={eta}")
        o, lse = wise.sparse_attn(*dev13, sched, want_lse=True)
        torch.cuda.synchronize()
        rows = csr_rows(sched.row_ptr, sched.col_idx)
        assert int(sched.nnz.item()) == int(sched.row_ptr[-1].item())
        flagged_total, flagged_rows, compared = 0, 0, 0
        worst_abs = worst_tol = 0.0
        for h in case["heads"]:
            qh, kh, vh = f64(q13[0, h]), f64(k13[0, h // w.group]), f64(v13[0, h // w.group])
            for qb in qbs:
                sup, flags = oracle_union_row([orc[(h, t, qb)][:qb + 1] for t in (9, 10, 11, 12)], eta)
                got = rows[h * w.nq + qb]
                diff = set(got.tolist()) ^ set(sup.tolist())
                assert diff <= flags, f"{name} eta {eta} head {h} block {qb}: unflagged mismatch {diff - flags}"
                flagged_total += len(diff)
                flagged_rows += int(bool(diff))
                compared += 1
                # every sampled row against the oracle over the GPU's own row (the
                # oracle's row itself unless a flagged block differs)
                sup_rows = [np.array([0])] * w.nq
                sup_rows[qb] = got
                ro, rl = O.sparse_attention(qh, kh, vh, sup_rows, qblocks=(qb, qb + 1))
                sl = slice(32 * qb, 32 * qb + 32)
                ea, er = assert_attn_close(f64(o[0, h, sl]), ro, w.dtype, f"{name} eta {eta} head {h} block {qb} O")
                assert_lse_close(f64(lse[0, h, sl]), rl, w.dtype, f"{name} eta {eta} head {h} block {qb}")
                worst_abs, worst_tol = max(worst_abs, ea), max(worst_tol, er)
        note(f"{name} eta={eta}: flagged mismatching rows {flagged_rows}, blocks {flagged_total}")
        assert flagged_rows <= flagged_row_bound(compared), f"{flagged_rows} flagged rows of {compared}"
        record(f"full size {name} (eta {eta}, step 13, heads {case['heads']})", rows=compared,
               flagged_rows=flagged_rows, flagged_blocks=flagged_total, max_abs=worst_abs, tol_used=worst_tol)


@pytest.mark.parametrize("name", FULL)
def test_fullsize_dense_rows(name):
    from block_sparse_attention_wise_amd import wise
    w = WORKLOADS[name]
    case = CASES[name]
    g = Generator(w)
    (q, k, v), dev = step_pair(g, 1)
    note(f"{name} dense step 1")
    o, lse = wise.dense_attn(*dev, want_lse=True)
    torch.cuda.synchronize()
    qbs = case["qblocks"] if case["qblocks"] is not None else [0, 1, w.nq // 2, w.nq - 1]
    worst_abs = worst_tol = 0.0
    for h in case["heads"]:
        qh, kh, vh = f64(q[0, h]), f64(k[0, h // w.group]), f64(v[0, h // w.group])
        for qb in qbs:
            ro, rl = O.causal_attention(qh, kh, vh, rows=(32 * qb, 32 * qb + 32))
            sl = slice(32 * qb, 32 * qb + 32)
            ea, er = assert_attn_close(f64(o[0, h, sl]), ro, w.dtype, f"{name} head {h} block {qb} O")
            assert_lse_close(f64(lse[0, h, sl]), rl, w.dtype, f"{name} head {h} block {qb}")
            worst_abs, worst_tol = max(worst_abs, ea), max(worst_tol, er)
    record(f"full size {name} dense (step 1, heads {case['heads']})", rows=len(case["heads"]) * len(qbs),
           max_abs=worst_abs, tol_used=worst_tol)


@pytest.mark.parametrize("name,block", [("4k", 32), ("4k", 16), ("huginn4k", 32)])
def test_fullsize_mass_epilogues_agree(name, block):
    """At the full size, the one-pass block masses (from stored block log-sum-exps)
    equal the second-sweep masses (logits recomputed once the row log-sum-exp is
    known) to fp32 rounding, over every (head, query block, key block)."""
    from block_sparse_attention_wise_amd import wise
    w = WORKLOADS[name]
    _, dq = step_pair(Generator(w), 10)
    note(f"{name} block {block} mass epilogues")
    _, _, m1 = wise.full_attn_mass(*dq, want_mass=True, block=block)
    _, _, m2 = wise.full_attn_mass(*dq, want_mass=True, block=block, workspace=False)
    torch.cuda.synchronize()
    d = (m1 - m2).abs()
    assert float(d.max()) <= 2e-5, f"max |one-pass - sweep| = {float(d.max()):.3e}"
    nb = m1.shape[-1]
    upper = torch.triu(torch.ones(nb, nb, dtype=torch.bool, device=m1.device), 1)
    assert bool((m1[:, upper] == 0).all())
    # every causal row sums to 1 (Eq. 5 over all key blocks is the row's total probability / B per query)
    rs = m1.sum(-1)
    assert float((rs - 1.0).abs().max()) <= 1e-4
