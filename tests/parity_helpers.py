"""Shared helpers of the GPU parity tests (tolerances, oracle-side schedules).

Tolerances (elementwise, allclose semantics |gpu - ref| <= atol + rtol*|ref|):
  attention output  bf16: atol 1e-2, rtol 2e-2      fp32: atol 1e-5, rtol 1e-5
  row log-sum-exp   bf16: atol 1e-3                 fp32: atol 1e-5
  block mass        bf16: atol 1e-5                 fp32: atol 1e-6
Block supports must match the oracle exactly except blocks the oracle flags as
within 1e-4 of the eta boundary (cumulative) or within 1e-6 of a mass on the
other side of the cut (ranking near-tie).
"""
import sys

import numpy as np
import torch

import oracle as O

TOL = {
    "bf16": dict(o_atol=1e-2, o_rtol=2e-2, lse_atol=1e-3, mass_atol=1e-5),
    "fp32": dict(o_atol=1e-5, o_rtol=1e-5, lse_atol=1e-5, mass_atol=1e-6),
}
CUM_TOL, TIE_TOL = 1e-4, 1e-6
# rows whose GPU support may differ from the oracle's in flagged blocks only:
# at most this fraction of the rows compared (and at least 2 rows)
FLAGGED_ROW_FRACTION = 0.01

# per-configuration parity figures, printed at the end of the pytest run
REPORT = []


def record(config, **fields):
    """Add one line to the parity report printed by the terminal-summary hook."""
    REPORT.append((config, fields))


def flagged_row_bound(rows):
    return max(2, int(np.ceil(FLAGGED_ROW_FRACTION * rows)))


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def step_pair(gen, step, device="cuda"):
    """(host, device) copies of one step's Q, K, V: the oracle reads the host
    tensors the generator produced, the HIP path reads their device copies."""
    host = gen.step_torch(step)
    return host, tuple(x.to(device) for x in host)


def assert_attn_close(gpu, ref, dtype, what):
    tol = TOL[dtype]
    err = np.abs(gpu - ref)
    bound = tol["o_atol"] + tol["o_rtol"] * np.abs(ref)
    bad = err > bound
    used = float((err / bound).max()) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance; max abs err "
                           f"{float(err.max()):.3e}, worst err/(atol+rtol|ref|) {used:.3f}")
    # (max abs error, largest fraction of the elementwise tolerance used)
    return float(err.max()), used


def assert_lse_close(gpu, ref, dtype, what):
    tol = TOL[dtype]["lse_atol"]
    both_inf = np.isneginf(gpu) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    assert np.all(err <= tol), f"{what}: lse max abs err {float(np.nanmax(err)):.3e} > {tol}"


def assert_mass_close(gpu, ref, dtype, what):
    tol = TOL[dtype]["mass_atol"]
    err = np.abs(gpu - ref)
    assert np.all(err <= tol), f"{what}: mass max abs err {float(err.max()):.3e} > {tol}"


def csr_rows(row_ptr, col_idx):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    return [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]


def oracle_union_row(masses_steps, eta, cum_tol=CUM_TOL, tie_tol=TIE_TOL):
    """Union support of one (head, query block) row over the given per-step mass
    rows (each the q+1 admissible masses), plus the blocks flagged in any step."""
    sup = set()
    flagged = set()
    for m in masses_steps:
        sup.update(int(b) for b in O.select_support(m, eta))
        fc, ft = O.boundary_flags(m, eta, cum_tol, tie_tol)
        flagged.update(int(b) for b in np.nonzero(fc | ft)[0])
    return np.array(sorted(sup), dtype=np.int64), flagged


def compare_supports(gpu_rows, oracle_rows, flags, flagged_rows=None):
    """Returns (unflagged mismatching rows, flagged mismatching blocks); the rows
    that differ in flagged blocks only are appended to flagged_rows if given."""
    bad_rows = []
    flagged_blocks = 0
    for r, (g, o) in enumerate(zip(gpu_rows, oracle_rows)):
        diff = set(g.tolist()) ^ set(o.tolist())
        if not diff:
            continue
        if diff <= flags[r]:
            flagged_blocks += len(diff)
            if flagged_rows is not None:
                flagged_rows.append(r)
        else:
            bad_rows.append((r, sorted(diff - flags[r])))
    return bad_rows, flagged_blocks


def schedule_from_rows(rows, device):
    """Upload a host-built schedule (list of index arrays per row) as int32 CSR."""
    from block_sparse_attention_wise_amd import wise
    rp, ci = O.build_csr(rows)
    nnz = int(rp[-1])
    row_ptr = torch.from_numpy(rp.astype(np.int32)).to(device)
    col_idx = torch.from_numpy(np.concatenate([ci, np.zeros(1)]).astype(np.int32)).to(device)
    return wise.Schedule(row_ptr, col_idx, torch.tensor([nnz], dtype=torch.int32, device=device), 0, 0)
