"""wise_build_support_static (no workspace, no allocation) against wise_build_support
on the same masses: the CSR schedule and the execution plan must match bit for bit,
on two calls in a row, the second with a smaller input (the static scratch keeps the
first call's contents)."""
import numpy as np
import pytest
import torch

from parity_helpers import note

DEV = "cuda"


def _masses(rng, steps, bh, nq):
    m = np.zeros((steps, bh, nq, nq), dtype=np.float32)
    for s in range(steps):
        for r in range(bh):
            for qb in range(nq):
                m[s, r, qb, :qb + 1] = rng.dirichlet(np.full(qb + 1, 0.4))
    return torch.from_numpy(m).to(DEV)


@pytest.mark.gpu
def test_static_scratch_builder_matches_workspace_builder():
    from block_sparse_attention_wise_amd import wise
    rng = np.random.default_rng(2024)
    for steps, bh, nq, eta, hd in ((4, 32, 128, 0.95, 128), (3, 3, 37, 0.9, 64)):
        note(f"static scratch builder steps={steps} bh={bh} nq={nq} eta={eta}")
        mass = _masses(rng, steps, bh, nq)
        ref = wise.build_support(mass, eta, plan_head_dim=hd)
        got = wise.build_support_static(mass, eta, plan_head_dim=hd)
        torch.cuda.synchronize()
        nnz = int(ref.nnz.item())
        assert int(got.nnz.item()) == nnz
        assert torch.equal(got.row_ptr, ref.row_ptr)
        assert torch.equal(got.col_idx[:nnz], ref.col_idx[:nnz])
        # the plan: entry counts, slot stride, group rows, and each group's first
        # n_g entries of its fixed slot (the rest of a slot is never written)
        gh = (nq + 3) // 4 + (nq + 15) // 16
        groups = bh * gh
        pg, pr = got.plan.cpu().numpy(), ref.plan.cpu().numpy()
        head = groups + 1 + 4 * groups
        assert np.array_equal(pg[:head], pr[:head])
        for g in range(groups):
            n = int(pr[g])
            at = head + g * nq
            assert np.array_equal(pg[at:at + n], pr[at:at + n]), f"group {g}"
