"""wise_build_support_static (no workspace, no allocation) against wise_build_support
on the same masses: the CSR schedule and the row order must match bit for bit,
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
    for steps, bh, nq, eta in ((4, 32, 128, 0.95), (3, 3, 37, 0.9)):
        note(f"static scratch builder steps={steps} bh={bh} nq={nq} eta={eta}")
        mass = _masses(rng, steps, bh, nq)
        ref = wise.build_support(mass, eta)
        got = wise.build_support_static(mass, eta)
        torch.cuda.synchronize()
        nnz = int(ref.nnz.item())
        assert int(got.nnz.item()) == nnz
        assert torch.equal(got.row_ptr, ref.row_ptr)
        assert torch.equal(got.col_idx[:nnz], ref.col_idx[:nnz])
        assert torch.equal(got.plan, ref.plan)
