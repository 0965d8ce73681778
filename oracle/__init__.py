"""fp64 CPU oracle of the WISE working-set attention path.

Test infrastructure: only the tests, the smoke check of ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may use it; the HIP library never does.
"""
from .wise_oracle import (  # noqa: F401
    attention_probs, block_density, block_mass, boundary_flags, build_csr,
    causal_attention, expand_supports, mass_matched_support, retained_mass, scheduled_pairs,
    select_support, size_matched_support, sorted_order, sparse_attention,
    step_supports, union_supports,
)
