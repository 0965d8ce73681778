"""Seeded synthetic recurrent-step Q/K/V inputs (the only code shared by the
HIP path's tests/benchmark and the CPU oracle).

This module draws random numbers and nothing else: it contains no attention,
block-mass, selection or schedule arithmetic.  Both sides read the arrays it
returns, after the cast to the compute dtype.

The WISE paper (Wan & Chen, arXiv 2609.27373) measures on saved working-set
workloads of a recurrent-depth model (App. B, "Systems evaluation"), which are
not available; these synthetic inputs stand in for them.  Recipe, per head h:

1. base  Q_b, K_b, V_b ~ N(0, 1), shape [n, d];
2. planted relevance: every query block q >= 1 gets R_q = min(R, q) distinct
   earlier key blocks drawn uniformly from 0..q-1; with m_q the mean of K_b over
   their M_q = 32 R_q keys, v_q is added to every query row of block q.
   ``planted="scaled"`` (default): v_q = g (M_q / sqrt(d)) m_q with g = 4, an
   expected logit boost of g on the relevant keys.  ``planted="literal"``:
   v_q = 0.8 m_q, the workload text taken word for word (boost ~0.8 sqrt(d)/M_q
   logits, which leaves attention nearly uniform);
3. sink (when enabled): a unit vector u_h, a = sqrt(2 sqrt(d)); Q += a u_h on all
   rows and K[0:32] += a u_h, an expected +2 logits on key block 0;
4. drift for recurrent step t = 1..T: X_t = X + (0.05 / t) N(0, 1), a fresh draw
   per (head, step, X) for X in {Q, K, V};
5. cast to the compute dtype (bf16 round-to-nearest-even via torch, or fp32).

Random streams: numpy PCG64 seeded with [cfg_seed, head, step, stream] where
stream is 0/1/2 for Q/K/V, 3 for the relevance draw, 4 for the sink direction;
the base tensors use step 0.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

BLOCK = 32
T_STEPS = 32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32" or "bf16"
    heads: int
    head_dim: int
    seqlen: int
    relevant: int       # R, planted relevant blocks per query block
    sink: bool
    etas: tuple         # eta values the workload is run at (first is the default)
    seed: int
    batch: int = 1

    @property
    def nq(self) -> int:
        return self.seqlen // BLOCK


WORKLOADS = {
    "tiny": Workload("tiny", "fp32", 1, 64, 256, 2, False, (0.95,), 0),
    "1k": Workload("1k", "bf16", 8, 128, 1024, 3, False, (0.95,), 1),
    "2k": Workload("2k", "bf16", 32, 128, 2048, 4, True, (0.95,), 2),
    "4k": Workload("4k", "bf16", 32, 128, 4096, 4, True, (0.95,), 3),
    "16k": Workload("16k", "bf16", 32, 128, 16384, 6, True, (0.90, 0.95, 0.99), 4),
}


def _rng(seed, head, step, stream):
    return np.random.default_rng([int(seed), int(head), int(step), int(stream)])


def base_head(w: Workload, head: int, planted: str = "scaled"):
    """Base (step-independent) Q, K, V of one head as float32 [n, d] arrays."""
    n, d = w.seqlen, w.head_dim
    q = _rng(w.seed, head, 0, 0).standard_normal((n, d), dtype=np.float32)
    k = _rng(w.seed, head, 0, 1).standard_normal((n, d), dtype=np.float32)
    v = _rng(w.seed, head, 0, 2).standard_normal((n, d), dtype=np.float32)
    rel = _rng(w.seed, head, 0, 3)
    nq = n // BLOCK
    for qb in range(1, nq):
        r = min(w.relevant, qb)
        chosen = rel.choice(qb, size=r, replace=False)
        keys = k.reshape(nq, BLOCK, d)[chosen].reshape(-1, d)
        mean = keys.mean(axis=0, dtype=np.float64)
        if planted == "scaled":
            add = 4.0 * (keys.shape[0] / np.sqrt(d)) * mean
        elif planted == "literal":
            add = 0.8 * mean
        else:
            raise ValueError(f"unknown planted mode {planted!r}")
        q[qb * BLOCK:(qb + 1) * BLOCK] += add.astype(np.float32)
    if w.sink:
        u = _rng(w.seed, head, 0, 4).standard_normal(d)
        u = (u / np.linalg.norm(u) * np.sqrt(2.0 * np.sqrt(d))).astype(np.float32)
        q += u
        k[:BLOCK] += u
    return q, k, v


def drift_head(w: Workload, head: int, step: int, base):
    """Q, K, V of one head at recurrent step ``step`` (1-based), float32."""
    if not 1 <= step <= T_STEPS:
        raise ValueError("recurrent steps are numbered 1..32")
    amp = np.float32(0.05 / step)
    out = []
    for stream, x in enumerate(base):
        noise = _rng(w.seed, head, step, stream).standard_normal(x.shape, dtype=np.float32)
        out.append(x + amp * noise)
    return tuple(out)


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


class Generator:
    """Caches the base tensors of a workload and produces per-step inputs.

    heads: optional subset of head indices (default all).
    """

    def __init__(self, w: Workload, heads=None, planted: str = "scaled"):
        self.w = w
        self.heads = list(range(w.heads)) if heads is None else list(heads)
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            self.base = list(ex.map(lambda h: base_head(w, h, planted), self.heads))

    def step_f32(self, step: int):
        """float32 arrays [len(heads), n, d] for Q, K, V at ``step``."""
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            per_head = list(ex.map(lambda i: drift_head(self.w, self.heads[i], step, self.base[i]),
                                   range(len(self.heads))))
        return tuple(np.stack([ph[j] for ph in per_head]) for j in range(3))

    def step_torch(self, step: int, device="cpu"):
        """Q, K, V at ``step`` as torch tensors [batch=1, heads, n, d] in the
        workload's dtype (bf16 cast is round-to-nearest-even)."""
        import torch
        dt = torch.bfloat16 if self.w.dtype == "bf16" else torch.float32
        out = []
        for x in self.step_f32(step):
            t = torch.from_numpy(x).unsqueeze(0).to(dt)
            out.append(t.to(device) if device != "cpu" else t)
        return tuple(out)


def as_f64(t):
    """Exact float64 copy of a (CPU or device) torch tensor's values."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
