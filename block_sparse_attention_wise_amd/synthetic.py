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

Grouped-query workloads (kv_heads < heads, the Recurrent-Llama geometry of the
WISE paper, App. B) draw K, V and the sink direction per key-value head g (head
index g in the seeds) and Q and the relevance draw per query head h; query head
h reads key-value head h // (heads / kv_heads), and its planted relevance is the
mean of that head's keys.  With kv_heads = heads this is the recipe above.
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
    kv_heads: int = 0   # 0: one key-value head per query head

    @property
    def nq(self) -> int:
        return self.seqlen // BLOCK

    @property
    def kvh(self) -> int:
        return self.kv_heads or self.heads

    @property
    def group(self) -> int:
        return self.heads // self.kvh


WORKLOADS = {
    "tiny": Workload("tiny", "fp32", 1, 64, 256, 2, False, (0.95,), 0),
    "1k": Workload("1k", "bf16", 8, 128, 1024, 3, False, (0.95,), 1),
    "2k": Workload("2k", "bf16", 32, 128, 2048, 4, True, (0.95,), 2),
    "4k": Workload("4k", "bf16", 32, 128, 4096, 4, True, (0.95,), 3),
    "16k": Workload("16k", "bf16", 32, 128, 16384, 6, True, (0.90, 0.95, 0.99), 4),
    # the pages' geometries (App. B): Huginn, d = 96 with 55 heads per recurrent
    # layer and 4 recurrent layers per step; Recurrent-Llama, grouped-query
    # attention with 32 query / 8 key-value heads of d = 64; plus small cases of
    # each for full parity
    "d96": Workload("d96", "bf16", 5, 96, 1024, 3, True, (0.95,), 5),
    "gqa": Workload("gqa", "bf16", 8, 64, 1024, 3, True, (0.95,), 6, kv_heads=2),
    "huginn4k": Workload("huginn4k", "bf16", 55, 96, 4096, 4, True, (0.95,), 7),
    # one Huginn recurrent step: its 4 recurrent attention layers of 55 heads in
    # one call (independent heads, each with its own K and V)
    "huginn4k_step": Workload("huginn4k_step", "bf16", 220, 96, 4096, 4, True, (0.95,), 9),
    "llama4k": Workload("llama4k", "bf16", 32, 64, 4096, 4, True, (0.95,), 8, kv_heads=8),
}


def _rng(seed, head, step, stream):
    return np.random.default_rng([int(seed), int(head), int(step), int(stream)])


def base_kv(w: Workload, g: int):
    """Base K, V of key-value head g as float32 [n, d] arrays, before the sink."""
    n, d = w.seqlen, w.head_dim
    k = _rng(w.seed, g, 0, 1).standard_normal((n, d), dtype=np.float32)
    v = _rng(w.seed, g, 0, 2).standard_normal((n, d), dtype=np.float32)
    return k, v


def sink_vector(w: Workload, g: int):
    d = w.head_dim
    u = _rng(w.seed, g, 0, 4).standard_normal(d)
    return (u / np.linalg.norm(u) * np.sqrt(2.0 * np.sqrt(d))).astype(np.float32)


def base_q(w: Workload, head: int, k, planted: str = "scaled"):
    """Base Q of query head ``head`` given its key-value head's base keys k."""
    n, d = w.seqlen, w.head_dim
    q = _rng(w.seed, head, 0, 0).standard_normal((n, d), dtype=np.float32)
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
        q += sink_vector(w, head // w.group)
    return q


def base_head(w: Workload, head: int, planted: str = "scaled"):
    """Base (step-independent) Q, K, V of one query head (K, V of its key-value
    head) as float32 [n, d] arrays."""
    g = head // w.group
    k, v = base_kv(w, g)
    q = base_q(w, head, k, planted)
    if w.sink:
        k[:BLOCK] += sink_vector(w, g)
    return q, k, v


def drift(w: Workload, head: int, step: int, stream: int, x):
    """x at recurrent step ``step`` (1-based): x + (0.05 / step) N(0, 1)."""
    if not 1 <= step <= T_STEPS:
        raise ValueError("recurrent steps are numbered 1..32")
    noise = _rng(w.seed, head, step, stream).standard_normal(x.shape, dtype=np.float32)
    return x + np.float32(0.05 / step) * noise


def drift_head(w: Workload, head: int, step: int, base):
    """Q, K, V of one head at recurrent step ``step`` (1-based), float32 (K, V
    drawn with the key-value head's seeds)."""
    g = head // w.group
    return (drift(w, head, step, 0, base[0]), drift(w, g, step, 1, base[1]), drift(w, g, step, 2, base[2]))


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


class Generator:
    """Caches the base tensors of a workload and produces per-step inputs.

    heads: optional subset of query-head indices (default all).  Q has one slice
    per listed head; K and V have one slice per key-value head those heads read,
    in order of first use (all key-value heads when ``heads`` is None), so with
    one key-value head per query head the three tensors line up head by head.
    """

    def __init__(self, w: Workload, heads=None, planted: str = "scaled"):
        self.w = w
        self.heads = list(range(w.heads)) if heads is None else list(heads)
        self.kv = []
        for h in self.heads:
            if h // w.group not in self.kv:
                self.kv.append(h // w.group)
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            kv = dict(zip(self.kv, ex.map(lambda g: base_kv(w, g), self.kv)))
            self.base_q = list(ex.map(lambda h: base_q(w, h, kv[h // w.group][0], planted), self.heads))
        self.base_kv = []
        for g in self.kv:
            k, v = kv[g]
            if w.sink:
                k = k.copy()
                k[:BLOCK] += sink_vector(w, g)
            self.base_kv.append((k, v))

    def step_f32(self, step: int):
        """float32 arrays Q [len(heads), n, d], K and V [len(kv heads), n, d] at ``step``."""
        w = self.w
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            q = list(ex.map(lambda i: drift(w, self.heads[i], step, 0, self.base_q[i]), range(len(self.heads))))
            kv = list(ex.map(lambda j: (drift(w, self.kv[j], step, 1, self.base_kv[j][0]),
                                        drift(w, self.kv[j], step, 2, self.base_kv[j][1])), range(len(self.kv))))
        return np.stack(q), np.stack([x[0] for x in kv]), np.stack([x[1] for x in kv])

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
