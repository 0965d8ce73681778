"""Benchmark of the WISE working-set attention path on one MI355X.

One bench "step" is one full T = 32 recurrent-step attention trajectory of the
WISE method on the synthetic workload (default: 4k -- bf16, batch 1, 32 heads,
head_dim 128, n = 4096, block 32, eta = 0.95):
  steps 1..8    dense causal attention                      (wise_dense_attn)
  steps 9..12   dense attention + block-mass epilogue        (wise_full_attn_mass)
  once          selection + temporal union + CSR             (wise_build_support)
  steps 13..32  block-sparse attention over the schedule     (wise_sparse_attn)
The in-run baseline -- 32 dense steps on the same inputs -- is timed in the same
passes, alternating which of the two runs first.  Every step reads its own
pre-generated Q/K/V, resident in HBM before timing starts.

Printed JSON line: value = late-step sparse effective TFLOP/s (4*d FLOP per
scheduled admissible (query, key) pair, kernel-only), ms_per_step = WISE 32-step
attention ms, plus setup-inclusive / kernel-only late-step speedups over the
in-house dense kernel, the dense trajectory, the roofline of the sparse kernel
and the fp64 CPU oracle timed on a bounded sample (the cpu_baseline leg).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

METRIC = "late-step sparse attn TFLOP/s + speedup vs dense at 4K; 32-step attn ms"
PEAK_HBM_GBS = 8000.0
# dense bf16 MFMA work per compute unit and clock on CDNA4: four SIMDs, each
# retiring a v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 = 32768 FLOP) every 32 cycles
BF16_FLOP_PER_CLK_PER_CU = 4 * 32768 // 32
HIP_DEVICE_ATTRIBUTE_CLOCK_RATE = 5   # hipDeviceAttributeClockRate (kHz), hip_runtime_api.h


def device_peak_bf16_tflops(device_index=0):
    """Dense bf16 MFMA peak of the device in the run: compute units x 4096 FLOP
    per clock x the peak engine clock (hipDeviceAttributeClockRate)."""
    import ctypes
    import torch
    cus = torch.cuda.get_device_properties(device_index).multi_processor_count
    khz = ctypes.c_int(0)
    hip = ctypes.CDLL("libamdhip64.so")
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), HIP_DEVICE_ATTRIBUTE_CLOCK_RATE, device_index) != 0:
        raise RuntimeError("hipDeviceGetAttribute(hipDeviceAttributeClockRate) failed")
    tflops = cus * BF16_FLOP_PER_CLK_PER_CU * khz.value * 1e3 / 1e12
    return tflops, {"compute_units": cus, "clock_mhz": khz.value / 1e3, "flop_per_clk_per_cu": BF16_FLOP_PER_CLK_PER_CU}
DISCOVERY_DENSE = range(1, 9)
DISCOVERY_MASS = range(9, 13)
REUSE = range(13, 33)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(_ROOT, "profiles", "hbm_traffic_attn_sparse_4k.txt")
KERNEL_SOURCES = ("attn_bf16.hip", "common.h", "kernels.h")


def kernel_source_digest():
    """sha256 over the sparse kernel's sources, to tell whether the committed HBM
    counter figures still describe the kernel being timed."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(_ROOT, "block_sparse_attention_wise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """Counter figures per sparse launch from the committed rocprofv3 summary
    (FETCH_SIZE / WRITE_SIZE bytes, L2 hits and misses), or None if it is
    missing, for another workload, or was taken on a different kernel source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if "=" in line and not line.startswith("#"):
                    key, val = line.strip().split("=", 1)
                    kv[key] = val
        if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_digest():
            return None
        out = {"hbm_bytes": float(kv["hbm_bytes_per_launch"])}
        for key in ("hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch", "l2_hit_rate"):
            if key in kv:
                out[key] = float(kv[key])
        return out
    except (OSError, KeyError, ValueError):
        return None


def pairs_from_csr(row_ptr, col_idx, nq):
    """Scheduled admissible (query, key) pairs of a CSR schedule (host arrays)."""
    total = 0
    for r in range(len(row_ptr) - 1):
        qb = r % nq
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        off = int(np.count_nonzero((cols >= 0) & (cols < qb)))
        diag = int(np.count_nonzero(cols == qb))
        total += off * 32 * 32 + diag * 32 * 33 // 2
    return total


def cpu_baseline(w, eta, gen_f32, budget_s=20.0, gpu_rows=None, gpu_o13=None):
    """The fp64 oracle on a bounded sample: heads 0.. of the same workload, timed
    per stage; the late-step rate is scheduled-pair FLOP / oracle sparse time.

    With gpu_rows (the GPU schedule's rows, head-major) and gpu_o13 (the GPU's
    step-13 output, [heads, n, d] on the host), the same heads also give a parity
    sample, outside the timed stages: the GPU supports against the oracle's
    (mismatches outside blocks within 1e-4 of the eta boundary, or within 1e-6 of
    a mass across the cut, must be 0; the rows and blocks differing in such
    flagged blocks are counted), and the GPU output against the oracle's sparse
    attention over the GPU's own rows (max abs error, and the largest fraction
    of the bf16 tolerance used)."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    heads_done = 0
    t_sparse = t_dense = t_mass = t_sel = 0.0
    flops = 0
    par = {"rows": 0, "unflagged_mismatch_rows": 0, "flagged_rows": 0, "flagged_blocks": 0,
           "max_abs_err": 0.0, "tol_used": 0.0}
    start = time.perf_counter()
    for h in range(w.heads):
        qkv = {t: gen_f32(t, h) for t in (1, 9, 10, 11, 12, 13)}
        t0 = time.perf_counter()
        O.causal_attention(*qkv[1])
        t1 = time.perf_counter()
        masses = [O.block_mass(qkv[t][0], qkv[t][1]) for t in (9, 10, 11, 12)]
        t2 = time.perf_counter()
        sup = O.union_supports([O.step_supports(m, eta) for m in masses])
        t3 = time.perf_counter()
        O.sparse_attention(*qkv[13], sup)
        t4 = time.perf_counter()
        t_dense += t1 - t0
        t_mass += (t2 - t1) / 4 + (t1 - t0)   # mass step = attention + block mass
        t_sel += t3 - t2
        t_sparse += t4 - t3
        flops += 4 * w.head_dim * O.scheduled_pairs(sup, w.nq)
        heads_done += 1
        if gpu_rows is not None:
            rows_h = gpu_rows[h * w.nq:(h + 1) * w.nq]
            for qb in range(w.nq):
                flagged = set()
                for m in masses:
                    fc, ft = O.boundary_flags(m[qb, :qb + 1], eta, 1e-4, 1e-6)
                    flagged.update(int(b) for b in np.nonzero(fc | ft)[0])
                diff = set(int(b) for b in rows_h[qb]) ^ set(int(b) for b in sup[qb])
                par["rows"] += 1
                if diff and diff <= flagged:
                    par["flagged_rows"] += 1
                    par["flagged_blocks"] += len(diff)
                elif diff:
                    par["unflagged_mismatch_rows"] += 1
            ro, _ = O.sparse_attention(*qkv[13], rows_h)
            err = np.abs(gpu_o13[h] - ro)
            par["max_abs_err"] = max(par["max_abs_err"], float(err.max()))
            # largest fraction of the bf16 tolerance 1e-2 + 2e-2 |ref| used
            par["tol_used"] = max(par["tol_used"], float((err / (1e-2 + 2e-2 * np.abs(ro))).max()))
        if time.perf_counter() - start > budget_s:
            break
    scale = w.heads / heads_done
    traj_s = scale * (8 * t_dense + 4 * t_mass + t_sel + 20 * t_sparse)
    return {
        "value": flops / t_sparse / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on heads 0..{heads_done - 1} of {w.heads} of the {w.name} workload: "
                   f"one dense step, four block-mass steps, selection+union, one sparse step (step 13); "
                   f"value = late-step scheduled-pair FLOP / oracle sparse time"),
        "sparse_step_ms_extrapolated": 1e3 * scale * t_sparse,
        "trajectory_ms_extrapolated": 1e3 * traj_s,
    }, (dict(par, heads=list(range(heads_done)), step=13) if gpu_rows is not None else None)


def support_diagnostics(wise, w, eta, steps, mass, sched, ws, stream):
    """Untimed-trajectory extras (the WISE paper, App. B): retained future mass of
    the WISE schedule at late steps; the intervention-control schedules
    (Static-95, SizeMatched, MassMatched from step-1 masses) and the schedules
    selected at block sizes 16, 64 and 128 (Table 8): density, retained future
    mass, build time and sparse-step time on each."""
    import torch
    bh, nq = w.batch * w.heads, w.nq
    out = torch.empty_like(steps[1][0])
    late = torch.empty((bh, nq, nq), dtype=torch.float32, device=mass.device)
    m1 = torch.empty_like(late)
    wise.full_attn_mass(*steps[1], out=out, mass=m1)
    causal = bh * nq * (nq + 1) // 2

    def timed(fn, reps=5):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    def retained(s, t):
        wise.full_attn_mass(*steps[t], out=out, mass=late)
        r = wise.retained_mass(late, s).cpu().numpy()
        return {"mean": round(float(r.mean()), 5), "min": round(float(r.min()), 5)}

    res = {"wise": {"block_density": round(int(sched.nnz.item()) / causal, 5),
                    "retained_future_mass": {f"t{t}": retained(sched, t) for t in (13, 20, 32)}}}
    for kind in ("static", "size_matched", "mass_matched"):
        ctl = wise.alloc_schedule(bh, nq, mass.device)
        build = lambda: wise.build_support_variant(kind, m1, eta=eta, reference=sched, schedule=ctl, workspace=ws)
        build_ms = timed(build)
        sparse_ms = timed(lambda: wise.sparse_attn(*steps[32], ctl, out=out))
        res[{"static": "static95"}.get(kind, kind)] = {
            "block_density": round(int(ctl.nnz.item()) / causal, 5),
            "retained_future_mass": {"t32": retained(ctl, 32)},
            "build_ms": round(build_ms, 4), "sparse_step_ms": round(sparse_ms, 4)}
    if nq % 4 == 0:
        for block in (64, 128):
            blk = wise.alloc_schedule(bh, nq, mass.device)
            wsb = torch.empty(int(wise.lib.wise_build_support_blocked_workspace_bytes(bh, nq, 4, block)),
                              dtype=torch.uint8, device=mass.device)
            build_ms = timed(lambda: wise.build_support(mass, eta, schedule=blk, workspace=wsb, block=block))
            sparse_ms = timed(lambda: wise.sparse_attn(*steps[32], blk, out=out))
            res[f"block{block}"] = {
                "block_density": round(int(blk.nnz.item()) / causal, 5),
                "retained_future_mass": {"t32": retained(blk, 32)},
                "build_ms": round(build_ms, 4), "sparse_step_ms": round(sparse_ms, 4)}
    if 2 * nq <= 2048:
        # B = 16: 16-token masses from the discovery kernel, the plain builder on
        # them, the sparse step over the 16-token CSR; density is reported over the
        # 16-token causal block pairs, retained mass against 16-token future masses
        n16 = 2 * nq
        m16 = torch.empty((4, bh, n16, n16), dtype=torch.float32, device=mass.device)
        disc_ms = timed(lambda: [wise.full_attn_mass(*steps[t], out=out, mass=m16[i], block=16)
                                 for i, t in enumerate((9, 10, 11, 12))])
        blk = wise.alloc_schedule(bh, n16, mass.device, with_plan=False)
        ws16 = torch.empty(int(wise.build_support_workspace_bytes(bh, n16, 4)), dtype=torch.uint8,
                           device=mass.device)
        build_ms = timed(lambda: wise.build_support(m16, eta, schedule=blk, workspace=ws16, with_plan=False))
        sparse_ms = timed(lambda: wise.sparse_attn(*steps[32], blk, out=out, block=16))
        late16 = torch.empty((bh, n16, n16), dtype=torch.float32, device=mass.device)
        wise.full_attn_mass(*steps[32], out=out, mass=late16, block=16)
        r = wise.retained_mass(late16, blk).cpu().numpy()
        res["block16"] = {
            "block_density": round(int(blk.nnz.item()) / (bh * n16 * (n16 + 1) // 2), 5),
            "retained_future_mass": {"t32": {"mean": round(float(r.mean()), 5), "min": round(float(r.min()), 5)}},
            "discovery_mass_ms_4_steps": round(disc_ms, 4),
            "build_ms": round(build_ms, 4), "sparse_step_ms": round(sparse_ms, 4)}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed trajectories (balanced passes; ~8 ms each at 4k, so ~1.7 s of timed GPU work)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="4k")
    ap.add_argument("--eta", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-matched", action="store_true",
                    help="skip the full-support sparse runs (profiling: keeps one sparse launch kind)")
    ap.add_argument("--no-diagnostics", action="store_true",
                    help="skip the retained-mass and intervention-control diagnostics")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from block_sparse_attention_wise_amd import wise
    from block_sparse_attention_wise_amd.synthetic import WORKLOADS, Generator

    w = WORKLOADS[args.workload]
    eta = args.eta if args.eta is not None else w.etas[0]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    log(f"[bench] generating {w.name} inputs for 32 steps")
    t0 = time.time()
    gen = Generator(w)
    steps = {}
    for t in range(1, 33):
        steps[t] = tuple(x.to(dev) for x in gen.step_torch(t))
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.time() - t0:.1f}s)")

    bh, nq = w.batch * w.heads, w.nq
    out = torch.empty_like(steps[1][0])
    mass = torch.empty((4, bh, nq, nq), dtype=torch.float32, device=dev)
    sched = wise.alloc_schedule(bh, nq, dev)
    ws = torch.empty(wise.build_support_workspace_bytes(bh, nq, 4), dtype=torch.uint8, device=dev)
    full_sched = wise.alloc_schedule(bh, nq, dev)
    wise.build_support(torch.ones((1, bh, nq, nq), dtype=torch.float32, device=dev), 1.0,
                       schedule=full_sched, workspace=ws)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def wise_traj():
        e = [ev() for _ in range(5)]
        e[0].record(stream)
        for t in DISCOVERY_DENSE:
            wise.dense_attn(*steps[t], out=out)
        e[1].record(stream)
        for si, t in enumerate(DISCOVERY_MASS):
            wise.full_attn_mass(*steps[t], out=out, mass=mass[si])
        e[2].record(stream)
        wise.build_support(mass, eta, schedule=sched, workspace=ws)
        e[3].record(stream)
        for t in REUSE:
            wise.sparse_attn(*steps[t], sched, out=out)
        e[4].record(stream)
        return e

    def dense_traj():
        e = [ev() for _ in range(3)]
        e[0].record(stream)
        for t in range(1, 13):
            wise.dense_attn(*steps[t], out=out)
        e[1].record(stream)
        for t in REUSE:
            wise.dense_attn(*steps[t], out=out)
        e[2].record(stream)
        return e

    def matched_full():
        e = [ev() for _ in range(2)]
        e[0].record(stream)
        for t in REUSE:
            wise.sparse_attn(*steps[t], full_sched, out=out)
        e[1].record(stream)
        return e

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)   # reads and writes exactly n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        wise_traj()
        dense_traj()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} balanced passes")
    recs = []
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for p in range(args.steps):
        if p % 2 == 0:
            a = wise_traj()
            b = dense_traj()
        else:
            b = dense_traj()
            a = wise_traj()
        recs.append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    m_rec = [] if args.no_matched else [matched_full() for _ in range(max(3, args.steps // 2))]
    torch.cuda.synchronize()
    diagnostics = None if args.no_diagnostics else support_diagnostics(wise, w, eta, steps, mass, sched, ws, stream)

    def ms(e0, e1):
        return e0.elapsed_time(e1)

    ph = {k: [] for k in ("disc_dense", "disc_mass", "build", "reuse", "wise_traj", "dense_early", "dense_late",
                          "dense_traj")}
    for a, b in recs:
        ph["disc_dense"].append(ms(a[0], a[1]))
        ph["disc_mass"].append(ms(a[1], a[2]))
        ph["build"].append(ms(a[2], a[3]))
        ph["reuse"].append(ms(a[3], a[4]))
        ph["wise_traj"].append(ms(a[0], a[4]))
        ph["dense_early"].append(ms(b[0], b[1]))
        ph["dense_late"].append(ms(b[1], b[2]))
        ph["dense_traj"].append(ms(b[0], b[2]))
    med = {k: statistics.median(v) for k, v in ph.items()}
    iqr = {k: float(np.percentile(v, 75) - np.percentile(v, 25)) for k, v in ph.items()}
    matched_ms = statistics.median(ms(e[0], e[1]) for e in m_rec) if m_rec else float("nan")

    rp = sched.row_ptr.cpu().numpy().astype(np.int64)
    ci = sched.col_idx.cpu().numpy().astype(np.int64)
    pairs = pairs_from_csr(rp, ci, nq)
    nnz = int(rp[-1])
    causal_blocks = bh * nq * (nq + 1) // 2
    sparse_flop = 4.0 * w.head_dim * pairs                 # per sparse launch
    dense_pairs = bh * (w.seqlen * (w.seqlen + 1) // 2)
    dense_flop = 4.0 * w.head_dim * dense_pairs
    sparse_ms = med["reuse"] / len(REUSE)                  # average launch duration
    dense_ms = med["dense_late"] / len(REUSE)
    tflops = sparse_flop / (sparse_ms * 1e-3) / 1e12
    dense_tflops = dense_flop / (dense_ms * 1e-3) / 1e12
    peak, peak_info = device_peak_bf16_tflops(dev.index or 0)
    # algorithmic bytes of one sparse launch: Q, K, V read once, O written once
    alg_bytes = 2 * w.head_dim * w.seqlen * w.batch * (2 * w.heads + 2 * w.kvh)
    traffic = measured_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med["wise_traj"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "seq_len": w.seqlen, "block": 32, "eta": eta, "recurrent_steps": 32,
                   "discovery_union_steps": [9, 12], "reuse_steps": [13, 32]},
        "late_step_tflops": round(tflops, 3),
        "late_step_frac_of_peak": round(tflops / peak, 4),
        "late_step_tflops_setup_inclusive": round(len(REUSE) * sparse_flop / ((med["reuse"] + med["build"]) * 1e-3)
                                                  / 1e12, 3),
        "dense_kernel_tflops": round(dense_tflops, 3),
        "dense_kernel_frac_of_peak": round(dense_tflops / peak, 4),
        "late_speedup_kernel_only": round(med["dense_late"] / med["reuse"], 4),
        "late_speedup_setup_inclusive": round(med["dense_late"] / (med["reuse"] + med["build"]), 4),
        "matched_full_support_late_ms": None if not m_rec else round(matched_ms, 4),
        "matched_speedup": None if not m_rec else round(matched_ms / med["reuse"], 4),
        "wise_trajectory_ms": round(med["wise_traj"], 4),
        "dense_trajectory_ms": round(med["dense_traj"], 4),
        "trajectory_speedup": round(med["dense_traj"] / med["wise_traj"], 4),
        "phase_ms_median": {k: round(v, 4) for k, v in med.items()},
        "phase_ms_iqr": {k: round(v, 4) for k, v in iqr.items()},
        "block_density": round(nnz / causal_blocks, 5),
        "pair_density": round(pairs / dense_pairs, 5),
        "nnz_blocks": nnz,
        "timed_wall_s": round(wall, 3),
        "support_diagnostics": diagnostics,
        "roofline": {
            "kernel": f"wise_sparse_attn: attn_rows_kernel<{w.head_dim}>",
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": round(peak, 1),
            "peak_from": dict(peak_info, formula="compute_units x flop_per_clk_per_cu x clock"),
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": None if traffic is None else traffic["hbm_bytes"],
            "traffic_over_algorithmic": None if traffic is None else round(traffic["hbm_bytes"] / alg_bytes, 3),
            "hbm_read_bytes": None if traffic is None else traffic.get("hbm_read_bytes_per_launch"),
            "l2_hit_rate": None if traffic is None else traffic.get("l2_hit_rate"),
            "algorithmic_flop_per_launch": sparse_flop,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_ms": round(sparse_ms, 5),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")

        per_head = {}

        def gen_f32(t, h):
            # regenerated on the host for one head: the same cast values the GPU read
            if h not in per_head:
                per_head[h] = Generator(w, heads=[h])
            return tuple(x[0, 0].to(torch.float64).numpy() for x in per_head[h].step_torch(t))

        # the GPU's step-13 output and schedule rows of the heads the oracle samples
        o13, _ = wise.sparse_attn(*steps[13], sched)
        torch.cuda.synchronize()
        o13_host = o13[0].to(torch.float64).cpu().numpy()
        gpu_rows = [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(w, eta, gen_f32, args.cpu_budget,
                                                                      gpu_rows, o13_host)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
