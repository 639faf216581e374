#!/usr/bin/env python3
"""Throughput benchmark of the log-domain Sinkhorn hot path on one MI355X.

One step = one whole solve of the workload (cold start, every iteration of
alternating f/g half-steps) followed by its plan statistics (transport cost
and marginal errors), on seeded synthetic inputs already resident in HBM.
The headline workload is the 65536 x 65536 point-cloud problem in d = 64
(fp32, Dirichlet weights, eps = 0.5, 100 iterations), whose half-steps form
each fp32 dot product as three split f16 matrix-core products. ``value`` =
n*m*iterations*steps / timed seconds.

Printed: one JSON line with the metric, the roofline of the dominant kernel
(the half-step), the fp64 CPU oracle timed on a bounded sample of the same
workload on this host's cores, and secondary measurements of the other
workloads (d = 3 VALU path, eps-scaling schedule, the feature workload at
d = 192, transport application, batched 4x4 projection by Sinkhorn-Knopp and
by Newton with its backward).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline] [--no-secondary]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sinkhorn pair-evals/sec (n·m·iters/s) at n=m=65536 + % of FP32/exp roofline"

# MI355X published peaks used for the roofline fractions (dense).
PEAK_MFMA_FP32_TFLOPS = 157.3
PEAK_MFMA_FP16_TFLOPS = 2500.0
# Vector-ALU capacity at the published fp32 vector peak (157.3 TFLOP/s, an
# FMA being 2 flops): 7.865e13 fp32 FMA lane-operations per second. One
# "slot" below is one such FMA lane-operation; what an exp2, a log2 or an add
# costs in slots is measured in the same run by the rate microbenchmarks
# (ratebench/rates.hip) as the FMA rate over its own rate.
VALU_SLOTS_PER_S = 157.3e12 / 2.0
# Work of the method per unit, from the operation counts of the update
# (not from the kernels' instruction mix):
#  d < 32 half-step, per pair-side: d FMAs for the score with the bias folded
#    in, 1 max, 1 subtract, 1 add (2d + 3 flops, d + 3 slots) and one exp2;
#  d >= 32 half-step, per pair-side: the 2d flops of the dot product (the
#    bias enters the accumulator; the epilogue is the d < 32 one minus the
#    score);
#  4x4 Sinkhorn-Knopp iteration: 8 max-subtracted log-sum-exps of 4 terms,
#    24 exp2 + 8 log2 + about 100 other operations.
BIRKHOFF_EXP2, BIRKHOFF_LOG2, BIRKHOFF_OTHER = 24, 8, 100
# One step of the 4x4 Newton dual solver (fp64 exponents and row maxima, row
# softmaxes, gradient and 3x3 Hessian, Cholesky solve, line search), from the
# rocprofv3 instruction counts of the 2^20-matrix batch: 7363 VALU
# instructions per matrix, 755 of them transcendental (two issue slots), over
# 5.37 steps per matrix on average; each non-transcendental counted as one
# slot and each transcendental at its measured cost. (The pages give no
# operation count for the Newton solve; this is the implementation's.)
NEWTON_VALU_PER_MATRIX, NEWTON_TRANS_PER_MATRIX, NEWTON_STEPS = 7363.0, 755.0, 5.37
HBM_PEAK_BYTES_PER_S = 8.0e12


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="feature64_64k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--secondary-only", default=None,
                   help="comma list of secondary workloads to run (default: all)")
    return p.parse_args()


# f16 MFMA stream with data-carrying operands (random mantissas that change
# every step) over ~0.2 s: under it the board lowers its clock (power), so
# this is the f16 matrix rate a long product can sustain, below the
# published peak, which assumes 2.4 GHz.
SUSTAINED_F16 = "v_mfma_f32_32x32x16_f16 sustained, random operands"
RATE_KINDS = {  # kind -> (name, chain steps per lane); see ratebench/rates.hip
    0: ("v_fma_f32", 20000), 1: ("v_exp_f32", 20000), 2: ("v_log_f32 + v_add_f32", 10000),
    3: ("v_exp_f32 beside v_fma_f32", 10000), 4: ("v_fma_f64", 10000),
    5: ("v_mfma_f32_32x32x16_f16", 12000), 6: ("v_mfma_f32_32x32x2f32", 4000),
    7: ("v_add_f32", 20000), 8: (SUSTAINED_F16, 300000)}


def measure_rates():
    """Instruction rates of this GPU (ratebench/librates.so) with the shader
    clock each ran at, and the slot costs (relative to an fp32 FMA) of exp2,
    log2 and add that the ALU ceilings use."""
    import ctypes

    path = os.path.join(ROOT, "log_domain_sinkhorn_amd", "ratebench", "librates.so")
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.otr_measure.argtypes = [ctypes.c_int, ctypes.c_int, dp, dp]
    rates, clocks = {}, {}
    for kind, (name, iters) in RATE_KINDS.items():
        v, hz = ctypes.c_double(0.0), ctypes.c_double(0.0)
        st = lib.otr_measure(kind, iters, ctypes.byref(v), ctypes.byref(hz))
        if st != 0:
            raise RuntimeError(f"rate microbenchmark {name} failed with HIP error {st}")
        rates[name], clocks[name] = v.value, hz.value
    fma = rates["v_fma_f32"]
    add_slots = fma / rates["v_add_f32"]
    per_clk = {k: rates[k] / (clocks[k] * 256) for k in rates if clocks[k] > 0}
    return {
        "lane_ops_per_s": {k: v for k, v in rates.items() if "mfma" not in k},
        "mfma_tflops": {k: v / 1e12 for k, v in rates.items() if "mfma" in k},
        "shader_clock_ghz": {k: v / 1e9 for k, v in clocks.items()},
        "per_clock_per_cu": per_clk,
        "exp2_slots": fma / rates["v_exp_f32"],
        "log2_slots": fma / rates["v_log_f32 + v_add_f32"] - add_slots,
        "add_slots": add_slots,
        "exp2_beside_fma_slots": 2.0 * fma / rates["v_exp_f32 beside v_fma_f32"],
        "source": "log_domain_sinkhorn_amd/ratebench/rates.hip",
    }


def alu_slots_per_pair_side(d: int, rates) -> float:
    """Slots of the method's work per pair-side of a d < 32 half-step: d FMAs,
    max, subtract, add, one exp2."""
    return d + 3 * rates["add_slots"] + rates["exp2_slots"]


def source_digest(files):
    """Digest of the named sources; None if one of them no longer exists."""
    h = hashlib.sha256()
    for f in files:
        path = os.path.join(ROOT, f)
        if not os.path.exists(path):
            return None
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, only while
    the kernel source still matches the one the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}:{workload}")
    except (ValueError, OSError):
        return None
    if not rec:
        return None
    digest = source_digest(rec.get("sources", []))
    if digest is None or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP events on the stream the library launches on (torch's current)."""

    def __init__(self, torch):
        self.torch = torch
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def __enter__(self):
        self.a.record()
        return self

    def __exit__(self, *exc):
        self.b.record()

    def ms(self) -> float:
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


COPY_BYTES = 64 << 20


def calibration_copy(torch):
    """One plain device-to-device copy of COPY_BYTES: the reference kernel that
    scales the FETCH_SIZE / WRITE_SIZE counters of a profiled run."""
    src = torch.ones(COPY_BYTES // 4, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    return COPY_BYTES


def run_cloud_workload(name, steps, warmup, torch, lds, with_stats=True):
    from workloads import make_clouds

    c = make_clouds(name)
    dev = torch.device("cuda:0")
    x, y, a, b = (torch.from_numpy(c[k]).to(dev) for k in "xyab")
    n, m, d = c["n"], c["m"], c["d"]
    eps_list, iters = c["eps"], c["iters"]
    f = torch.zeros(n, device=dev)
    g = torch.zeros(m, device=dev)
    cost = torch.zeros(1, dtype=torch.float64, device=dev)
    marg = torch.zeros(2, dtype=torch.float64, device=dev)

    def solve():
        g.zero_()
        if len(eps_list) == 1:
            lds.ot_sinkhorn_solve(x, y, a, b, eps_list[0], iters, f, g)
        else:
            lds.ot_sinkhorn_solve_eps_scaling(x, y, a, b, eps_list[0], eps_list[-1],
                                              len(eps_list), iters, f, g)

    def stats():
        lds.ot_plan_stats(x, y, a, b, f, g, eps_list[-1], cost, marg)

    for _ in range(warmup):
        solve()
        if with_stats:
            stats()
    torch.cuda.synchronize()
    solve_ms, stats_ms = [], []
    t0 = time.perf_counter()
    with Timer(torch) as total:
        for _ in range(steps):
            with Timer(torch) as ts:
                solve()
            solve_ms.append(ts)
            if with_stats:
                with Timer(torch) as tp:
                    stats()
                stats_ms.append(tp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = total.ms()
    solve_ms = [t.ms() for t in solve_ms]
    stats_ms = [t.ms() for t in stats_ms]
    total_iters = iters * len(eps_list)
    # The half-step launch duration, live, on the stream the library launches
    # on: solves of k_long and k_short iterations differ by exactly
    # 2 (k_long - k_short) half-steps (each: the half-step kernel and, with
    # column splits, its merge); the per-solve record preparation cancels.
    k_long, k_short = min(iters, 21), 1
    eps_last = eps_list[-1]

    def solve_k(k):
        g.zero_()
        lds.ot_sinkhorn_solve(x, y, a, b, eps_last, k, f, g)

    half_ms = None
    if k_long > k_short:
        t_long, t_short = [], []
        for _ in range(3):
            with Timer(torch) as tl:
                solve_k(k_long)
            with Timer(torch) as tsh:
                solve_k(k_short)
            t_long.append(tl)
            t_short.append(tsh)
        d_ms = [tl.ms() - tsh.ms() for tl, tsh in zip(t_long, t_short)]
        half_ms = sorted(d_ms)[1] / (2 * (k_long - k_short))
    return {
        "name": name, "n": n, "m": m, "d": d, "eps": list(eps_list), "iters": iters,
        "total_iters": total_iters, "steps": steps, "total_ms": total_ms, "wall_s": wall,
        "ms_per_step": total_ms / steps, "solve_ms": sum(solve_ms) / steps,
        "stats_ms": (sum(stats_ms) / steps) if stats_ms else None,
        "half_step_ms": half_ms,
        "half_step_ms_whole_solve": sum(solve_ms) / steps / (2 * total_iters),
        "pair_evals_per_s": n * m * total_iters * steps / (total_ms / 1e3),
        "cost": cost.item(), "marg": marg.cpu().tolist(),
    }


def h3_kp(d: int) -> int:
    """Coordinates per record of the split-f16 half-step: d padded to a
    multiple of 32 up to 256, of 64 up to 448, of 128 above."""
    if d <= 256:
        return (d + 31) // 32 * 32
    return (d + 63) // 64 * 64 if d <= 448 else (d + 127) // 128 * 128


def h3_kernel(kp: int) -> str:
    """The half-step kernel the library runs for kp coordinates per record."""
    return "lse_rows_h3_kernel" if kp <= 192 else (
        "lse_rows_wide_kernel" if kp <= 448 else "lse_rows_gemm_kernel")


def roofline_for(r, workload, rates):
    """Roofline of the half-step kernel: the method's work per launch (per
    pair-side counts above) over the live launch duration, against the peak
    of what executes it."""
    n, m, d = r["n"], r["m"], r["d"]
    launch_s = r["half_step_ms"] / 1e3
    if d >= 32:
        # The dot products run on the f16 matrix cores (each fp32 product as
        # three split f16 products), so the peak is the f16 dense peak; the
        # method's work is 2d flops per pair-side.
        kp = h3_kp(d)
        kernel = h3_kernel(kp)
        work = 2.0 * d * n * m
        ach = work / launch_s / 1e12
        # Implementation model, beside it: the kernel issues 6*kp f16 MFMA
        # flops (three split products over the kp padded coordinates) and
        # fp32 MFMA flops for the column bias and row offset per pair-side on
        # the one matrix pipe, one after the other: 4 on 32x32 tiles (d <=
        # 192; 448 cycles per 32x32 subtile-wave at d = 64), 8 on the 16x16
        # tiles up to d = 448 (the 16x16x4 instruction's four k-slots, two
        # used), none above (the kernel tiled like a matrix product adds the
        # bias on the vector ALUs). At the published peaks its ceiling on the method's
        # rate is 2d / (6 kp + fp32 flops * 2500/157.3).
        bias_flops = {"lse_rows_h3_kernel": 4.0, "lse_rows_wide_kernel": 8.0}.get(kernel, 0.0)
        impl_flops = 6.0 * kp + bias_flops * PEAK_MFMA_FP16_TFLOPS / PEAK_MFMA_FP32_TFLOPS
        impl_ach = impl_flops * n * m / launch_s / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": PEAK_MFMA_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_MFMA_FP16_TFLOPS,
                "traffic": traffic_for(kernel, workload),
                "kernel": f"{kernel}<{kp}>",
                "launch_ms": r["half_step_ms"],
                "work_per_launch": f"{n}*{m} pair-sides x {2 * d} flops (the dot product, 2d)",
                "peak_dtype": "f16 (dense matrix cores; the fp32 dot products are formed as "
                              "three split f16 products with fp32 accumulation)",
                "implementation_model": {
                    "matrix_flops_per_pair_side": f"{6 * kp} f16 + {bias_flops:.0f} fp32 MFMA",
                    "f16_equivalent_per_pair_side": impl_flops,
                    "achieved_f16_equivalent_tflops": impl_ach,
                    "frac_of_f16_peak": impl_ach / PEAK_MFMA_FP16_TFLOPS,
                    "ceiling_on_frac": 2.0 * d / impl_flops},
                "vs_sustained_f16_mfma": {
                    "sustained_tflops": rates["mfma_tflops"][SUSTAINED_F16],
                    "shader_clock_ghz": rates["shader_clock_ghz"][SUSTAINED_F16],
                    "implementation_frac": impl_ach / rates["mfma_tflops"][SUSTAINED_F16]},
                "vs_fp32_mfma_peak": {"fp32_equivalent_tflops": ach,
                                      "peak": PEAK_MFMA_FP32_TFLOPS,
                                      "ratio": ach / PEAK_MFMA_FP32_TFLOPS}}
    slots = alu_slots_per_pair_side(d, rates)
    flops_per_ps = 2 * d + 3
    ach = flops_per_ps * n * m / launch_s / 1e12
    peak = VALU_SLOTS_PER_S / slots * flops_per_ps / 1e12
    return {"bound": "alu", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
            "frac": ach / peak, "traffic": traffic_for("lse_rows_valu_kernel", workload),
            "kernel": "lse_rows_valu_kernel", "launch_ms": r["half_step_ms"],
            "work_per_launch": f"{n}*{m} pair-sides x ({flops_per_ps} flops + 1 exp2)",
            "peak_model": f"{VALU_SLOTS_PER_S:.4g} fp32 FMA lane-ops/s (157.3 TFLOP/s) / "
                          f"{slots:.2f} slots per pair-side ({d} FMA + max + sub + add at "
                          f"{rates['add_slots']:.2f} + exp2 at {rates['exp2_slots']:.2f} slots, "
                          "measured)"}


def stats_roofline(n, m, d, stats_ms, rates):
    """Plan statistics (one row pass with cost, one column pass) against the
    method's work. Per pair and pass: the score (d FMAs), the exp2, the sum
    of P (1 add) and in the row pass the cost term (C from the score: 2
    flops, P*C: 1 FMA). d < 32: issue slots at the published clock; d >= 32:
    the score's 2d flops per pass on the f16 matrix-core peak."""
    if d >= 32:
        work_ms = 2.0 * 2.0 * d * n * m / (PEAK_MFMA_FP16_TFLOPS * 1e12) * 1e3
        return {"bound": "mfma", "model_ms": work_ms, "frac": work_ms / stats_ms,
                "model": "2 passes x 2d flops per pair on the f16 peak"}
    e, ad = rates["exp2_slots"], rates["add_slots"]
    slots = (d + ad + e + 3 * ad) + (d + ad + e)
    model_ms = n * m * slots / VALU_SLOTS_PER_S * 1e3
    return {"bound": "alu", "model_ms": model_ms, "frac": model_ms / stats_ms,
            "model": f"{slots:.2f} issue slots per pair over both passes"}


def gemm_calibration(torch, n=8192, reps=10):
    """A plain f16 GEMM (n x n x n, torch.matmul on the vendor BLAS) timed on the
    same GPU in the same run: the matrix-core throughput a dense library
    product sustains here, under the same power and clock limits as the
    half-step kernel. Context for the matrix roofline fraction; not a peak."""
    try:
        a = torch.randn(n, n, device="cuda:0", dtype=torch.float16)
        b = torch.randn(n, n, device="cuda:0", dtype=torch.float16)
        for _ in range(3):
            c = a @ b
        with Timer(torch) as t:
            for _ in range(reps):
                c = a @ b
        del a, b, c
    except RuntimeError as exc:  # context only: never lose the benchmark line for it
        return {"op": f"f16 GEMM {n}^3 (torch.matmul)", "error": str(exc)[:200]}
    tflops = 2.0 * n ** 3 * reps / (t.ms() / 1e3) / 1e12
    return {"op": f"f16 GEMM {n}^3 (torch.matmul)", "tflops": tflops,
            "frac_of_peak": tflops / PEAK_MFMA_FP16_TFLOPS}


def cpu_baseline(name):
    import oracle
    from workloads import make_clouds

    c = make_clouds(name)
    ns = min(c["n"], 16384 if c["d"] >= 32 else 32768)
    ms = min(c["m"], ns)
    it = 10 if c["d"] >= 32 else 4
    sub = {"x": c["x"][:ns], "y": c["y"][:ms], "a": c["a"][:ns], "b": c["b"][:ms]}
    t0 = time.perf_counter()
    oracle.sinkhorn(sub["x"], sub["y"], sub["a"], sub["b"], c["eps"][0], it)
    dt = time.perf_counter() - t0
    return {"value": ns * ms * it / dt, "unit": "pair-evals/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 oracle solve of the first {ns} x {ms} points of {name}, {it} "
                      f"iterations at eps={c['eps'][0]} ({dt:.1f} s)"}


def run_birkhoff(name, torch, lds, rates, reps=5):
    from workloads import BIRKHOFF_WORKLOADS, make_logits

    slots = (BIRKHOFF_EXP2 * rates["exp2_slots"] + BIRKHOFF_LOG2 * rates["log2_slots"]
             + BIRKHOFF_OTHER * rates["add_slots"])
    w = BIRKHOFF_WORKLOADS[name]
    L = torch.from_numpy(make_logits(w.batch, w.sigmas, seed=0)).to("cuda:0")
    out = torch.empty_like(L)
    it = torch.empty(w.batch, dtype=torch.int32, device=L.device)
    lds.ot_birkhoff_project_batched(L, w.eps, w.max_iters, w.tol, out, it)
    torch.cuda.synchronize()
    with Timer(torch) as t:
        for _ in range(reps):
            lds.ot_birkhoff_project_batched(L, w.eps, w.max_iters, w.tol, out, it)
    ms = t.ms() / reps
    iters = it.to(torch.int64)
    issued = int(iters.view(-1, 64).max(dim=1).values.sum().item()) * 64
    useful = int(iters.sum().item())
    # Histogram of the iterations each matrix took (upper edges inclusive).
    edges = [e for e in (1, 5, 10, 20, 50, 100, 150, 199) if e < w.max_iters] + [w.max_iters]
    counts, lo = {}, 0
    for e in edges:
        counts[f"{lo + 1}-{e}"] = int(((iters > lo) & (iters <= e)).sum().item())
        lo = e
    return {"name": name, "batch": w.batch, "max_iters": w.max_iters, "tol": w.tol,
            "ms": ms, "matrices_per_s": w.batch / (ms / 1e3),
            "useful_matrix_iters_per_s": useful / (ms / 1e3),
            "issued_matrix_iters_per_s": issued / (ms / 1e3),
            "mean_iters": useful / w.batch,
            "iters_histogram": counts,
            "hbm_gb_per_s": w.batch * (64 + 64 + 4) / (ms / 1e3) / 1e9,
            # Iterations issued (a wave runs until its slowest lane stops)
            # against the issue-slot ceiling of the method's work per
            # iteration (24 exp2 + 8 log2 + ~100 operations, transcendentals
            # at their measured slot cost).
            "roofline": {"bound": "alu", "achieved": issued / (ms / 1e3),
                         "peak": VALU_SLOTS_PER_S / slots,
                         "unit": "matrix-iterations/s",
                         "frac": issued / (ms / 1e3) / (VALU_SLOTS_PER_S / slots),
                         "slots_per_iteration": slots}}


def run_birkhoff_newton(name, torch, lds, rates, reps=5):
    """Newton forward (tol 1e-6, cap 50 steps) and the implicit backward on the
    batch of ``name``; the backward is HBM-bound (plan and dl/dP in, dl/dL
    out: 192 bytes per matrix)."""
    from workloads import BIRKHOFF_WORKLOADS, make_logits

    w = BIRKHOFF_WORKLOADS[name]
    L = torch.from_numpy(make_logits(w.batch, w.sigmas, seed=0)).to("cuda:0")
    out = torch.empty_like(L)
    grad = torch.randn(L.shape, generator=torch.Generator().manual_seed(1)).to(L.device)
    gl = torch.empty_like(L)
    it = torch.empty(w.batch, dtype=torch.int32, device=L.device)
    lds.ot_birkhoff_project_newton_batched(L, w.eps, 50, 1e-6, out, it)
    lds.ot_birkhoff_projection_backward_batched(out, grad, w.eps, gl)
    torch.cuda.synchronize()
    with Timer(torch) as tf:
        for _ in range(reps):
            lds.ot_birkhoff_project_newton_batched(L, w.eps, 50, 1e-6, out, it)
    with Timer(torch) as tb:
        for _ in range(reps):
            lds.ot_birkhoff_projection_backward_batched(out, grad, w.eps, gl)
    fms, bms = tf.ms() / reps, tb.ms() / reps
    steps = it.to(torch.int64)
    step_slots = ((NEWTON_VALU_PER_MATRIX - NEWTON_TRANS_PER_MATRIX) * rates["add_slots"]
                  + NEWTON_TRANS_PER_MATRIX * rates["exp2_slots"]) / NEWTON_STEPS
    return {"name": f"{name}:newton", "batch": w.batch, "tol": 1e-6, "max_steps": 50,
            "forward_ms": fms, "backward_ms": bms,
            "forward_matrices_per_s": w.batch / (fms / 1e3),
            "forward_backward_matrices_per_s": w.batch / ((fms + bms) / 1e3),
            "mean_steps": float(steps.float().mean().item()), "max_steps_taken": int(steps.max()),
            "backward_hbm_gb_per_s": w.batch * 192 / (bms / 1e3) / 1e9,
            # forward: ALU-bound (one matrix per lane, fp64 and exp2 work in
            # registers), against the implementation's instruction count;
            # backward: HBM-bound, 192 bytes per matrix
            "roofline": {"bound": "alu",
                         "achieved": float(steps.sum().item()) / (fms / 1e3),
                         "peak": VALU_SLOTS_PER_S / step_slots,
                         "unit": "matrix-steps/s",
                         "frac": float(steps.sum().item()) / (fms / 1e3)
                         / (VALU_SLOTS_PER_S / step_slots),
                         "slots_per_step": step_slots},
            "backward_roofline": {"bound": "hbm",
                                  "achieved": w.batch * 192 / (bms / 1e3) / 1e9,
                                  "peak": HBM_PEAK_BYTES_PER_S / 1e9, "unit": "GB/s",
                                  "frac": w.batch * 192 / (bms / 1e3) / HBM_PEAK_BYTES_PER_S}}


def run_transport(name, torch, lds, rates, reps=10, warm=3):
    """Transport application P·y (values = the target points) and the
    x-gradient at the potentials of a short solve of workload ``name``."""
    from workloads import make_clouds

    c = make_clouds(name)
    dev = torch.device("cuda:0")
    x, y, a, b = (torch.from_numpy(c[k]).to(dev) for k in "xyab")
    n, m, d = c["n"], c["m"], c["d"]
    eps = c["eps"][-1]
    f = torch.zeros(n, device=dev)
    g = torch.zeros(m, device=dev)
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 5, f, g)
    out = torch.empty((n, d), device=dev)
    res = {"name": name, "n": n, "m": m, "d": d, "dv": d}
    for label, fn in (("apply", lambda: lds.ot_transport_apply(x, y, f, g, eps, y, out)),
                      ("grad", lambda: lds.ot_cost_gradient_x(x, y, f, g, eps, out))):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        with Timer(torch) as t:
            for _ in range(reps):
                fn()
        ms = t.ms() / reps
        res[f"{label}_ms"] = ms
        res[f"{label}_pairs_per_s"] = n * m / (ms / 1e3)
    if d >= 32:
        # Matrix-pipe time per 32x32 subtile and wave: the split-f16 score
        # once (3*kp/16 f16 MFMAs of 32 cycles + one fp32 MFMA of 64) and P.V
        # (12 bf16 MFMAs of 32 cycles per 32 value channels: 2 column chunks
        # x 6 split products), at 2.4 GHz on 1024 SIMDs; frac = that time /
        # the measured call, so the 32x32 kernel's score recomputation per
        # pass of 32 value channels (d <= 192) counts against it; above 192
        # the score is formed once for every channel.
        kp = h3_kp(d)
        cycles = 3 * kp // 16 * 32 + 64 + 12 * 32 * ((d + 31) // 32)
        model_ms = (n / 32) * (m / 32) * cycles / (1024 * 2.4e9) * 1e3
        res["roofline_whole_call"] = {"bound": "mfma", "model_ms": model_ms,
                                      "frac": model_ms / res["apply_ms"],
                                      "model": f"{cycles} matrix-pipe cycles per 32x32 subtile"}
    else:
        # VALU path, the method's work per pair: the exponent (d FMAs and
        # the bias add), one exp2, dv FMAs (P v).
        slots = d + rates["add_slots"] + rates["exp2_slots"] + d
        model_ms = n * m * slots / VALU_SLOTS_PER_S * 1e3
        res["roofline_whole_call"] = {"bound": "alu", "model_ms": model_ms,
                                      "frac": model_ms / res["apply_ms"],
                                      "model": f"{slots:g} issue slots per pair"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import log_domain_sinkhorn_amd as lds

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    lds.load_library()
    copy_bytes = calibration_copy(torch)

    print(f"# headline {args.workload}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr,
          flush=True)
    r = run_cloud_workload(args.workload, args.steps, args.warmup, torch, lds)
    print("# instruction rates", file=sys.stderr, flush=True)
    rates = measure_rates()
    dtype = ("f32 (dot products as three split f16 matrix-core products, fp32 accumulation)"
             if r["d"] >= 32 else "f32 (scores formed in f64)")
    out = {
        "metric": METRIC, "value": r["pair_evals_per_s"], "unit": "pair-evals/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": args.workload, "n": r["n"], "m": r["m"], "d": r["d"],
                   "eps": r["eps"], "iters": r["iters"],
                   "step": "cold-start solve + plan statistics"},
        "roofline": roofline_for(r, args.workload, rates),
        "detail": {"calibration_copy_bytes": copy_bytes,
                   "f16_gemm_same_gpu": gemm_calibration(torch) if r["d"] >= 32 else None,
                   "solve_ms": r["solve_ms"], "stats_ms": r["stats_ms"],
                   "stats_roofline": stats_roofline(r["n"], r["m"], r["d"], r["stats_ms"],
                                                    rates),
                   "half_step_ms": r["half_step_ms"],
                   "half_step_ms_whole_solve": r["half_step_ms_whole_solve"],
                   "cost": r["cost"], "marg": r["marg"], "rates": rates},
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload)
    if not args.no_secondary:
        sec = {}
        wanted = None if args.secondary_only is None else set(args.secondary_only.split(","))
        for name in ("cube_gauss3d_64k", "cube_gauss3d_16k", "mixture_sphere3d_eps_scaling",
                     "feature192_64k", "feature256_64k", "feature1024_50k"):
            if name == args.workload or (wanted is not None and name not in wanted):
                continue
            print(f"# secondary {name}", file=sys.stderr, flush=True)
            s = run_cloud_workload(name, 1, 1, torch, lds)
            sec[name] = {"pair_evals_per_s": s["pair_evals_per_s"], "ms_per_step": s["ms_per_step"],
                         "solve_ms": s["solve_ms"], "stats_ms": s["stats_ms"],
                         "stats_roofline": stats_roofline(s["n"], s["m"], s["d"], s["stats_ms"],
                                                          rates),
                         "roofline": roofline_for(s, name, rates)}
        for name, reps, warm in (("feature64_64k", 10, 3), ("cube_gauss3d_64k", 10, 3),
                                 ("feature1024_50k", 3, 1)):
            key = f"transport:{name}"
            if wanted is not None and key not in wanted:
                continue
            print(f"# secondary {key}", file=sys.stderr, flush=True)
            sec[key] = run_transport(name, torch, lds, rates, reps=reps, warm=warm)
        for name in ("birkhoff4x4_1m_fixed20", "birkhoff4x4_1m"):
            if wanted is not None and name not in wanted:
                continue
            print(f"# secondary {name}", file=sys.stderr, flush=True)
            sec[name] = run_birkhoff(name, torch, lds, rates)
        if wanted is None or "birkhoff4x4_1m:newton" in wanted:
            print("# secondary birkhoff4x4_1m:newton", file=sys.stderr, flush=True)
            sec["birkhoff4x4_1m:newton"] = run_birkhoff_newton("birkhoff4x4_1m", torch, lds,
                                                               rates)
        out["secondary"] = sec
    print(json.dumps(out))


if __name__ == "__main__":
    main()
