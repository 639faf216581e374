"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
library through its binding, compare with the fp64 oracle.

Tolerances (from the target statement of the workloads): potentials
normwise ``max|v - v*| / max|v*| <= 1e-4``; transport cost relative
``<= 1e-5``; marginal L1 error absolute difference ``<= 1e-5``; 4x4 plans
``max|P - P*| <= 1e-5`` at the same iteration count."""
import numpy as np
import torch

import log_domain_sinkhorn_amd as lds

DEV = "cuda:0"
TOL_POT = 1e-4
TOL_COST = 1e-5
TOL_MARG = 1e-5
TOL_P4 = 1e-5


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def rel_inf(v, ref, floor: float = 0.0) -> float:
    """max|v - ref| / max(max|ref|, floor). The floor (eps for potentials)
    keeps the measure defined when the reference potential is ~0, e.g. a
    single target point, where g* is zero up to rounding."""
    v = np.asarray(v, np.float64)
    ref = np.asarray(ref, np.float64)
    den = max(float(np.max(np.abs(ref))) if ref.size else 0.0, floor)
    return float(np.max(np.abs(v - ref)) / (den if den > 0 else 1.0))


def gpu_solve(c, eps, iters, g0=None, f0=None):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    n, m = x.shape[0], y.shape[0]
    f = dev(np.zeros(n, np.float32) if f0 is None else np.asarray(f0, np.float32))
    g = dev(np.zeros(m, np.float32) if g0 is None else np.asarray(g0, np.float32))
    lds.ot_sinkhorn_solve(x, y, a, b, eps, iters, f, g)
    torch.cuda.synchronize()
    return f.cpu().numpy(), g.cpu().numpy()


def gpu_solve_schedule(c, eps0, eps_end, stages, iters):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(x.shape[0], device=DEV)
    g = torch.zeros(y.shape[0], device=DEV)
    lds.ot_sinkhorn_solve_eps_scaling(x, y, a, b, eps0, eps_end, stages, iters, f, g)
    torch.cuda.synchronize()
    return f.cpu().numpy(), g.cpu().numpy()


def gpu_plan_stats(c, f, g, eps):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    lds.ot_plan_stats(x, y, a, b, dev(np.asarray(f, np.float32)), dev(np.asarray(g, np.float32)),
                      eps, cost, marg)
    torch.cuda.synchronize()
    mg = marg.cpu().numpy()
    return {"cost": float(cost.item()), "marg_row": float(mg[0]), "marg_col": float(mg[1]),
            "marg": float(mg[0] + mg[1])}


def gpu_birkhoff(L, eps, max_iters, tol):
    Lt = dev(np.asarray(L, np.float32))
    out = torch.empty_like(Lt)
    it = torch.empty(Lt.shape[0], dtype=torch.int32, device=DEV)
    lds.ot_birkhoff_project_batched(Lt, eps, max_iters, tol, out, it)
    torch.cuda.synchronize()
    return out.cpu().numpy(), it.cpu().numpy()
