"""GPU parity of the cosine-cost solve and plan statistics against the fp64
oracle, which evaluates 1 - x.y / (|x| |y|) from its definition ("FlashSinkhorn:
IO-Aware Entropic Optimal Transport on GPU", significance section: cosine
distance after normalisation). The GPU runs the squared Euclidean kernels on
the normalised points at 2 eps."""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import make_clouds, random_clouds

from gpu_helpers import DEV, TOL_COST, TOL_MARG, TOL_POT, dev, rel_inf

pytestmark = pytest.mark.gpu


def gpu_solve_cos(c, eps, iters, g0=None):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(x.shape[0], device=DEV)
    g = (torch.zeros(y.shape[0], device=DEV) if g0 is None
         else dev(np.asarray(g0, np.float32)))
    lds.ot_sinkhorn_solve_cosine(x, y, a, b, eps, iters, f, g)
    torch.cuda.synchronize()
    return f.cpu().numpy(), g.cpu().numpy()


def gpu_stats_cos(c, f, g, eps):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    lds.ot_plan_stats_cosine(x, y, a, b, dev(np.asarray(f, np.float32)),
                             dev(np.asarray(g, np.float32)), eps, cost, marg)
    torch.cuda.synchronize()
    return cost.item(), marg.cpu().numpy()


@pytest.mark.parametrize("name,n,m,eps,iters", [
    ("gauss3d_1k", 1024, 1024, 0.05, 50), ("feature64_64k", 1500, 2100, 0.1, 30),
    ("mixture_sphere3d_eps_scaling", 1200, 900, 0.02, 40), ("cube_gauss3d_16k", 700, 900, 0.01, 60),
])
def test_cosine_solve_and_stats(name, n, m, eps, iters):
    c = make_clouds(name, n=n, m=m)
    f, g = gpu_solve_cos(c, eps, iters)
    fo, go = oracle.sinkhorn_cosine(c["x"], c["y"], c["a"], c["b"], eps, iters)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    cost, marg = gpu_stats_cos(c, f, g, eps)
    so = oracle.plan_stats_cosine(c["x"], c["y"], c["a"], c["b"], fo, go, eps)
    ec = abs(cost - so["cost"]) / abs(so["cost"])
    em = abs(marg.sum() - so["marg"])
    print(f"{name} cos eps {eps}: f {ef:.2e} g {eg:.2e}; cost {cost:.8g} vs {so['cost']:.8g} "
          f"(rel {ec:.1e}); marg {marg.sum():.2e} vs {so['marg']:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    assert ec <= TOL_COST and em <= TOL_MARG


@pytest.mark.parametrize("d", [160, 192, 384, 1024])
def test_cosine_high_dimension(d):
    # Embedding-sized features: the normalised points go through the
    # 64-column-tile kernels above 128 coordinates, the 16x16-tile kernels
    # above 192 and the kernels tiled like a matrix product above 448.
    c = random_clouds(600, 800, d, seed=d, spread=1.0)
    eps, iters = 0.02, 20
    f, g = gpu_solve_cos(c, eps, iters)
    fo, go = oracle.sinkhorn_cosine(c["x"], c["y"], c["a"], c["b"], eps, iters)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    cost, marg = gpu_stats_cos(c, f, g, eps)
    so = oracle.plan_stats_cosine(c["x"], c["y"], c["a"], c["b"], fo, go, eps)
    ec = abs(cost - so["cost"]) / abs(so["cost"])
    em = abs(marg.sum() - so["marg"])
    print(f"d={d} cos eps {eps}: f {ef:.2e} g {eg:.2e}; cost rel {ec:.1e}; marg diff {em:.1e}",
          flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    assert ec <= TOL_COST and em <= TOL_MARG


def test_cosine_scale_invariance_and_warm_start():
    c = random_clouds(500, 700, 16, seed=3)
    rng = np.random.default_rng(4)
    f1, g1 = gpu_solve_cos(c, 0.05, 10)
    c2 = dict(c)
    c2["x"] = (c["x"] * rng.uniform(0.01, 100.0, size=(500, 1))).astype(np.float32)
    c2["y"] = (c["y"] * rng.uniform(0.01, 100.0, size=(700, 1))).astype(np.float32)
    f2, g2 = gpu_solve_cos(c2, 0.05, 10)
    assert rel_inf(f2, f1, 0.05) <= 1e-5 and rel_inf(g2, g1, 0.05) <= 1e-5
    # warm start: 10 + 10 iterations equal 20 from cold
    f3, g3 = gpu_solve_cos(c, 0.05, 10, g0=g1)
    fo, go = oracle.sinkhorn_cosine(c["x"], c["y"], c["a"], c["b"], 0.05, 20)
    assert rel_inf(f3, fo, 0.05) <= TOL_POT and rel_inf(g3, go, 0.05) <= TOL_POT


def test_cosine_single_source_closed_form():
    rng = np.random.default_rng(5)
    c = {"x": rng.normal(size=(1, 64)).astype(np.float32),
         "y": rng.normal(size=(3000, 64)).astype(np.float32)}
    b = rng.dirichlet(np.ones(3000)).astype(np.float32)
    c["b"] = b
    c["a"] = np.array([b.astype(np.float64).sum()], np.float32)
    f, g = gpu_solve_cos(c, 0.2, 2)
    cost, marg = gpu_stats_cos(c, f, g, 0.2)
    x = c["x"].astype(np.float64)
    y = c["y"].astype(np.float64)
    C = 1 - (y @ x[0]) / (np.linalg.norm(y, axis=1) * np.linalg.norm(x[0]))
    assert cost == pytest.approx(float(b.astype(np.float64) @ C), rel=1e-5)
    assert marg[1] < 1e-5
