"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

* Whole solves at sizes the oracle finishes in seconds, spanning several
  tiles, column splits and ragged tails, at the workloads' eps and iteration
  counts (the eps-scaling workload with its 8-stage schedule).
* At the workloads' full sizes (same launch configuration as the benchmark):
  one f and one g half-step from identical inputs, checked on sampled rows
  and columns the oracle computes one by one, plus plan statistics.
* Edge cases: n = 1, m = 1, tiny and odd shapes, d at every kernel boundary,
  iters = 0, warm starts, determinism.

The update being checked: "FlashSinkhorn: IO-Aware Entropic Optimal Transport
on GPU", Methodik section 1 (log-domain f/g updates; exact online LSE,
section 2).
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import make_clouds, random_clouds

from gpu_helpers import (DEV, TOL_COST, TOL_MARG, TOL_POT, dev, gpu_plan_stats, gpu_solve,
                         gpu_solve_schedule, rel_inf)

pytestmark = pytest.mark.gpu

# one exact half-step from identical fp32 inputs: fp32 rounding only
TOL_HALF = 1e-5


def _check_solve(c, eps, iters, label):
    f, g = gpu_solve(c, eps, iters)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, iters)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    print(f"{label}: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    return f, g, fo, go


def _check_stats(c, f, g, fo, go, eps, label):
    st = gpu_plan_stats(c, f, g, eps)
    so = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], fo, go, eps)
    ec = abs(st["cost"] - so["cost"]) / abs(so["cost"])
    em = abs(st["marg"] - so["marg"])
    print(f"{label}: cost {st['cost']:.8g} vs {so['cost']:.8g} (rel {ec:.1e}); "
          f"marg {st['marg']:.3e} vs {so['marg']:.3e} (abs {em:.1e})", flush=True)
    assert ec <= TOL_COST
    assert em <= TOL_MARG
    # the kernel alone: same fp32 (f, g) on both sides
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    assert abs(st["cost"] - sk["cost"]) <= 1e-6 * abs(sk["cost"])
    assert abs(st["marg_row"] - sk["marg_row"]) <= 1e-6
    assert abs(st["marg_col"] - sk["marg_col"]) <= 1e-6


# --------------------------------------------------------------------------- #
# whole solves                                                                  #
# --------------------------------------------------------------------------- #

def test_gauss3d_1k_full_workload():
    c = make_clouds("gauss3d_1k")
    eps, iters = c["eps"][0], c["iters"]
    f, g, fo, go = _check_solve(c, eps, iters, "gauss3d_1k")
    _check_stats(c, f, g, fo, go, eps, "gauss3d_1k")


@pytest.mark.parametrize("name,n,m", [
    ("cube_gauss3d_16k", 2048, 2048),
    ("cube_gauss3d_16k", 3001, 2777),
    ("feature64_64k", 2048, 2048),
    ("feature64_64k", 1500, 2600),
])
def test_workload_distributions_reduced_size(name, n, m):
    c = make_clouds(name, n=n, m=m)
    eps, iters = c["eps"][0], c["iters"]
    f, g, fo, go = _check_solve(c, eps, iters, f"{name}[{n}x{m}]")
    _check_stats(c, f, g, fo, go, eps, f"{name}[{n}x{m}]")


def test_eps_scaling_schedule_reduced_size():
    c = make_clouds("mixture_sphere3d_eps_scaling", n=2048, m=1536)
    eps_list = c["eps"]
    f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), c["iters"])
    fo, go = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], eps_list, c["iters"])
    ef, eg = rel_inf(f, fo), rel_inf(g, go)
    print(f"mixture schedule: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps_list[-1], "mixture schedule")


SHAPES = [
    (1, 1, 3), (1, 97, 3), (97, 1, 3), (7, 7, 3), (1023, 777, 3), (129, 4097, 1),
    (300, 200, 2), (2000, 1500, 5), (5000, 300, 3), (300, 5000, 3), (256, 256, 31),
    (256, 256, 32), (256, 256, 33), (512, 384, 64), (200, 300, 128), (257, 1000, 48),
    (1, 97, 64), (97, 1, 64), (1, 1, 40), (129, 700, 96),
    # above 128 coordinates: 64-column tiles, hi operands read twice
    (129, 700, 129), (300, 257, 160), (257, 300, 192), (1, 97, 192), (97, 1, 160),
]


@pytest.mark.parametrize("n,m,d", SHAPES)
def test_shapes(n, m, d):
    c = random_clouds(n, m, d, seed=n * 7 + m * 3 + d)
    eps = 0.5 * d ** 0.5
    _check_solve(c, eps, 10, f"shape {n}x{m}x{d}")


STATS_SHAPES = [(1, 300, 64), (300, 1, 64), (129, 257, 33), (600, 200, 96), (257, 300, 128),
                (1, 1, 40), (300, 500, 31), (129, 257, 150), (300, 200, 192)]


@pytest.mark.parametrize("n,m,d", STATS_SHAPES)
def test_plan_stats_shapes(n, m, d):
    # Plan statistics on the same fp32 (f, g) as the oracle: the kernels alone.
    c = random_clouds(n, m, d, seed=n + 5 * m + d, spread=1.0 / np.sqrt(d))
    eps = 0.3
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    st = gpu_plan_stats(c, f, g, eps)
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    ec = abs(st["cost"] - sk["cost"]) / abs(sk["cost"])
    print(f"stats {n}x{m}x{d}: cost rel {ec:.1e}; marg {st['marg_row']:.3e}/{st['marg_col']:.3e} "
          f"vs {sk['marg_row']:.3e}/{sk['marg_col']:.3e}", flush=True)
    assert ec <= TOL_COST
    assert abs(st["marg_row"] - sk["marg_row"]) <= TOL_MARG
    assert abs(st["marg_col"] - sk["marg_col"]) <= TOL_MARG


@pytest.mark.parametrize("d,offset", [(64, 30.0), (40, -50.0), (3, 30.0)])
def test_plan_stats_offset_clouds(d, offset):
    # Both clouds far from the origin: the d >= 32 records are built from the
    # centred points, so cost and marginals keep the precision they have near
    # the origin (the d < 32 path forms its scores in fp64).
    c = random_clouds(400, 500, d, seed=d + 11, spread=1.0 / np.sqrt(d))
    c["x"] = c["x"] + np.float32(offset)
    c["y"] = c["y"] + np.float32(offset)
    eps = 0.3
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    st = gpu_plan_stats(c, f, g, eps)
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    ec = abs(st["cost"] - sk["cost"]) / abs(sk["cost"])
    print(f"stats offset {offset:g} d={d}: cost rel {ec:.1e}; marg {st['marg_row']:.3e}/"
          f"{st['marg_col']:.3e} vs {sk['marg_row']:.3e}/{sk['marg_col']:.3e}", flush=True)
    assert ec <= TOL_COST
    assert abs(st["marg_row"] - sk["marg_row"]) <= TOL_MARG
    assert abs(st["marg_col"] - sk["marg_col"]) <= TOL_MARG


# d >= 32 runs on split-f16 matrix-core products (three f16 products per fp32
# product, fp32 accumulation). The split itself keeps ~22 bits of each
# coordinate; the matrix core's aligned sums lose about 2^-21 of the largest
# product per instruction (measured), comparable to fp32 accumulation. These
# cases use N(0, I) clouds (coordinates up to ~4.5, so products up to ~20 and
# many coordinates small enough that their lo parts are f16 subnormals), at
# several eps; one half-step is held to the same bound as the other paths.
# The records hold the points centred on the mean of the two cloud means, so
# clouds far from the origin (offset != 0) meet the same bound: uncentred,
# the expanded |x|^2 + |y|^2 - 2 x.y of clouds 30 units out cancels about
# 2^10 of the products' precision (measured 2.8e-4 after three iterations).
TOL_SPLIT_HALF = TOL_HALF


@pytest.mark.parametrize("d,eps_factor,offset", [(32, 0.5, 0.0), (64, 0.5, 0.0), (64, 0.1, 0.0),
                                                 (128, 0.1, 0.0), (96, 1.0, 0.0),
                                                 (64, 0.5, 30.0), (32, 0.1, -50.0),
                                                 (160, 0.5, 0.0), (192, 0.1, 0.0),
                                                 (192, 0.5, 40.0)])
def test_split_f16_half_step_on_unit_gaussians(d, eps_factor, offset):
    # offset != 0: both clouds moved far from the origin. The records hold
    # x - c and y - c (c the mean of the two cloud means; the cost does not
    # change), so the products stay near the size of the costs and the same
    # bound holds.
    c = random_clouds(1024, 1536, d, seed=d, spread=1.0)
    c["x"] = c["x"] + np.float32(offset)
    c["y"] = c["y"] + np.float32(offset)
    eps = eps_factor * d ** 0.5
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 5)
    g32 = go.astype(np.float32)
    f1, g1 = gpu_solve(c, eps, 1, g0=g32)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g32, eps)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f1, eps)
    ef, eg = rel_inf(f1, f_ref), rel_inf(g1, g_ref)
    print(f"d={d} eps={eps:.3g} offset {offset:g}: one half-step rel err f {ef:.2e} g {eg:.2e}",
          flush=True)
    assert ef <= TOL_SPLIT_HALF and eg <= TOL_SPLIT_HALF


@pytest.mark.parametrize("d,eps", [(3, 1e-3), (64, 1e-3), (3, 1e4), (64, 1e4)])
def test_extreme_eps_half_step(d, eps):
    # The degenerate ends of the method: eps far below the costs (the plan is
    # close to an assignment, the log-sum-exp is its max term) and far above
    # them (the plan is close to the product a b^T). One f and one g half-step
    # from the oracle's iterate, on both paths (fp64 VALU scores for d = 3,
    # split-f16 matrix cores for d = 64).
    c = random_clouds(700, 500, d, seed=int(d + 1e3 * eps) % 9973, spread=1.0 / np.sqrt(d))
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 5)
    g32 = go.astype(np.float32)
    f1, g1 = gpu_solve(c, eps, 1, g0=g32)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g32, eps)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f1, eps)
    ef, eg = rel_inf(f1, f_ref), rel_inf(g1, g_ref)
    print(f"d={d} eps={eps:g}: one half-step rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF


def test_split_f16_long_solve_on_unit_gaussians():
    c = random_clouds(700, 900, 64, seed=3, spread=1.0)
    _check_solve(c, 0.25 * 8.0, 60, "d=64 N(0,I) 60 iterations")


@pytest.mark.parametrize("log2_range,finite", [(29, True), (34, False)])
def test_split_f16_range_precondition(log2_range, finite):
    # The split-f16 records hold (2 log2(e)/eps) max|x| max|y| = T split
    # evenly over the two sides up to a factor 2^(1/2); below T = 2^30 the hi
    # parts stay finite in f16 and one half-step is as accurate as elsewhere,
    # at T = 2^34 they overflow and the documented outcome is non-finite f.
    c = random_clouds(300, 400, 32, seed=5, spread=1.0)
    mx = float(np.abs(c["x"]).max()) * float(np.abs(c["y"]).max())
    eps = 2.0 * np.log2(np.e) * mx / 2.0 ** log2_range
    f1, _ = gpu_solve(c, eps, 1)
    if finite:
        f_ref = oracle.half_update(c["x"], c["y"], c["a"], np.zeros(400, np.float32), eps)
        err = rel_inf(f1, f_ref)
        print(f"T = 2^{log2_range}: eps {eps:.3g}, one half-step rel err f {err:.2e}", flush=True)
        assert err <= TOL_SPLIT_HALF
    else:
        assert not np.all(np.isfinite(f1))


def test_iters_zero_leaves_potentials():
    c = random_clouds(100, 80, 3, seed=1)
    f0 = np.linspace(-1, 1, 100).astype(np.float32)
    g0 = np.linspace(2, 3, 80).astype(np.float32)
    f, g = gpu_solve(c, 0.3, 0, g0=g0, f0=f0)
    np.testing.assert_array_equal(f, f0)
    np.testing.assert_array_equal(g, g0)


def test_eps_scaling_schedule_d64():
    # The split-f16 records are rebuilt per stage (their scale is 2 log2(e)/eps).
    from workloads import geometric_eps_schedule
    c = make_clouds("feature64_64k", n=1200, m=1700)
    eps_list = geometric_eps_schedule(2.0, 0.05, 5)
    f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), 15)
    fo, go = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], eps_list, 15)
    ef, eg = rel_inf(f, fo, eps_list[-1]), rel_inf(g, go, eps_list[-1])
    print(f"d=64 schedule: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps_list[-1], "d=64 schedule")


def test_eps_scaling_schedule_d160():
    # Above 128 coordinates (64-column tiles, hi operands read twice), with
    # the records rebuilt per stage; the d = 64 workload's distributions at
    # d = 160 (N(0, I/d), the target shifted by 0.3 along a unit vector).
    from workloads import geometric_eps_schedule
    c = make_clouds("feature64_64k", n=900, m=1300, d=160)
    eps_list = geometric_eps_schedule(2.0, 0.05, 5)
    f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), 15)
    fo, go = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], eps_list, 15)
    ef, eg = rel_inf(f, fo, eps_list[-1]), rel_inf(g, go, eps_list[-1])
    print(f"d=160 schedule: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps_list[-1], "d=160 schedule")


def test_warm_start_d64():
    c = random_clouds(600, 900, 64, seed=8, spread=0.2)
    eps = 0.1
    f1, g1 = gpu_solve(c, eps, 4)
    f2, g2 = gpu_solve(c, eps, 6, g0=g1)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 10)
    assert rel_inf(f2, fo, eps) <= TOL_POT and rel_inf(g2, go, eps) <= TOL_POT


def test_warm_start_continues_the_iteration():
    c = random_clouds(700, 900, 3, seed=2)
    eps = 0.2
    f1, g1 = gpu_solve(c, eps, 5)
    f2, g2 = gpu_solve(c, eps, 7, g0=g1)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 12)
    assert rel_inf(f2, fo) <= TOL_POT and rel_inf(g2, go) <= TOL_POT


def test_warm_start_from_shifted_g():
    # (f + c, g - c) covariance of the iteration (Birkhoff page, section 2.1)
    c = random_clouds(600, 500, 3, seed=3)
    eps, shift = 0.25, 0.75
    f1, g1 = gpu_solve(c, eps, 6)
    f2, g2 = gpu_solve(c, eps, 6, g0=np.full(500, -shift, np.float32))
    np.testing.assert_allclose(f2, f1 + shift, atol=2e-5)
    np.testing.assert_allclose(g2, g1 - shift, atol=2e-5)


@pytest.mark.parametrize("n,m,d", [(1024, 1024, 3), (65536, 4096, 3), (3000, 2000, 64),
                                   (2000, 3000, 160)])
def test_bitwise_deterministic(n, m, d):
    c = random_clouds(n, m, d, seed=4)
    f1, g1 = gpu_solve(c, 0.3, 3)
    f2, g2 = gpu_solve(c, 0.3, 3)
    np.testing.assert_array_equal(f1, f2)
    np.testing.assert_array_equal(g1, g2)
    s1 = gpu_plan_stats(c, f1, g1, 0.3)
    s2 = gpu_plan_stats(c, f1, g1, 0.3)
    assert s1 == s2


def test_plan_cost_and_marginal_error_wrappers():
    c = random_clouds(500, 400, 3, seed=5)
    f, g = gpu_solve(c, 0.3, 4)
    st = gpu_plan_stats(c, f, g, 0.3)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    ft, gt = dev(f), dev(g)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    lds.ot_plan_cost(x, y, ft, gt, 0.3, cost)
    lds.ot_marginal_error(x, y, a, b, ft, gt, 0.3, marg)
    torch.cuda.synchronize()
    assert cost.item() == st["cost"]
    assert marg[0].item() == st["marg_row"] and marg[1].item() == st["marg_col"]


def test_single_source_point_closed_form_on_gpu():
    # n = 1: after one iteration P_1j = b_j, so cost = sum_j b_j C_1j and the
    # column error is zero (closed form, independent of the oracle).
    rng = np.random.default_rng(6)
    c = {"x": rng.normal(size=(1, 3)).astype(np.float32),
         "y": rng.normal(size=(3000, 3)).astype(np.float32)}
    b = rng.dirichlet(np.ones(3000)).astype(np.float32)
    c["b"] = b
    c["a"] = np.array([b.astype(np.float64).sum()], np.float32)
    f, g = gpu_solve(c, 0.2, 2)
    st = gpu_plan_stats(c, f, g, 0.2)
    C1 = ((c["x"].astype(np.float64) - c["y"].astype(np.float64)) ** 2).sum(1)
    assert st["cost"] == pytest.approx(float(b.astype(np.float64) @ C1), rel=1e-5)
    assert st["marg_col"] < 1e-5


# --------------------------------------------------------------------------- #
# full sizes: sampled half-steps                                               #
# --------------------------------------------------------------------------- #

FULL = [("cube_gauss3d_16k", 5), ("feature64_64k", 3), ("cube_gauss3d_64k", 3)]


def _sampled_half_steps(c, eps, gK, label, seed=7, k=96):
    f1, g1 = gpu_solve(c, eps, 1, g0=gK)
    rng = np.random.default_rng(seed)
    n, m = c["x"].shape[0], c["y"].shape[0]
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, k, replace=False)]))
    cols = np.unique(np.concatenate([[0, m - 1], rng.choice(m, k, replace=False)]))
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], gK, eps, rows=rows)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f1, eps, rows=cols)
    ef, eg = rel_inf(f1[rows], f_ref), rel_inf(g1[cols], g_ref)
    print(f"{label}: sampled half-step rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF
    return f1, g1


@pytest.mark.parametrize("name,K", FULL)
def test_full_size_sampled_half_steps(name, K):
    c = make_clouds(name)
    eps = c["eps"][0]
    print(f"{name}: {K} GPU iterations", flush=True)
    _, gK = gpu_solve(c, eps, K)
    f1, g1 = _sampled_half_steps(c, eps, gK, name)
    st = gpu_plan_stats(c, f1, g1, eps)
    assert np.isfinite(st["cost"]) and st["cost"] > 0
    assert st["marg_col"] < 1e-4  # the last half-step fixed the column marginal


def test_full_size_eps_scaling_then_sampled_half_steps():
    c = make_clouds("mixture_sphere3d_eps_scaling")
    e = c["eps"]
    print("mixture full schedule on GPU", flush=True)
    f, g = gpu_solve_schedule(c, e[0], e[-1], len(e), c["iters"])
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    _sampled_half_steps(c, e[-1], g, "mixture full")


def test_full_size_plan_stats_cube_gauss3d_16k():
    c = make_clouds("cube_gauss3d_16k")
    eps = c["eps"][0]
    f, g = gpu_solve(c, eps, 20)
    st = gpu_plan_stats(c, f, g, eps)
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    print(f"16k stats: cost {st['cost']:.10g} vs {sk['cost']:.10g}; marg {st['marg']:.4e} vs "
          f"{sk['marg']:.4e}", flush=True)
    assert abs(st["cost"] - sk["cost"]) <= 1e-6 * abs(sk["cost"])
    assert abs(st["marg_row"] - sk["marg_row"]) <= 1e-6
    assert abs(st["marg_col"] - sk["marg_col"]) <= 1e-6
