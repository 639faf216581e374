"""Pins of the fp64 oracle against facts fixed outside it.

Nothing here re-types the oracle's update. Each test checks the oracle against
one of: a closed form, an invariant every iterate must satisfy, a library
routine (scipy), a different algorithm reaching the same unique solution, or
brute force on tiny inputs. The form of the update these pin is the
log-domain Sinkhorn step of "FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU" (Methodik section 1) in the convention with eps*log a
outside the log-sum-exp; the 4x4 case is the Birkhoff projection of the
"Aceleración de la Proyección de Birkhoff ..." page (sections 1, 2, 4).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment, minimize
from scipy.spatial.distance import cdist
from scipy.special import logsumexp

import oracle
from workloads import make_logits, random_clouds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_cost(x, y):
    return cdist(np.asarray(x, np.float64), np.asarray(y, np.float64), "sqeuclidean")


def dense_plan(x, y, f, g, eps):
    return np.exp((f[:, None] + g[None, :] - dense_cost(x, y)) / eps)


# --------------------------------------------------------------------------- #
# One half-step                                                                #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("eps", [1.0, 0.1, 0.003])
def test_half_step_matches_scipy_logsumexp(eps):
    c = random_clouds(37, 53, 3, seed=1)
    rng = np.random.default_rng(7)
    g = rng.normal(0, 0.3, size=53)
    f = oracle.half_update(c["x"], c["y"], c["a"], g, eps)
    C = dense_cost(c["x"], c["y"])
    ref = eps * np.log(c["a"].astype(np.float64)) - eps * logsumexp((g[None, :] - C) / eps, axis=1)
    np.testing.assert_allclose(f, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_half_step_rows_subset_matches_full():
    c = random_clouds(50, 41, 5, seed=2)
    g = np.linspace(-0.2, 0.2, 41)
    full = oracle.half_update(c["x"], c["y"], c["a"], g, 0.2)
    rows = np.array([49, 0, 17, 17, 3])
    np.testing.assert_array_equal(oracle.half_update(c["x"], c["y"], c["a"], g, 0.2, rows=rows),
                                  full[rows])


def test_half_step_survives_extreme_exponents():
    # exp(-C/eps) underflows to 0 for every j in naive arithmetic here; the
    # max-subtracted log-sum-exp must still be finite and exact.
    x = np.array([[0.0, 0.0, 0.0], [10.0, 0.0, 0.0]])
    y = np.array([[3.0, 0.0, 0.0], [4.0, 0.0, 0.0], [-5.0, 1.0, 0.0]])
    a = np.array([0.5, 0.5])
    g = np.zeros(3)
    eps = 1e-3
    f = oracle.half_update(x, y, a, g, eps)
    C = dense_cost(x, y)
    ref = eps * np.log(a) - eps * logsumexp(-C / eps, axis=1)
    assert np.all(np.isfinite(f))
    np.testing.assert_allclose(f, ref, rtol=1e-13)
    # As eps -> 0 the soft-min becomes the min: f_i -> min_j C_ij.
    np.testing.assert_allclose(f, C.min(axis=1), atol=20 * eps)


# --------------------------------------------------------------------------- #
# Marginal invariants: each half-step is the unique scaling that makes its    #
# side's marginal exact.                                                       #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("K", [1, 2, 7])
def test_each_half_step_makes_its_marginal_exact(K):
    c = random_clouds(23, 31, 4, seed=3)
    eps = 0.25
    # state after K-1 iterations, then the f half-step, then the g half-step
    f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, K - 1)
    f_new = oracle.half_update(c["x"], c["y"], c["a"], g, eps)
    P_half = dense_plan(c["x"], c["y"], f_new, g, eps)
    np.testing.assert_allclose(P_half.sum(axis=1), c["a"].astype(np.float64), rtol=1e-12)
    f_k, g_k = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, K)
    np.testing.assert_allclose(f_k, f_new, rtol=0, atol=1e-14)
    P = dense_plan(c["x"], c["y"], f_k, g_k, eps)
    np.testing.assert_allclose(P.sum(axis=0), c["b"].astype(np.float64), rtol=1e-12)


def test_iters_zero_leaves_potentials():
    c = random_clouds(5, 6, 2, seed=4)
    f0 = np.arange(5.0)
    g0 = -np.arange(6.0)
    f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], 0.3, 0, f0, g0)
    np.testing.assert_array_equal(f, f0)
    np.testing.assert_array_equal(g, g0)


# --------------------------------------------------------------------------- #
# Closed forms                                                                 #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("K", [1, 3])
def test_single_source_point_closed_form(K):
    # n = 1: g_j = eps log b_j + C_1j - f_1 and P_1j = b_j after every
    # iteration; with a_1 = sum b the potentials are a fixed point.
    rng = np.random.default_rng(5)
    x = rng.normal(size=(1, 3))
    y = rng.normal(size=(17, 3))
    b = rng.dirichlet(np.ones(17))
    a = np.array([b.sum()])
    eps = 0.2
    f, g = oracle.sinkhorn(x, y, a, b, eps, K)
    C1 = dense_cost(x, y)[0]
    f1 = eps * math.log(a[0]) - eps * logsumexp(-C1 / eps)  # first f from g = 0
    assert f[0] == pytest.approx(f1, rel=1e-13, abs=1e-13)
    np.testing.assert_allclose(g, eps * np.log(b) + C1 - f[0], rtol=1e-12, atol=1e-13)
    P = dense_plan(x, y, f, g, eps)[0]
    np.testing.assert_allclose(P, b, rtol=1e-12)
    st = oracle.plan_stats(x, y, a, b, f, g, eps)
    assert st["cost"] == pytest.approx(float(b @ C1), rel=1e-12)
    assert st["marg"] == pytest.approx(0.0, abs=1e-14)


def test_single_target_point_closed_form():
    # m = 1, cold start: f_i = eps log a_i + C_i1, g_1 = eps log b_1 - eps log sum a,
    # P_i1 = a_i b_1 / sum a.
    rng = np.random.default_rng(6)
    x = rng.normal(size=(13, 2))
    y = rng.normal(size=(1, 2))
    a = rng.dirichlet(np.ones(13)) * 0.7
    b = np.array([0.7])
    eps = 0.05
    f, g = oracle.sinkhorn(x, y, a, b, eps, 1)
    C = dense_cost(x, y)[:, 0]
    np.testing.assert_allclose(f, eps * np.log(a) + C, rtol=1e-12)
    assert g[0] == pytest.approx(eps * math.log(b[0]) - eps * math.log(a.sum()), abs=1e-13)
    np.testing.assert_allclose(dense_plan(x, y, f, g, eps)[:, 0], a * b[0] / a.sum(), rtol=1e-11)


def test_large_eps_gives_product_coupling():
    # eps -> infinity: P -> a b^T and <P, C> -> sum a|x|^2 + sum b|y|^2 - 2 (sum a x).(sum b y).
    c = random_clouds(40, 30, 3, seed=8)
    a, b = c["a"].astype(np.float64), c["b"].astype(np.float64)
    a, b = a / a.sum(), b / b.sum()
    x, y = c["x"].astype(np.float64), c["y"].astype(np.float64)
    eps = 1e7
    f, g = oracle.sinkhorn(x, y, a, b, eps, 3)
    P = dense_plan(x, y, f, g, eps)
    np.testing.assert_allclose(P, np.outer(a, b), rtol=1e-5)
    closed = a @ (x * x).sum(1) + b @ (y * y).sum(1) - 2 * (a @ x) @ (b @ y)
    st = oracle.plan_stats(x, y, a, b, f, g, eps)
    assert st["cost"] == pytest.approx(closed, rel=1e-5)


# --------------------------------------------------------------------------- #
# The pages' own form of the update and the dual shift                         #
# --------------------------------------------------------------------------- #

def test_matches_page_form_with_log_b_inside():
    # FlashSinkhorn, Methodik 1, writes f_i <- -eps LSE_j[(g_j - C_ij)/eps + log b_j]
    # (and the symmetric g with log a_i). That iteration, started from
    # g' = -eps log b, must give the same plan as the oracle's form, with
    # f = f' + eps log a and g = g' + eps log b at every iteration.
    c = random_clouds(19, 26, 3, seed=9)
    x, y = c["x"].astype(np.float64), c["y"].astype(np.float64)
    a, b = c["a"].astype(np.float64), c["b"].astype(np.float64)
    eps = 0.15
    C = dense_cost(x, y)
    gp = -eps * np.log(b)
    for K in range(1, 6):
        fp = -eps * logsumexp((gp[None, :] - C) / eps + np.log(b)[None, :], axis=1)
        gp = -eps * logsumexp((fp[:, None] - C) / eps + np.log(a)[:, None], axis=0)
        f, g = oracle.sinkhorn(x, y, a, b, eps, K)
        np.testing.assert_allclose(f, fp + eps * np.log(a), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g, gp + eps * np.log(b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shift", [0.37, -2.5])
def test_shift_covariance(shift):
    # Potentials are defined up to (f + c, g - c) (Birkhoff page, section 2.1):
    # starting from g0 - c gives (f + c, g - c) at every iteration, same plan.
    c = random_clouds(14, 11, 3, seed=10)
    eps = 0.3
    g0 = np.linspace(-0.1, 0.2, 11)
    f1, g1 = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6, g0=g0)
    f2, g2 = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6, g0=g0 - shift)
    np.testing.assert_allclose(f2, f1 + shift, atol=1e-12)
    np.testing.assert_allclose(g2, g1 - shift, atol=1e-12)
    np.testing.assert_allclose(dense_plan(c["x"], c["y"], f2, g2, eps),
                               dense_plan(c["x"], c["y"], f1, g1, eps), rtol=1e-11)


# --------------------------------------------------------------------------- #
# Fixed point: a different algorithm (Newton on the dual) reaches the same    #
# unique entropic plan                                                         #
# --------------------------------------------------------------------------- #

def dual_newton_plan(C, a, b, eps):
    n, m = C.shape

    def split(z):
        return z[:n], np.concatenate([z[n:], [0.0]])  # g_m = 0 removes the shift

    def fun(z):
        f, g = split(z)
        P = np.exp((f[:, None] + g[None, :] - C) / eps)
        val = -(a @ f + b @ g - eps * P.sum())
        grad = np.concatenate([P.sum(1) - a, (P.sum(0) - b)[:-1]])
        return val, grad

    def hess(z):
        f, g = split(z)
        P = np.exp((f[:, None] + g[None, :] - C) / eps)
        H = np.zeros((n + m - 1, n + m - 1))
        H[:n, :n] = np.diag(P.sum(1))
        H[n:, n:] = np.diag(P.sum(0)[:-1])
        H[:n, n:] = P[:, :-1]
        H[n:, :n] = P[:, :-1].T
        return H / eps

    res = minimize(fun, np.zeros(n + m - 1), jac=True, hess=hess, method="trust-exact",
                   options={"gtol": 1e-14, "maxiter": 500})
    f, g = split(res.x)
    return np.exp((f[:, None] + g[None, :] - C) / eps)


@pytest.mark.parametrize("eps", [1.0, 0.3])
def test_converged_plan_equals_dual_newton_plan(eps):
    c = random_clouds(12, 9, 3, seed=11)
    a, b = c["a"].astype(np.float64), c["b"].astype(np.float64)
    a, b = a / a.sum(), b / b.sum()
    f, g = oracle.sinkhorn(c["x"], c["y"], a, b, eps, 3000)
    P = dense_plan(c["x"], c["y"], f, g, eps)
    Pn = dual_newton_plan(dense_cost(c["x"], c["y"]), a, b, eps)
    np.testing.assert_allclose(P, Pn, atol=1e-10 * Pn.max())
    st = oracle.plan_stats(c["x"], c["y"], a, b, f, g, eps)
    assert st["marg"] < 1e-10


# --------------------------------------------------------------------------- #
# eps -> 0: exact OT by brute force / assignment / 1-D sorting                 #
# --------------------------------------------------------------------------- #

def _small_eps_solve(x, y, a, b, eps_end):
    eps_list = np.geomspace(1.0, eps_end, 25)
    return oracle.sinkhorn_schedule(x, y, a, b, eps_list, 400)


def _check_entropic_bound(x, y, ot, eps_end, n):
    a = np.full(n, 1.0 / n)
    f, g = _small_eps_solve(x, y, a, a, eps_end)
    st = oracle.plan_stats(x, y, a, a, f, g, eps_end)
    slack = st["marg"] * dense_cost(x, y).max()
    assert st["cost"] >= ot - slack - 1e-12
    assert st["cost"] <= ot + eps_end * math.log(n) + slack + 1e-12
    return f, g


@pytest.mark.parametrize("n", [3, 5, 7])
def test_small_eps_brute_force_permutations(n):
    rng = np.random.default_rng(100 + n)
    x = rng.normal(size=(n, 2))
    y = rng.normal(size=(n, 2))
    C = dense_cost(x, y)
    costs = {p: C[np.arange(n), list(p)].mean() for p in itertools.permutations(range(n))}
    best = min(costs, key=costs.get)
    f, g = _check_entropic_bound(x, y, costs[best], 2e-3, n)
    # The plan concentrates on the optimal permutation.
    P = dense_plan(x, y, f, g, 2e-3)
    assert list(P.argmax(axis=1)) == list(best)


def test_small_eps_assignment():
    n = 40
    rng = np.random.default_rng(12)
    x = rng.normal(size=(n, 3))
    y = rng.normal(size=(n, 3))
    C = dense_cost(x, y)
    r, cidx = linear_sum_assignment(C)
    _check_entropic_bound(x, y, C[r, cidx].mean(), 2e-3, n)


def test_small_eps_one_dimension_sorted_matching():
    n = 64
    rng = np.random.default_rng(13)
    x = rng.normal(size=(n, 1))
    y = rng.uniform(-1, 2, size=(n, 1))
    ot = np.mean((np.sort(x[:, 0]) - np.sort(y[:, 0])) ** 2)
    _check_entropic_bound(x, y, ot, 2e-3, n)


# --------------------------------------------------------------------------- #
# Stages (warm start)                                                          #
# --------------------------------------------------------------------------- #

def test_stage_composition_equals_longer_run():
    c = random_clouds(16, 21, 3, seed=14)
    f1, g1 = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], 0.2, 5)
    f2, g2 = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], 0.2, 7, f1, g1)
    f3, g3 = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], 0.2, 12)
    np.testing.assert_array_equal(f2, f3)
    np.testing.assert_array_equal(g2, g3)
    f4, g4 = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], [0.2, 0.2], 6)
    np.testing.assert_array_equal(f4, f3)
    np.testing.assert_array_equal(g4, g3)


def test_schedule_converges_to_final_eps_fixed_point():
    c = random_clouds(10, 8, 3, seed=15)
    a, b = c["a"].astype(np.float64), c["b"].astype(np.float64)
    a, b = a / a.sum(), b / b.sum()
    f, g = oracle.sinkhorn_schedule(c["x"], c["y"], a, b, [2.0, 1.0, 0.5], 2000)
    P = dense_plan(c["x"], c["y"], f, g, 0.5)
    np.testing.assert_allclose(P, dual_newton_plan(dense_cost(c["x"], c["y"]), a, b, 0.5),
                               atol=1e-10)


# --------------------------------------------------------------------------- #
# plan statistics                                                              #
# --------------------------------------------------------------------------- #

def test_plan_stats_single_target_unbalanced_closed_form():
    # m = 1 with b_1 != sum a, one iteration from g = 0: the f step makes
    # P_i1 = a_i, the g step rescales the column to b_1, so
    # P_i1 = a_i b_1 / sum a. Row sums miss a_i by a_i (b_1/sum a - 1), all of
    # one sign: the row L1 error is |b_1 - sum a| exactly, while an L-inf or
    # squared reduction of the same deviations gives a different number for
    # non-uniform a. The column is exact after the g step.
    rng = np.random.default_rng(40)
    x = rng.normal(size=(9, 3))
    y = rng.normal(size=(1, 3))
    a = rng.dirichlet(np.ones(9))
    b = np.array([0.6])
    eps = 0.3
    f, g = oracle.sinkhorn(x, y, a, b, eps, 1)
    st = oracle.plan_stats(x, y, a, b, f, g, eps)
    np.testing.assert_allclose(st["rowsum"], a * b[0] / a.sum(), rtol=1e-12)
    assert st["marg_row"] == pytest.approx(abs(b[0] - a.sum()), rel=1e-12)
    dev = np.abs(a * b[0] / a.sum() - a)
    assert abs(st["marg_row"] - dev.max()) > 0.1 * dev.sum()   # not L-inf
    assert abs(st["marg_row"] - (dev**2).sum()) > 0.1 * dev.sum()  # not squared
    assert st["marg_col"] == pytest.approx(0.0, abs=1e-14)
    assert st["marg"] == pytest.approx(st["marg_row"] + st["marg_col"], rel=1e-15)
    C = dense_cost(x, y)[:, 0]
    assert st["cost"] == pytest.approx(float((a * b[0] / a.sum()) @ C), rel=1e-12)


def test_plan_stats_single_target_after_f_step_only():
    # m = 1 after an f half-step alone (any g): P_i1 = a_i, so the row error is
    # zero and the column sum is sum a: column L1 error |sum a - b_1|.
    rng = np.random.default_rng(41)
    x = rng.normal(size=(11, 2))
    y = rng.normal(size=(1, 2))
    a = rng.dirichlet(np.ones(11))
    b = np.array([1.7])
    eps = 0.25
    g = np.array([0.37])
    f = oracle.half_update(x, y, a, g, eps)
    st = oracle.plan_stats(x, y, a, b, f, g, eps)
    assert st["marg_row"] == pytest.approx(0.0, abs=1e-14)
    assert st["marg_col"] == pytest.approx(abs(a.sum() - b[0]), rel=1e-12)
    np.testing.assert_allclose(st["colsum"], [a.sum()], rtol=1e-13)


def test_plan_stats_column_errors_of_mixed_sign_closed_form():
    # n = 1 at the origin, targets at +-1 on a line: every cost is exactly 1.
    # After an f half-step from g = 0 the plan is P_1j = a_1 / m, so the
    # column sums miss the Dirichlet b_j with both signs and the column L1
    # error is sum_j |a_1/m - b_j|; the row error is zero.
    rng = np.random.default_rng(42)
    m = 12
    x = np.zeros((1, 1))
    y = np.where(np.arange(m) % 2 == 0, 1.0, -1.0).reshape(m, 1)
    a = np.array([1.0])
    b = rng.dirichlet(np.ones(m))
    eps = 0.4
    f = oracle.half_update(x, y, a, np.zeros(m), eps)
    st = oracle.plan_stats(x, y, a, b, f, np.zeros(m), eps)
    dev = np.abs(a[0] / m - b)
    assert (a[0] / m - b).min() < 0 < (a[0] / m - b).max()  # both signs present
    assert st["marg_col"] == pytest.approx(dev.sum(), rel=1e-12)
    assert st["marg_row"] == pytest.approx(0.0, abs=1e-14)
    np.testing.assert_allclose(st["colsum"], np.full(m, a[0] / m), rtol=1e-13)
    assert st["cost"] == pytest.approx(1.0, rel=1e-13)


def test_plan_stats_row_errors_of_mixed_sign_closed_form():
    # m = 1 at the origin, sources at +-1 on a line (every cost 1), row
    # potentials f_i = eps log w_i: the g half-step gives
    # P_i1 = b_1 w_i / sum w, so the row L1 error is sum_i |b_1 w_i/sum w - a_i|
    # (deviations of both signs) and the column error is zero.
    rng = np.random.default_rng(43)
    n = 10
    x = np.where(np.arange(n) % 3 == 0, 1.0, -1.0).reshape(n, 1)
    y = np.zeros((1, 1))
    a = rng.dirichlet(np.ones(n))
    w = rng.dirichlet(np.ones(n))
    b = np.array([1.0])
    eps = 0.15
    f = eps * np.log(w)
    g = oracle.half_update(y, x, b, f, eps)
    st = oracle.plan_stats(x, y, a, b, f, g, eps)
    P = b[0] * w / w.sum()
    assert (P - a).min() < 0 < (P - a).max()
    np.testing.assert_allclose(st["rowsum"], P, rtol=1e-12)
    assert st["marg_row"] == pytest.approx(np.abs(P - a).sum(), rel=1e-12)
    assert st["marg_col"] == pytest.approx(0.0, abs=1e-14)
    assert st["cost"] == pytest.approx(1.0, rel=1e-13)


def test_plan_stats_column_marginal_exact_after_g_step():
    c = random_clouds(30, 25, 3, seed=16)
    f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], 0.4, 4)
    st = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, 0.4)
    assert st["marg_col"] < 1e-14
    assert st["marg_row"] > 1e-8  # not converged after 4 iterations
    np.testing.assert_allclose(st["colsum"], c["b"], rtol=1e-12)


# --------------------------------------------------------------------------- #
# 4x4 Birkhoff projection                                                       #
# --------------------------------------------------------------------------- #

def test_birkhoff_converged_doubly_stochastic():
    L = make_logits(256, (1.0, 3.0), seed=17)
    P, it = oracle.birkhoff4(L, 1.0, 5000, 1e-12)
    assert np.all(it < 5000)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, atol=1e-12)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)


@pytest.mark.parametrize("iters", [1, 20])
def test_birkhoff_cross_ratio_invariant(iters):
    # Every iterate is diag(u) exp(L/eps) diag(v), so the cross ratios of P are
    # those of exp(L/eps), whatever the iteration count.
    L = make_logits(64, (1.0, 10.0), seed=18).astype(np.float64)
    eps = 1.0
    P, _ = oracle.birkhoff4(L, eps, iters, -1.0)
    for i, k in [(0, 1), (2, 3), (0, 3)]:
        for j, l in [(0, 2), (1, 3), (1, 2)]:
            lhs = np.log(P[:, i, j]) + np.log(P[:, k, l]) - np.log(P[:, i, l]) - np.log(P[:, k, j])
            rhs = (L[:, i, j] + L[:, k, l] - L[:, i, l] - L[:, k, j]) / eps
            assert np.all(np.abs(lhs - rhs) <= 1e-9 * (1 + np.abs(rhs)))


def test_birkhoff_constant_logits():
    L = np.full((3, 4, 4), 2.5)
    P, it = oracle.birkhoff4(L, 1.0, 200, 1e-6)
    np.testing.assert_allclose(P, 0.25, rtol=1e-14)
    assert list(it) == [1, 1, 1]


def test_birkhoff_circulant_exact_after_one_iteration():
    # A circulant exp(L) has equal row and column sums, so the first f step
    # already gives a doubly-stochastic plan: K / rowsum.
    c = np.array([0.3, -1.2, 2.0, 0.7])
    L = np.array([[c[(j - i) % 4] for j in range(4)] for i in range(4)])[None]
    P, it = oracle.birkhoff4(L, 1.0, 200, 1e-12)
    K = np.exp(L[0])
    np.testing.assert_allclose(P[0], K / K.sum(axis=1, keepdims=True), rtol=1e-13)
    assert it[0] == 1


def test_birkhoff_dominant_permutation():
    perm = [2, 0, 3, 1]
    L = np.zeros((1, 4, 4))
    L[0, np.arange(4), perm] = 30.0
    P, _ = oracle.birkhoff4(L, 1.0, 200, 1e-9)
    Pi = np.zeros((4, 4))
    Pi[np.arange(4), perm] = 1.0
    np.testing.assert_allclose(P[0], Pi, atol=1e-9)


def test_birkhoff_limit_matches_dual_newton():
    # Sinkhorn's theorem: the limit is the unique doubly-stochastic matrix of
    # the form diag(u) exp(L) diag(v); Newton on the 4x4 dual finds it too.
    L = make_logits(6, (1.0, 4.0), seed=19).astype(np.float64)
    P, _ = oracle.birkhoff4(L, 1.0, 20000, 1e-14)
    for k in range(L.shape[0]):
        Pn = dual_newton_plan(-L[k], np.ones(4), np.ones(4), 1.0)
        np.testing.assert_allclose(P[k], Pn, atol=1e-11)


def test_birkhoff_stopping_rule_is_first_crossing():
    L = make_logits(512, (1.0, 10.0), seed=20)
    tol = 1e-6
    P, it = oracle.birkhoff4(L, 1.0, 200, tol)
    Pr, err = oracle.birkhoff4_replay(L, it, 1.0)
    np.testing.assert_array_equal(P, Pr)
    conv = it < 200
    assert np.all(err[conv] <= tol)
    assert conv.sum() > 100
    prev = np.maximum(it - 1, 0)
    _, err_prev = oracle.birkhoff4_replay(L, prev, 1.0)
    assert np.all(err_prev[conv & (it > 1)] > tol)


def test_birkhoff_fixed20_sigma_split():
    claim = {c["id"]: c for c in json.load(open(os.path.join(GOLDEN, "page_claims.json")))["claims"]}
    ratio_min = claim["birkhoff_fixed20_sigma"]["min_median_ratio"]
    L = make_logits(4096, (1.0, 10.0), seed=21)
    P, it = oracle.birkhoff4(L, 1.0, 20, -1.0)
    assert np.all(it == 20)
    err = np.maximum(np.abs(P.sum(2) - 1).max(1), np.abs(P.sum(1) - 1).max(1))
    med1 = np.median(err[:2048])
    med10 = np.median(err[2048:])
    assert med10 > ratio_min * med1


# --------------------------------------------------------------------------- #
# Cosine cost (FlashSinkhorn page, significance section)                       #
# --------------------------------------------------------------------------- #

def _cos_cost(x, y):
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return 1.0 - (x @ y.T) / (np.linalg.norm(x, axis=1)[:, None] * np.linalg.norm(y, axis=1)[None])


def test_cosine_first_half_step_matches_scipy():
    c = random_clouds(31, 44, 5, seed=60)
    eps = 0.07
    g0 = np.random.default_rng(61).normal(0, 0.1, size=44)
    f, _ = oracle.sinkhorn_cosine(c["x"], c["y"], c["a"], c["b"], eps, 1, g0=g0)
    # after one iteration f is the half-step from g0 (the g half-step follows)
    ref = eps * np.log(c["a"].astype(np.float64)) - eps * logsumexp(
        (g0[None, :] - _cos_cost(c["x"], c["y"])) / eps, axis=1)
    np.testing.assert_allclose(f, ref, rtol=1e-12, atol=1e-13)


def test_cosine_unit_sphere_equals_half_sqeuclid_at_twice_eps():
    # On unit vectors 1 - cos = |x - y|^2 / 2, so the cosine problem at eps is
    # the squared Euclidean one at 2 eps with potentials doubled.
    c = random_clouds(40, 35, 6, seed=62)
    xs = c["x"] / np.linalg.norm(c["x"].astype(np.float64), axis=1, keepdims=True)
    ys = c["y"] / np.linalg.norm(c["y"].astype(np.float64), axis=1, keepdims=True)
    eps = 0.05
    fc, gc = oracle.sinkhorn_cosine(xs, ys, c["a"], c["b"], eps, 30)
    fq, gq = oracle.sinkhorn(xs, ys, c["a"], c["b"], 2 * eps, 30)
    np.testing.assert_allclose(fc, fq / 2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(gc, gq / 2, rtol=1e-11, atol=1e-12)
    sc = oracle.plan_stats_cosine(xs, ys, c["a"], c["b"], fc, gc, eps)
    sq = oracle.plan_stats(xs, ys, c["a"], c["b"], fq, gq, 2 * eps)
    assert sc["cost"] == pytest.approx(sq["cost"] / 2, rel=1e-11)
    assert sc["marg"] == pytest.approx(sq["marg"], rel=1e-8, abs=1e-14)


def test_cosine_scale_and_rotation_invariance():
    c = random_clouds(25, 30, 4, seed=63)
    rng = np.random.default_rng(64)
    Q, _ = np.linalg.qr(rng.normal(size=(4, 4)))
    sx = rng.uniform(0.1, 10.0, size=(25, 1))
    sy = rng.uniform(0.1, 10.0, size=(30, 1))
    f0, g0 = oracle.sinkhorn_cosine(c["x"], c["y"], c["a"], c["b"], 0.1, 20)
    f1, g1 = oracle.sinkhorn_cosine((c["x"] * sx) @ Q, (c["y"] * sy) @ Q, c["a"], c["b"], 0.1, 20)
    np.testing.assert_allclose(f1, f0, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(g1, g0, rtol=1e-10, atol=1e-11)


def test_cosine_single_source_and_cost_range():
    rng = np.random.default_rng(65)
    x = rng.normal(size=(1, 8))
    y = rng.normal(size=(50, 8))
    b = rng.dirichlet(np.ones(50))
    a = np.array([b.sum()])
    f, g = oracle.sinkhorn_cosine(x, y, a, b, 0.3, 2)
    st = oracle.plan_stats_cosine(x, y, a, b, f, g, 0.3)
    C = _cos_cost(x, y)[0]
    assert st["cost"] == pytest.approx(float(b @ C), rel=1e-12)   # P_1j = b_j
    assert st["marg"] < 1e-12
    assert np.all(C >= 0) and np.all(C <= 2)


# --------------------------------------------------------------------------- #
# 4x4 projection by Newton's method on the dual, and its backward             #
# (Birkhoff page, sections 2.1 and 2.2)                                        #
# --------------------------------------------------------------------------- #

def test_newton_limit_matches_long_sinkhorn():
    # Sinkhorn's theorem: one doubly-stochastic matrix of the form
    # diag(u) exp(L/eps) diag(v); Sinkhorn-Knopp (a different algorithm)
    # reaches it after enough iterations.
    L = make_logits(64, (1.0, 2.0), seed=40)
    for eps in (1.0, 0.5):
        Pn, it = oracle.birkhoff4_newton(L, eps, 100, 1e-13)
        Ps, its = oracle.birkhoff4(L, eps, 1000000, 1e-13)
        assert np.all(it < 100) and np.all(its < 1000000)
        np.testing.assert_allclose(Pn, Ps, atol=1e-10)


def test_newton_plan_structure_and_marginals():
    L = make_logits(256, (1.0, 10.0), seed=41).astype(np.float64)
    P, it = oracle.birkhoff4_newton(L, 1.0, 100, 1e-12)
    assert np.all(it < 100)
    np.testing.assert_allclose(P.sum(axis=2), 1.0, atol=1e-13)   # rows exact by construction
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)   # columns to tol
    # every plan is diag(u) exp(L) diag(v): cross ratios are those of exp(L)
    for (i, k), (j, l) in [((0, 1), (0, 2)), ((2, 3), (1, 3)), ((0, 3), (1, 2))]:
        lhs = np.log(P[:, i, j]) + np.log(P[:, k, l]) - np.log(P[:, i, l]) - np.log(P[:, k, j])
        rhs = L[:, i, j] + L[:, k, l] - L[:, i, l] - L[:, k, j]
        assert np.all(np.abs(lhs - rhs) <= 1e-8 * (1 + np.abs(rhs)))


def test_newton_constant_and_circulant_need_no_step():
    # Constant or circulant logits: the first row softmax (g = 0) already has
    # unit column sums, so no Newton step is taken.
    c = np.array([0.3, -1.2, 2.0, 0.7])
    circ = np.array([[c[(j - i) % 4] for j in range(4)] for i in range(4)])
    L = np.stack([np.full((4, 4), -3.0), circ])
    P, it = oracle.birkhoff4_newton(L, 1.0, 50, 1e-13)
    assert list(it) == [0, 0]
    np.testing.assert_allclose(P[0], 0.25, rtol=1e-14)
    K = np.exp(circ)
    np.testing.assert_allclose(P[1], K / K.sum(axis=1, keepdims=True), rtol=1e-13)


def test_newton_converges_quadratically():
    # Quadratic convergence at the end: the step that reaches 1e-12 starts
    # from an error below 1e-5 (a linearly converging method with the
    # observed early contraction, ~0.4 per step, would need ~1e-12 there).
    # Large-magnitude logits (N(0, 10^2)) converge in few steps where 20
    # Sinkhorn-Knopp iterations do not.
    L = make_logits(512, (1.0, 10.0), seed=42)
    P, it12 = oracle.birkhoff4_newton(L, 1.0, 200, 1e-12)
    assert np.max(it12) <= 40 and np.median(it12[256:]) <= 12
    for k in range(0, 512, 8):
        if it12[k] == 0:
            continue
        Pk, _ = oracle.birkhoff4_newton(L[k:k + 1], 1.0, int(it12[k]) - 1, -1.0)
        assert np.abs(Pk.sum(1) - 1).max() <= 1e-5
    P20, _ = oracle.birkhoff4(L[256:], 1.0, 20, -1.0)   # columns exact after its g step
    err20 = np.abs(P20.sum(2) - 1).max(1)
    assert np.median(err20) > 1e-6 and np.median(it12[256:]) < 20


def _loss_of_logits(L, G, eps):
    P, it = oracle.birkhoff4(L, eps, 200000, 1e-15)
    return float((P * G).sum())


@pytest.mark.parametrize("eps,sigma", [(1.0, 1.0), (0.5, 2.0), (1.0, 4.0)])
def test_backward_matches_finite_differences(eps, sigma):
    rng = np.random.default_rng(43)
    L = rng.normal(0.0, sigma, size=(1, 4, 4))
    G = rng.normal(size=(1, 4, 4))
    P, _ = oracle.birkhoff4_newton(L, eps, 100, 1e-14)
    grad = oracle.birkhoff4_backward(P, G, eps)[0]
    h = 1e-5
    fd = np.empty((4, 4))
    for i in range(4):
        for j in range(4):
            Lp, Lm = L.copy(), L.copy()
            Lp[0, i, j] += h
            Lm[0, i, j] -= h
            fd[i, j] = (_loss_of_logits(Lp, G, eps) - _loss_of_logits(Lm, G, eps)) / (2 * h)
    np.testing.assert_allclose(grad, fd, atol=1e-7 * (1 + np.abs(fd).max()))


def test_backward_row_and_column_sums_vanish():
    # Adding a constant to a row or a column of L leaves the projection
    # unchanged, so dl/dL has zero row and column sums.
    L = make_logits(128, (1.0, 5.0), seed=44)
    rng = np.random.default_rng(45)
    G = rng.normal(size=L.shape)
    P, _ = oracle.birkhoff4_newton(L, 1.0, 100, 1e-14)
    gL = oracle.birkhoff4_backward(P, G, 1.0)
    scale = np.abs(gL).max(axis=(1, 2))
    assert np.all(np.abs(gL.sum(axis=2)).max(axis=1) <= 1e-10 * (1 + scale))
    assert np.all(np.abs(gL.sum(axis=1)).max(axis=1) <= 1e-9 * (1 + scale))


# --------------------------------------------------------------------------- #
# Transport application (FlashSinkhorn page, Methodik section 3)               #
# --------------------------------------------------------------------------- #

def test_transport_apply_single_source_closed_form():
    # n = 1 after an iteration: P_1j = b_j, so sum_j P_1j v_j = sum_j b_j v_j.
    rng = np.random.default_rng(30)
    x = rng.normal(size=(1, 3))
    y = rng.normal(size=(23, 3))
    b = rng.dirichlet(np.ones(23))
    a = np.array([b.sum()])
    f, g = oracle.sinkhorn(x, y, a, b, 0.3, 2)
    v = rng.normal(size=(23, 4))
    np.testing.assert_allclose(oracle.transport_apply(x, y, f, g, 0.3, v)[0], b @ v, rtol=1e-12)
    np.testing.assert_allclose(oracle.barycentric_map(x, y, a, f, g, 0.3)[0], (b @ y) / a[0],
                               rtol=1e-12)


def test_transport_apply_product_coupling_limit():
    c = random_clouds(20, 15, 3, seed=31)
    a, b = c["a"].astype(np.float64), c["b"].astype(np.float64)
    a, b = a / a.sum(), b / b.sum()
    eps = 1e7
    f, g = oracle.sinkhorn(c["x"], c["y"], a, b, eps, 3)
    v = np.random.default_rng(32).normal(size=(15, 2))
    np.testing.assert_allclose(oracle.transport_apply(c["x"], c["y"], f, g, eps, v),
                               np.outer(a, b @ v), rtol=1e-5, atol=1e-12)


def test_transport_apply_of_ones_is_the_row_marginal_after_an_f_step():
    c = random_clouds(17, 21, 3, seed=33)
    eps = 0.2
    f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 3)
    f_new = oracle.half_update(c["x"], c["y"], c["a"], g, eps)
    np.testing.assert_allclose(oracle.transport_apply(c["x"], c["y"], f_new, g, eps, np.ones(21)),
                               c["a"], rtol=1e-12)


def test_barycentric_map_small_eps_is_the_optimal_matching():
    n = 5
    rng = np.random.default_rng(34)
    x = rng.normal(size=(n, 2))
    y = rng.normal(size=(n, 2))
    C = dense_cost(x, y)
    best = min(itertools.permutations(range(n)), key=lambda p: C[np.arange(n), list(p)].sum())
    a = np.full(n, 1.0 / n)
    eps = 2e-3
    f, g = _small_eps_solve(x, y, a, a, eps)
    T = oracle.barycentric_map(x, y, a, f, g, eps)
    np.testing.assert_allclose(T, y[list(best)], atol=1e-3)


def _entropic_value(x, y, a, b, eps, iters=4000):
    f, g = oracle.sinkhorn(x, y, a, b, eps, iters)
    return a @ f + b @ g, f, g


def test_grad_x_matches_finite_differences_of_the_entropic_value():
    # Envelope theorem: at the optimum, d/dx_i OT_eps = 2 sum_j P_ij (x_i - y_j).
    rng = np.random.default_rng(35)
    x = rng.normal(size=(6, 2))
    y = rng.normal(size=(5, 2))
    a = rng.dirichlet(np.ones(6))
    b = rng.dirichlet(np.ones(5))
    eps = 0.5
    _, f, g = _entropic_value(x, y, a, b, eps)
    G = oracle.grad_x(x, y, f, g, eps)
    h = 1e-5
    for i, k in [(0, 0), (3, 1), (5, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        fd = (_entropic_value(xp, y, a, b, eps)[0] - _entropic_value(xm, y, a, b, eps)[0]) / (2 * h)
        assert G[i, k] == pytest.approx(fd, rel=1e-6, abs=1e-9)
