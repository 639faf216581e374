"""GPU parity of the 4x4 projection by Newton's method on the dual and of its
implicit-differentiation backward, against the fp64 oracle.

Page: "Aceleración de la Proyección de Birkhoff para Hiper-conexiones con
Restricción de Variedad", section 2.1 (Newton on the 3-variable dual,
closed-form gradient and Hessian, max subtraction), section 2.2 (implicit
differentiation with the last Newton step's matrix), section 4 (N(0, 1) and
N(0, 10^2) inputs).

The projection is unique, so the GPU's plan (stopped at tol = 1e-6 on its
fp32 output) is compared with the oracle's converged one (1e-13): the
difference is bounded by the stopping tolerance, not by the iteration count.
The backward is compared on identical fp32 plans: both sides compute in
fp64, the GPU rounds the result to fp32.
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import make_logits

from gpu_helpers import DEV, TOL_P4, dev, gpu_birkhoff

pytestmark = pytest.mark.gpu

# Newton plan vs the converged projection: stopping tol 1e-6 on sums of four
# entries bounds each entry's distance to the solution by a few tol for
# well-conditioned plans; 1e-5 as for the Sinkhorn plans.
TOL_NEWTON = TOL_P4


def gpu_newton(L, eps, max_iters, tol, inplace=False):
    t = dev(np.ascontiguousarray(L, np.float32))
    out = t if inplace else torch.empty_like(t)
    it = torch.empty(t.shape[0], dtype=torch.int32, device=DEV)
    lds.ot_birkhoff_project_newton_batched(t, eps, max_iters, tol, out, it)
    torch.cuda.synchronize()
    return out.cpu().numpy(), it.cpu().numpy()


def gpu_backward(P, G, eps):
    p = dev(np.ascontiguousarray(P, np.float32))
    g = dev(np.ascontiguousarray(G, np.float32))
    out = torch.empty_like(p)
    lds.ot_birkhoff_projection_backward_batched(p, g, eps, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _err(P):
    P = np.asarray(P, np.float64)
    return np.maximum(np.abs(P.sum(2) - 1).max(1), np.abs(P.sum(1) - 1).max(1))


@pytest.mark.parametrize("batch,sigmas,eps", [(1, (1.0,), 1.0), (65, (1.0, 10.0), 1.0),
                                              (8192, (1.0, 10.0), 1.0), (4096, (3.0,), 0.5)])
def test_newton_matches_converged_projection(batch, sigmas, eps):
    L = make_logits(batch, sigmas, seed=batch + 7)
    P, it = gpu_newton(L, eps, 50, 1e-6)
    Po, ito = oracle.birkhoff4_newton(L, eps, 100, 1e-13)
    conv = it < 50
    d = np.abs(P - Po).max(axis=(1, 2))
    print(f"batch {batch} sigmas {sigmas} eps {eps}: converged {conv.mean():.4f}, steps median "
          f"{np.median(it):.0f} max {it.max()} (oracle median {np.median(ito):.0f}); "
          f"max|P-P*| {d.max():.2e}", flush=True)
    assert np.all(conv)
    assert np.all(_err(P) <= 1e-6 + 1e-7)
    assert d.max() <= TOL_NEWTON


def test_newton_full_batch_sampled():
    L = make_logits(1 << 20, (1.0, 10.0), seed=0)
    P, it = gpu_newton(L, 1.0, 50, 1e-6)
    idx = np.concatenate([np.random.default_rng(2).choice(1 << 20, 4096, replace=False),
                          [0, (1 << 19) - 1, 1 << 19, (1 << 20) - 1]])
    Po, _ = oracle.birkhoff4_newton(L[idx], 1.0, 100, 1e-13)
    d = np.abs(P[idx] - Po).max()
    print(f"2^20 batch: steps mean {it.mean():.2f} max {it.max()}, converged "
          f"{(it < 50).mean():.5f}; sampled max|P-P*| {d:.2e}", flush=True)
    assert np.all(it < 50)
    assert d <= TOL_NEWTON


def test_newton_agrees_with_sinkhorn_kernel():
    L = make_logits(4096, (1.0,), seed=5)
    Pn, _ = gpu_newton(L, 1.0, 50, 1e-7)
    Ps, _ = gpu_birkhoff(L, 1.0, 500, 1e-7)
    assert np.abs(Pn - Ps).max() <= 2e-6


def test_newton_edge_cases():
    # constant logits: the first plan is already doubly stochastic -> 0 steps
    L = np.full((3, 4, 4), -1.5, np.float32)
    P, it = gpu_newton(L, 1.0, 50, 1e-6)
    assert list(it) == [0, 0, 0]
    np.testing.assert_allclose(P, 0.25, rtol=1e-6)
    # max_iters = 0: the row softmax of L/eps, as the oracle with 0 steps
    L = make_logits(33, (2.0,), seed=9)
    P, it = gpu_newton(L, 0.7, 0, 1e-6)
    Po, _ = oracle.birkhoff4_newton(L, 0.7, 0, -1.0)
    assert np.all(it == 0)
    assert np.abs(P - Po).max() <= 1e-6
    # in place
    L = make_logits(300, (1.0, 10.0), seed=10)
    P1, it1 = gpu_newton(L, 1.0, 50, 1e-6)
    P2, it2 = gpu_newton(L, 1.0, 50, 1e-6, inplace=True)
    np.testing.assert_array_equal(P1, P2)
    np.testing.assert_array_equal(it1, it2)


@pytest.mark.parametrize("sigmas,eps", [((1.0,), 1.0), ((1.0, 10.0), 1.0), ((2.0,), 0.3)])
def test_backward_matches_oracle_on_same_plan(sigmas, eps):
    L = make_logits(4096, sigmas, seed=13)
    Po, _ = oracle.birkhoff4_newton(L, eps, 100, 1e-13)
    P32 = Po.astype(np.float32)
    G = np.random.default_rng(14).normal(size=L.shape).astype(np.float32)
    gL = gpu_backward(P32, G, eps)
    ref = oracle.birkhoff4_backward(P32, G, eps)
    scale = 1.0 + np.abs(ref).max(axis=(1, 2))
    rel = np.abs(gL - ref).max(axis=(1, 2)) / scale
    print(f"backward sigmas {sigmas} eps {eps}: max rel err {rel.max():.2e}", flush=True)
    assert rel.max() <= 1e-6


def test_backward_end_to_end_and_invariants():
    # GPU forward then GPU backward against the oracle's converged forward and
    # backward; zero row and column sums (shift invariance of the projection).
    L = make_logits(8192, (1.0,), seed=15)
    G = np.random.default_rng(16).normal(size=L.shape).astype(np.float32)
    P, _ = gpu_newton(L, 1.0, 50, 1e-7)
    gL = gpu_backward(P, G, 1.0)
    Po, _ = oracle.birkhoff4_newton(L, 1.0, 100, 1e-13)
    ref = oracle.birkhoff4_backward(Po, G, 1.0)
    scale = 1.0 + np.abs(ref).max(axis=(1, 2))
    rel = np.abs(gL - ref).max(axis=(1, 2)) / scale
    rows = np.abs(gL.astype(np.float64).sum(2)).max(1) / scale
    cols = np.abs(gL.astype(np.float64).sum(1)).max(1) / scale
    print(f"end to end: max rel err {rel.max():.2e}, row sums {rows.max():.1e}, "
          f"col sums {cols.max():.1e}", flush=True)
    assert rel.max() <= 1e-4
    assert rows.max() <= 1e-5 and cols.max() <= 1e-4
