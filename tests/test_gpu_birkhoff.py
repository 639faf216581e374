"""GPU parity of the batched 4x4 Birkhoff projection against the fp64 oracle.

Page: "Aceleración de la Proyección de Birkhoff para Hiper-conexiones con
Restricción de Variedad", sections 1-2 (entropic OT with unit marginals,
Sinkhorn-Knopp, max subtraction), section 4 (N(0,1) vs N(0,10^2) inputs).
Stopping decisions are taken in fp32 on the GPU; the oracle replays the
GPU's iteration count per matrix and the plans are compared at that count.
"""
import numpy as np
import pytest

import oracle
from workloads import make_logits

from gpu_helpers import TOL_P4, gpu_birkhoff

pytestmark = pytest.mark.gpu


def _fp64_err(P):
    P = np.asarray(P, np.float64)
    return np.maximum(np.abs(P.sum(2) - 1).max(1), np.abs(P.sum(1) - 1).max(1))


@pytest.mark.parametrize("batch", [1, 63, 64, 65, 4096])
def test_fixed_20_iterations(batch):
    L = make_logits(batch, (1.0, 10.0), seed=batch)
    P, it = gpu_birkhoff(L, 1.0, 20, -1.0)
    assert np.all(it == 20)
    Po, _ = oracle.birkhoff4_replay(L, np.full(batch, 20, np.int32), 1.0)
    err = np.abs(P - Po).max()
    print(f"fixed20 batch {batch}: max|P-P*| {err:.2e}", flush=True)
    assert err <= TOL_P4


def test_until_converged_replay():
    L = make_logits(8192, (1.0, 10.0), seed=11)
    tol = 1e-6
    P, it = gpu_birkhoff(L, 1.0, 200, tol)
    Po, erro = oracle.birkhoff4_replay(L, it, 1.0)
    err = np.abs(P - Po).max()
    conv = it < 200
    e64 = _fp64_err(P)
    _, k_or = oracle.birkhoff4(L, 1.0, 200, tol)
    diff = it.astype(np.int64) - k_or
    print(f"converged {conv.mean():.3f}; max|P-P*| {err:.2e}; k_gpu - k_oracle "
          f"histogram {dict(zip(*np.unique(np.clip(diff, -3, 3), return_counts=True)))}",
          flush=True)
    assert err <= TOL_P4
    assert np.all(e64[conv] <= tol + 1e-6)
    assert np.all(it >= 1) and np.all(it <= 200)


def test_full_batch_sampled_replay():
    wl_batch = 1 << 20
    L = make_logits(wl_batch, (1.0, 10.0), seed=0)
    for mode, (max_iters, tol) in {"fixed20": (20, -1.0), "tol": (200, 1e-6)}.items():
        P, it = gpu_birkhoff(L, 1.0, max_iters, tol)
        idx = np.random.default_rng(1).choice(wl_batch, 4096, replace=False)
        idx = np.concatenate([idx, [0, wl_batch // 2 - 1, wl_batch // 2, wl_batch - 1]])
        Po, _ = oracle.birkhoff4_replay(L[idx], it[idx], 1.0)
        err = np.abs(P[idx] - Po).max()
        print(f"full batch {mode}: max|P-P*| {err:.2e}; mean iters {it.mean():.2f}", flush=True)
        assert err <= TOL_P4


def test_in_place_matches_out_of_place():
    import torch

    from gpu_helpers import dev

    import log_domain_sinkhorn_amd as lds

    L = make_logits(1000, (1.0, 10.0), seed=3)
    P, it = gpu_birkhoff(L, 1.0, 50, 1e-6)
    t = dev(L)
    it2 = torch.empty(1000, dtype=torch.int32, device=t.device)
    lds.ot_birkhoff_project_batched(t, 1.0, 50, 1e-6, t, it2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(t.cpu().numpy(), P)
    np.testing.assert_array_equal(it2.cpu().numpy(), it)


def test_constant_logits_and_zero_iterations():
    L = np.full((5, 4, 4), 1.5, np.float32)
    P, it = gpu_birkhoff(L, 1.0, 200, 1e-6)
    np.testing.assert_allclose(P, 0.25, atol=1e-7)
    assert np.all(it == 1)
    L2 = make_logits(8, (1.0,), seed=4)
    P0, it0 = gpu_birkhoff(L2, 2.0, 0, -1.0)
    np.testing.assert_allclose(P0, np.exp(L2.astype(np.float64) / 2.0), rtol=1e-6)
    assert np.all(it0 == 0)


def test_eps_other_than_one():
    L = make_logits(512, (1.0, 10.0), seed=5)
    P, it = gpu_birkhoff(L, 3.0, 30, -1.0)
    Po, _ = oracle.birkhoff4_replay(L, it, 3.0)
    assert np.abs(P - Po).max() <= TOL_P4


@pytest.mark.parametrize("eps", [0.2, 0.1])
def test_small_eps_extreme_logits(eps):
    # l = L log2(e)/eps reaches hundreds of log2 units: the first row step
    # subtracts the maximum, and column and row sums that underflow fp32 take
    # the max-subtracted LSE instead of the plain sum of 2^u. (Below eps ~
    # 0.05 the fp32 rounding of l itself, ~2^-24 |l|, brings plans of
    # near-tied assignments to ~1e-5 of the fp64 oracle.)
    L = make_logits(4096, (1.0, 10.0), seed=21)
    for max_iters, tol in ((20, -1.0), (200, 1e-6)):
        P, it = gpu_birkhoff(L, eps, max_iters, tol)
        assert np.all(np.isfinite(P))
        Po, _ = oracle.birkhoff4_replay(L, it, eps)
        err = np.abs(P - Po).max()
        print(f"eps {eps} max_iters {max_iters} tol {tol:g}: max|P-P*| {err:.2e}, "
              f"mean iters {it.mean():.1f}", flush=True)
        assert err <= TOL_P4
