"""Failure paths of the C ABI on the GPU: a temporary allocation that cannot
be had, and inputs that violate the documented (unchecked) preconditions.

* A call whose scratch does not fit in the device memory left free returns
  OT_ERROR_OUT_OF_MEMORY before anything is enqueued, and the next call that
  fits succeeds (the failed allocation's error is not reported again). The
  test first takes all but a few MiB of free device memory with one torch
  allocation, so that a valid call's scratch cannot be had.
* Zero or negative weights and zero vectors in the cosine calls are outside
  the domain. The calls still succeed and the violation shows up as inf or
  NaN, as the header states; the log of a zero weight is -inf, so that row's
  potential is -inf while the rest of the plan stays what the fp64 oracle
  computes from the same inputs (exp(-inf) = 0 drops the row from every
  other sum).
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import random_clouds

from gpu_helpers import DEV, TOL_POT, dev, rel_inf

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,n", [(3, 1 << 22), (64, 1 << 19)])
def test_out_of_memory_before_any_launch(d, n):
    # scratch of the solve: records of both clouds, >= 256 MiB at these sizes
    c = random_clouds(n, n, d, seed=1, spread=1.0 / np.sqrt(d))
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(n, device=DEV)
    g = torch.zeros(n, device=DEV)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info()
    hog = []
    for _ in range(6):  # allocation granularity: top up until < 96 MiB are free
        left = torch.cuda.mem_get_info()[0]
        if left < (96 << 20):
            break
        hog.append(torch.empty(left - (48 << 20), dtype=torch.uint8, device=DEV))
    left = torch.cuda.mem_get_info()[0]
    print(f"d={d}, n=m={n}: {free / 2**30:.1f} GiB free of {total / 2**30:.1f}; "
          f"left {left / 2**20:.0f} MiB after {len(hog)} allocations", flush=True)
    assert left < (200 << 20)
    try:
        with pytest.raises(lds.OTError) as e1:
            lds.ot_sinkhorn_solve(x, y, a, b, 0.5, 3, f, g)
        with pytest.raises(lds.OTError) as e2:
            lds.ot_plan_cost(x, y, f, g, 0.5, cost)
    finally:
        del hog
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    print(f"statuses: {e1.value.status}, {e2.value.status}", flush=True)
    assert e1.value.status == lds.OT_ERROR_OUT_OF_MEMORY
    assert e2.value.status == lds.OT_ERROR_OUT_OF_MEMORY
    assert torch.count_nonzero(f) == 0 and torch.count_nonzero(g) == 0  # nothing ran
    # the next call succeeds and is correct (sampled rows checked by the oracle)
    lds.ot_sinkhorn_solve(x, y, a, b, 0.5, 1, f, g)
    torch.cuda.synchronize()
    rows = np.arange(0, n, n // 64)
    fo = oracle.half_update(c["x"], c["y"], c["a"], np.zeros(n), 0.5, rows=rows)
    assert rel_inf(f.cpu().numpy()[rows], fo, 0.5) <= TOL_POT


@pytest.mark.parametrize("d", [3, 64])
def test_zero_weight_gives_minus_inf_potential(d):
    c = random_clouds(700, 500, d, seed=2, spread=1.0 / np.sqrt(d))
    a = c["a"].copy()
    a[5] = 0.0
    eps = 0.3
    x, y, at, b = dev(c["x"]), dev(c["y"]), dev(a), dev(c["b"])
    f = torch.zeros(700, device=DEV)
    g = torch.zeros(500, device=DEV)
    lds.ot_sinkhorn_solve(x, y, at, b, eps, 5, f, g)
    torch.cuda.synchronize()
    f, g = f.cpu().numpy(), g.cpu().numpy()
    fo, go = oracle.sinkhorn(c["x"], c["y"], a, c["b"], eps, 5)
    print(f"d={d}: f[5] = {f[5]} (oracle {fo[5]}), other f finite {np.isfinite(np.delete(f, 5)).all()}, "
          f"g finite {np.isfinite(g).all()}", flush=True)
    assert np.isneginf(fo[5]) and np.isneginf(f[5])
    keep = np.arange(700) != 5
    assert rel_inf(f[keep], fo[keep], eps) <= TOL_POT
    assert rel_inf(g, go, eps) <= TOL_POT


@pytest.mark.parametrize("d", [3, 64])
def test_negative_weight_gives_nan(d):
    c = random_clouds(300, 200, d, seed=3, spread=1.0 / np.sqrt(d))
    a = c["a"].copy()
    a[7] = -a[7]
    x, y, at, b = dev(c["x"]), dev(c["y"]), dev(a), dev(c["b"])
    f = torch.zeros(300, device=DEV)
    g = torch.zeros(200, device=DEV)
    lds.ot_sinkhorn_solve(x, y, at, b, 0.3, 2, f, g)
    torch.cuda.synchronize()
    print(f"d={d}: f[7] = {f[7].item()}, nonfinite g: {int((~torch.isfinite(g)).sum())}",
          flush=True)
    assert torch.isnan(f[7])
    assert not torch.isfinite(g).all()  # the NaN row enters every column's sum


def test_cosine_zero_vector_gives_nan():
    c = random_clouds(300, 200, 40, seed=4)
    x = c["x"].copy()
    x[11] = 0.0
    xt, y, a, b = dev(x), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(300, device=DEV)
    g = torch.zeros(200, device=DEV)
    lds.ot_sinkhorn_solve_cosine(xt, y, a, b, 0.1, 2, f, g)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    lds.ot_plan_stats_cosine(xt, y, a, b, torch.zeros_like(f), torch.zeros_like(g), 0.1, cost,
                             marg)
    torch.cuda.synchronize()
    fo, go = oracle.sinkhorn_cosine(x, c["y"], c["a"], c["b"], 0.1, 2)
    print(f"zero vector: GPU nonfinite f {int((~torch.isfinite(f)).sum())}, "
          f"g {int((~torch.isfinite(g)).sum())}, cost {cost.item()}; oracle nonfinite "
          f"f {int((~np.isfinite(fo)).sum())} g {int((~np.isfinite(go)).sum())}", flush=True)
    assert not np.isfinite(fo).all()
    assert not torch.isfinite(f).all() and not torch.isfinite(g).all()
    assert not np.isfinite(cost.item())
