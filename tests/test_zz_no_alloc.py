"""ot_sinkhorn_solve_no_alloc: the solve with its scratch in the library's
static device array, for callers that cannot allocate. It runs the kernels
of ot_sinkhorn_solve on the same inputs, so its potentials must equal that
call's bit for bit (the kernels are deterministic: fixed reduction orders,
no atomics). Two calls in a row, the second on a smaller problem, check
that the array's leftover contents from the first call do not leak into the
second; a problem whose scratch exceeds the array is refused before
anything is enqueued.
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
from workloads import make_clouds, random_clouds

from gpu_helpers import DEV, dev

pytestmark = pytest.mark.gpu


def _both(c, eps, iters, g0=None):
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    n, m = x.shape[0], y.shape[0]
    g_init = torch.zeros(m, device=DEV) if g0 is None else dev(np.asarray(g0, np.float32))
    f1, g1 = torch.zeros(n, device=DEV), g_init.clone()
    f2, g2 = torch.full((n,), 7.0, device=DEV), g_init.clone()
    lds.ot_sinkhorn_solve(x, y, a, b, eps, iters, f1, g1)
    lds.ot_sinkhorn_solve_no_alloc(x, y, a, b, eps, iters, f2, g2)
    torch.cuda.synchronize()
    return (f1, g1), (f2, g2)


@pytest.mark.parametrize("d", [3, 64, 256, 1024])
def test_no_alloc_matches_solve_two_calls(d):
    for call, (n, m) in enumerate([(3000, 2500), (700, 900)]):
        print(f"d={d} call {call}: {n}x{m}", flush=True)
        c = random_clouds(n, m, d, seed=100 * d + call, spread=1.0 / np.sqrt(d))
        (f1, g1), (f2, g2) = _both(c, 0.2, 11)
        assert torch.isfinite(f1).all() and torch.isfinite(g1).all()
        assert torch.equal(f1, f2) and torch.equal(g1, g2)


def test_no_alloc_headline_size_and_warm_start():
    # the 65536 x 65536 x 64 workload (69.25 MiB of scratch) fits the array
    c = make_clouds("feature64_64k")
    print("feature64_64k, 3 iterations", flush=True)
    (f1, g1), (f2, g2) = _both(c, 0.5, 3)
    assert torch.equal(f1, f2) and torch.equal(g1, g2)
    # then a small d = 3 problem warm-started from a nonzero g
    c = random_clouds(1000, 1200, 3, seed=9)
    g0 = np.linspace(-0.2, 0.3, 1200)
    (f1, g1), (f2, g2) = _both(c, 0.1, 5, g0)
    assert torch.equal(f1, f2) and torch.equal(g1, g2)


def test_no_alloc_refuses_scratch_beyond_the_array():
    # 65536 x 65536 at d = 128 needs 133.5 MiB > 128 MiB
    n = 65536
    x = torch.zeros(n, 128, device=DEV)
    a = torch.full((n,), 1.0 / n, device=DEV)
    f = torch.zeros(n, device=DEV)
    g = torch.zeros(n, device=DEV)
    with pytest.raises(lds.OTError) as e:
        lds.ot_sinkhorn_solve_no_alloc(x, x.clone(), a, a.clone(), 0.5, 1, f, g)
    assert e.value.status == lds.OT_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(f) == 0 and torch.count_nonzero(g) == 0
