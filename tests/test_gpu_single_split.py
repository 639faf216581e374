"""GPU parity of the half-step's one-split path, per kernel family.

Each half-step kernel deals the columns to several workgroups per row block
("column splits") and merges their (max, sum) pairs afterwards, unless the
row blocks alone already fill the chip: then one split covers all columns and
the kernel writes the biases and potentials itself, with no partials and no
merge. That happens only for many rows, which the other tests do not reach:
262144 rows on the 32x32 tiles (256 rows per block, 1024 blocks), 131072 on
the 16x16 tiles (128 rows per block, 1024 blocks) and 524288 above 448
coordinates (the latter in test_gpu_widest_dim.py). The update is the one of
"FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodik
section 1; one iteration from g = 0, checked on sampled rows of both sides
against the fp64 oracle's half-steps (the g rows see all the f potentials).
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import random_clouds

from gpu_helpers import DEV, dev, rel_inf

pytestmark = pytest.mark.gpu

TOL_HALF = 1e-5


@pytest.mark.parametrize("n,m,d", [(262144, 200, 64), (262144, 150, 192),
                                   (131072, 200, 256), (131072, 150, 448)])
def test_single_column_split(n, m, d):
    c = random_clouds(n, m, d, seed=d + 3, spread=1.0 / np.sqrt(d))
    eps = 0.3
    print(f"{n}x{m}x{d}: one iteration from g = 0", flush=True)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(n, device=DEV)
    g = torch.zeros(m, device=DEV)
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 1, f, g)
    torch.cuda.synchronize()
    f_np, g_np = f.cpu().numpy(), g.cpu().numpy()
    rows = np.arange(0, n, 2503)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], np.zeros(m), eps, rows=rows)
    g_rows = np.arange(0, m, 10)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f_np, eps, rows=g_rows)
    ef, eg = rel_inf(f_np[rows], f_ref), rel_inf(g_np[g_rows], g_ref)
    print(f"  sampled rows: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF
