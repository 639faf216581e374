"""GPU parity for feature dimensions above 192 (up to 512): the half-step and
the plan statistics on 16x16 matrix-core tiles (each wave owns 16 rows, so a
row's split operands take half the registers of the 32x32 kernels). The
pages measure up to d = 1024 ("FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU", "Experimentelle Ergebnisse"); the update is the one of
"Methodik" section 1, checked against the fp64 oracle:

* one f and one g half-step from identical fp32 inputs at every wide record
  size (224, 256, 320, 384, 448, 512 coordinates), with clouds at the origin
  and far from it, at the same 1e-5 bound as the other paths;
* whole solves on odd shapes (a single source or target point, ragged tiles)
  and at the feature workload's distributions at d = 256, the eps schedule,
  plan statistics on identical inputs, bitwise determinism;
* at 65536 x 65536 x 256, one half-step from the GPU's own iterate on sampled
  rows (the size the benchmark measures at d = 256);
* the transport application, barycentric map and x-gradient ("Methodik"
  section 3), on the one-pass transport kernel at every record size here
  (the x-gradient with the row sums beside the values).
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import geometric_eps_schedule, make_clouds, random_clouds

from gpu_helpers import (DEV, TOL_COST, TOL_MARG, TOL_POT, dev, gpu_plan_stats, gpu_solve,
                         gpu_solve_schedule, rel_inf)

pytestmark = pytest.mark.gpu

TOL_HALF = 1e-5


@pytest.mark.parametrize("d,eps_factor,offset", [
    (224, 0.5, 0.0), (256, 0.5, 0.0), (256, 0.1, 40.0), (320, 0.5, 0.0), (384, 0.25, 0.0),
    (448, 0.5, -30.0), (512, 0.5, 0.0), (512, 0.1, 0.0), (200, 1.0, 0.0), (300, 0.5, 0.0),
])
def test_wide_half_step_on_unit_gaussians(d, eps_factor, offset):
    c = random_clouds(1000, 1500, d, seed=d + 7, spread=1.0)
    c["x"] = c["x"] + np.float32(offset)
    c["y"] = c["y"] + np.float32(offset)
    eps = eps_factor * d ** 0.5
    print(f"d={d} eps={eps:.3g} offset {offset:g}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 4)
    g32 = go.astype(np.float32)
    f1, g1 = gpu_solve(c, eps, 1, g0=g32)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g32, eps)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f1, eps)
    ef, eg = rel_inf(f1, f_ref), rel_inf(g1, g_ref)
    print(f"  one half-step rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF


@pytest.mark.parametrize("n,m,d", [(1, 97, 256), (97, 1, 320), (129, 700, 224),
                                   (300, 257, 512), (257, 300, 448), (700, 129, 384),
                                   (1, 1, 256)])
def test_wide_shapes(n, m, d):
    c = random_clouds(n, m, d, seed=n * 7 + m * 3 + d)
    eps = 0.5 * d ** 0.5
    print(f"shape {n}x{m}x{d}", flush=True)
    f, g = gpu_solve(c, eps, 10)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 10)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    print(f"  rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT


def _check_stats(c, f, g, fo, go, eps, label):
    st = gpu_plan_stats(c, f, g, eps)
    so = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], fo, go, eps)
    ec = abs(st["cost"] - so["cost"]) / abs(so["cost"])
    em = abs(st["marg"] - so["marg"])
    print(f"{label}: cost rel {ec:.1e}; marg {st['marg']:.3e} vs {so['marg']:.3e} "
          f"(abs {em:.1e})", flush=True)
    assert ec <= TOL_COST and em <= TOL_MARG


def test_wide_feature_distribution_d256_whole_solve():
    c = make_clouds("feature64_64k", n=1200, m=1600, d=256)
    eps, iters = c["eps"][0], 50
    print("feature distribution at d=256, 1200x1600, 50 iterations", flush=True)
    f, g = gpu_solve(c, eps, iters)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, iters)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    print(f"  rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps, "  d=256 stats")


def test_wide_eps_scaling_schedule_d256():
    c = make_clouds("feature64_64k", n=900, m=1300, d=256)
    eps_list = geometric_eps_schedule(2.0, 0.05, 5)
    print("d=256 schedule", flush=True)
    f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), 15)
    fo, go = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], eps_list, 15)
    ef, eg = rel_inf(f, fo, eps_list[-1]), rel_inf(g, go, eps_list[-1])
    print(f"  rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps_list[-1], "  d=256 schedule stats")


@pytest.mark.parametrize("n,m,d,offset", [(129, 257, 224, 0.0), (300, 200, 256, 30.0),
                                          (200, 300, 512, 0.0), (257, 129, 384, 0.0),
                                          (1, 300, 256, 0.0), (300, 1, 448, 0.0)])
def test_wide_plan_stats(n, m, d, offset):
    # Statistics of the same fp32 (f, g) on both sides: the kernels alone.
    c = random_clouds(n, m, d, seed=n + 5 * m + d, spread=1.0 / np.sqrt(d))
    c["x"] = c["x"] + np.float32(offset)
    c["y"] = c["y"] + np.float32(offset)
    eps = 0.3
    print(f"stats {n}x{m}x{d} offset {offset:g}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    st = gpu_plan_stats(c, f, g, eps)
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    ec = abs(st["cost"] - sk["cost"]) / abs(sk["cost"])
    print(f"  cost rel {ec:.1e}; marg {st['marg_row']:.3e}/{st['marg_col']:.3e} vs "
          f"{sk['marg_row']:.3e}/{sk['marg_col']:.3e}", flush=True)
    assert ec <= TOL_COST
    assert abs(st["marg_row"] - sk["marg_row"]) <= TOL_MARG
    assert abs(st["marg_col"] - sk["marg_col"]) <= TOL_MARG


def test_wide_bitwise_deterministic():
    c = random_clouds(2000, 1700, 256, seed=3, spread=1.0 / 16.0)
    a = gpu_solve(c, 0.4, 7)
    b = gpu_solve(c, 0.4, 7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_wide_full_size_sampled_half_steps():
    # 65536 x 65536 at d = 256 (the feature workload's distributions): three
    # GPU iterations, then one more f half-step, checked on sampled rows
    # against the oracle's half-step from the GPU's own g.
    c = make_clouds("feature64_64k", d=256)
    eps = c["eps"][0]
    print("65536x65536x256: 3 iterations + one f half-step", flush=True)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(65536, device=DEV)
    g = torch.zeros(65536, device=DEV)
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 3, f, g)
    g3 = g.clone()
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 1, f, g)
    torch.cuda.synchronize()
    rows = np.arange(0, 65536, 1021)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g3.cpu().numpy(), eps, rows=rows)
    err = rel_inf(f.cpu().numpy()[rows], f_ref)
    print(f"  sampled rows: rel err f {err:.2e}", flush=True)
    assert err <= TOL_HALF


TOL_APPLY = 5e-5  # the transport tests' bound (see test_gpu_transport.py)


def _apply(c, f, g, eps, v):
    x, y = dev(c["x"]), dev(c["y"])
    out = torch.empty((x.shape[0], v.shape[1]), dtype=torch.float32, device=DEV)
    lds.ot_transport_apply(x, y, dev(f), dev(g), eps, dev(v), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n,m,d,dv", [(700, 900, 224, 224), (1000, 700, 256, 5),
                                      (300, 1300, 384, 40), (500, 600, 512, 512),
                                      (1, 300, 256, 33), (257, 1, 320, 64),
                                      (400, 500, 448, 70), (129, 640, 300, 300)])
def test_wide_transport_apply(n, m, d, dv):
    # out_i = sum_j P_ij v_j on 16x16 tiles; oracle potentials, random values.
    from workloads import random_values
    c = random_clouds(n, m, d, seed=n + m + d, spread=1.0 / np.sqrt(d))
    eps = 0.3
    print(f"transport {n}x{m}x{d}, dv={dv}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 8)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    v = random_values(m, dv, seed=d)
    out = _apply(c, f, g, eps, v)
    ref = oracle.transport_apply(c["x"], c["y"], f, g, eps, v)
    err = rel_inf(out, ref)
    print(f"  rel err {err:.2e}", flush=True)
    assert err <= TOL_APPLY


@pytest.mark.parametrize("d", [256, 448])
def test_wide_map_and_gradient(d):
    # The x-gradient takes the row sums beside the values in the same pass.
    c = make_clouds("feature64_64k", n=900, m=1100, d=d)
    eps = c["eps"][0]
    print(f"barycentric map and x-gradient at d={d}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 20)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    x, y, a = dev(c["x"]), dev(c["y"]), dev(c["a"])
    bary = torch.empty_like(x)
    grad = torch.empty_like(x)
    lds.ot_barycentric_map(x, y, a, dev(f), dev(g), eps, bary)
    lds.ot_cost_gradient_x(x, y, dev(f), dev(g), eps, grad)
    torch.cuda.synchronize()
    eb = rel_inf(bary.cpu().numpy(), oracle.barycentric_map(c["x"], c["y"], c["a"], f, g, eps))
    eg = rel_inf(grad.cpu().numpy(), oracle.grad_x(c["x"], c["y"], f, g, eps))
    print(f"  map rel err {eb:.2e}, gradient rel err {eg:.2e}", flush=True)
    assert eb <= TOL_APPLY and eg <= TOL_APPLY
