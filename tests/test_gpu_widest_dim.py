"""GPU parity for the widest feature dimensions, 448 < d <= 1024 (the pages
measure up to d = 1024, "FlashSinkhorn: IO-Aware Entropic Optimal Transport
on GPU", "Experimentelle Ergebnisse"). Records of 512, 640, 768, 896 or 1024
coordinates (staged above 512); the half-step and the statistics are tiled
like a matrix product, both sides streamed through LDS in 32-coordinate
stages, each stage's chains flushed into fp32 sums. The update is the one of
"Methodik" section 1, checked against the fp64 oracle at the bounds of the
other paths:

* one f and one g half-step from identical fp32 inputs at every record size,
  clouds at the origin and far from it;
* whole solves on odd shapes (a single source or target point, ragged tiles),
  the feature workload's distributions at d = 1024 with plan statistics, the
  eps schedule, statistics of identical potentials, bitwise determinism;
* at 65536 x 65536 x 1024, one half-step from the GPU's own iterate on
  sampled rows;
* the transport application, barycentric map and x-gradient ("Methodik"
  section 3) on the same pipeline with P.V per 128-column block, 64 value
  channels per pass: whole outputs against the oracle on odd shapes and value
  widths, and the refusal above OT_MAX_DIM.
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
    (513, 0.5, 0.0), (640, 0.5, 0.0), (700, 0.25, 0.0), (768, 0.1, 0.0), (800, 0.5, 30.0),
    (896, 0.5, 0.0), (1000, 0.5, -40.0), (1024, 0.5, 0.0), (1024, 0.1, 0.0),
])
def test_widest_half_step_on_unit_gaussians(d, eps_factor, offset):
    c = random_clouds(1000, 1500, d, seed=d + 11, spread=1.0)
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


@pytest.mark.parametrize("n,m,d", [(1, 97, 1024), (97, 1, 640), (129, 700, 768),
                                   (300, 257, 1024), (257, 300, 896), (700, 129, 600),
                                   (1, 1, 1024), (49, 51, 1000)])
def test_widest_shapes(n, m, d):
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


def test_widest_feature_distribution_d1024_whole_solve():
    c = make_clouds("feature64_64k", n=1100, m=1300, d=1024)
    eps, iters = c["eps"][0], 20
    print("feature distribution at d=1024, 1100x1300, 20 iterations", flush=True)
    f, g = gpu_solve(c, eps, iters)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, iters)
    ef, eg = rel_inf(f, fo, eps), rel_inf(g, go, eps)
    print(f"  rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps, "  d=1024 stats")


def test_widest_eps_scaling_schedule_d768():
    c = make_clouds("feature64_64k", n=800, m=1000, d=768)
    eps_list = geometric_eps_schedule(2.0, 0.05, 3)
    print("d=768 schedule", flush=True)
    f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), 10)
    fo, go = oracle.sinkhorn_schedule(c["x"], c["y"], c["a"], c["b"], eps_list, 10)
    ef, eg = rel_inf(f, fo, eps_list[-1]), rel_inf(g, go, eps_list[-1])
    print(f"  rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    _check_stats(c, f, g, fo, go, eps_list[-1], "  d=768 schedule stats")


@pytest.mark.parametrize("n,m,d,offset", [(129, 257, 640, 0.0), (300, 200, 1024, 30.0),
                                          (200, 300, 896, 0.0), (257, 129, 768, 0.0),
                                          (1, 300, 1024, 0.0), (300, 1, 700, 0.0)])
def test_widest_plan_stats(n, m, d, offset):
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


def test_widest_grid_rounding():
    # 2600 and 3000 rows are 11 and 12 blocks of 256: at least 8 but not a
    # multiple of 8, so the grid rounds the row-block count up to 16 (the
    # extra workgroups exit at once) and several column splits per row block
    # run; one half-step each way and the statistics against the oracle.
    c = random_clouds(2600, 3000, 768, seed=77, spread=1.0)
    eps = 0.5 * 768 ** 0.5
    print("2600x3000x768: one half-step each way, then statistics", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 3)
    g32 = go.astype(np.float32)
    f1, g1 = gpu_solve(c, eps, 1, g0=g32)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g32, eps)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f1, eps)
    ef, eg = rel_inf(f1, f_ref), rel_inf(g1, g_ref)
    print(f"  one half-step rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF
    f, g = fo.astype(np.float32), go.astype(np.float32)
    st = gpu_plan_stats(c, f, g, eps)
    sk = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    ec = abs(st["cost"] - sk["cost"]) / abs(sk["cost"])
    print(f"  cost rel {ec:.1e}; marg {st['marg_row']:.3e}/{st['marg_col']:.3e} vs "
          f"{sk['marg_row']:.3e}/{sk['marg_col']:.3e}", flush=True)
    assert ec <= TOL_COST
    assert abs(st["marg_row"] - sk["marg_row"]) <= TOL_MARG
    assert abs(st["marg_col"] - sk["marg_col"]) <= TOL_MARG


def test_widest_single_column_split():
    # 524288 rows are 2048 row blocks: the column split count drops to one,
    # so the f half-step writes its potentials directly (no partials, no
    # merge); the g half-step (200 rows) runs 2048 splits. One iteration from
    # g = 0, checked on sampled rows of both sides.
    n, m, d = 524288, 200, 513
    c = random_clouds(n, m, d, seed=13, spread=1.0 / np.sqrt(d))
    eps = 0.3
    print(f"{n}x{m}x{d}: one iteration from g = 0", flush=True)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(n, device=DEV)
    g = torch.zeros(m, device=DEV)
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 1, f, g)
    torch.cuda.synchronize()
    f_np, g_np = f.cpu().numpy(), g.cpu().numpy()
    rows = np.arange(0, n, 5003)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], np.zeros(m), eps, rows=rows)
    g_rows = np.arange(0, m, 10)
    g_ref = oracle.half_update(c["y"], c["x"], c["b"], f_np, eps, rows=g_rows)
    ef, eg = rel_inf(f_np[rows], f_ref), rel_inf(g_np[g_rows], g_ref)
    print(f"  sampled rows: rel err f {ef:.2e} g {eg:.2e}", flush=True)
    assert ef <= TOL_HALF and eg <= TOL_HALF


def test_widest_bitwise_deterministic():
    c = random_clouds(2000, 1700, 1024, seed=5, spread=1.0 / 32.0)
    a = gpu_solve(c, 0.4, 5)
    b = gpu_solve(c, 0.4, 5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_widest_full_size_sampled_half_steps():
    # 65536 x 65536 at d = 1024 (the feature workload's distributions): two
    # GPU iterations, then one more f half-step, checked on sampled rows
    # against the oracle's half-step from the GPU's own g.
    c = make_clouds("feature64_64k", d=1024)
    eps = c["eps"][0]
    print("65536x65536x1024: 2 iterations + one f half-step", flush=True)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(65536, device=DEV)
    g = torch.zeros(65536, device=DEV)
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 2, f, g)
    g2 = g.clone()
    lds.ot_sinkhorn_solve(x, y, a, b, eps, 1, f, g)
    torch.cuda.synchronize()
    rows = np.arange(0, 65536, 2039)
    f_ref = oracle.half_update(c["x"], c["y"], c["a"], g2.cpu().numpy(), eps, rows=rows)
    err = rel_inf(f.cpu().numpy()[rows], f_ref)
    print(f"  sampled rows: rel err f {err:.2e}", flush=True)
    assert err <= TOL_HALF


TOL_APPLY = 5e-5  # the transport tests' bound (see test_gpu_transport.py)


@pytest.mark.parametrize("n,m,d,dv", [(700, 900, 640, 640), (1000, 700, 1024, 5),
                                      (300, 1300, 768, 100), (1, 300, 896, 65),
                                      (257, 1, 1024, 1024), (129, 257, 1000, 64),
                                      (600, 500, 513, 130)])
def test_widest_transport_apply(n, m, d, dv):
    # out_i = sum_j P_ij v_j from the one-pass transport kernel; oracle
    # potentials, random values (256 to 1024 padded channels, ragged ends).
    from workloads import random_values
    c = random_clouds(n, m, d, seed=n + m + d, spread=1.0 / np.sqrt(d))
    eps = 0.3
    print(f"transport {n}x{m}x{d}, dv={dv}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 6)
    f, g = fo.astype(np.float32), go.astype(np.float32)
    v = random_values(m, dv, seed=d)
    x, y = dev(c["x"]), dev(c["y"])
    out = torch.empty((n, dv), dtype=torch.float32, device=DEV)
    lds.ot_transport_apply(x, y, dev(f), dev(g), eps, dev(v), out)
    torch.cuda.synchronize()
    err = rel_inf(out.cpu().numpy(), oracle.transport_apply(c["x"], c["y"], f, g, eps, v))
    print(f"  rel err {err:.2e}", flush=True)
    assert err <= TOL_APPLY


@pytest.mark.parametrize("d", [640, 1024])
def test_widest_map_and_gradient(d):
    # The x-gradient takes the row sums beside the values in the same pass.
    c = make_clouds("feature64_64k", n=600, m=700, d=d)
    eps = c["eps"][0]
    print(f"barycentric map and x-gradient at d={d}", flush=True)
    fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 10)
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


def test_transport_random_shapes():
    # Seeded random shapes over every record size of the matrix-product
    # transport (d from 193 to 1024), ragged row and column counts and value
    # widths; whole outputs against the oracle.
    from workloads import random_values
    rng = np.random.default_rng(1234)
    for case in range(8):
        d = int(rng.integers(193, 1025))
        n, m = (int(v) for v in rng.integers(1, 900, size=2))
        dv = int(rng.integers(1, 200))
        c = random_clouds(n, m, d, seed=case, spread=1.0 / np.sqrt(d))
        eps = float(rng.uniform(0.1, 1.0))
        print(f"case {case}: {n}x{m}x{d}, dv={dv}, eps={eps:.3f}", flush=True)
        fo, go = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, 3)
        f, g = fo.astype(np.float32), go.astype(np.float32)
        v = random_values(m, dv, seed=case)
        out = torch.empty((n, dv), dtype=torch.float32, device=DEV)
        lds.ot_transport_apply(dev(c["x"]), dev(c["y"]), dev(f), dev(g), eps, dev(v), out)
        torch.cuda.synchronize()
        err = rel_inf(out.cpu().numpy(), oracle.transport_apply(c["x"], c["y"], f, g, eps, v))
        print(f"  rel err {err:.2e}", flush=True)
        assert err <= TOL_APPLY


def test_widest_transport_deterministic():
    from workloads import random_values
    c = random_clouds(300, 700, 1024, seed=9, spread=1.0 / 32)
    v = random_values(700, 70, seed=2)
    x, y = dev(c["x"]), dev(c["y"])
    f = dev(np.zeros(300, np.float32))
    g = dev(np.zeros(700, np.float32))
    outs = []
    for _ in range(2):
        out = torch.empty((300, 70), dtype=torch.float32, device=DEV)
        lds.ot_transport_apply(x, y, f, g, 0.5, dev(v), out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1])


def test_calls_refuse_beyond_the_largest_dimension():
    # The transport calls cover every d the solve covers; beyond it, every
    # call returns NOT_SUPPORTED.
    assert lds.OT_MAX_TRANSPORT_DIM == lds.OT_MAX_DIM
    d = lds.OT_MAX_DIM + 1
    c = random_clouds(40, 50, d, seed=1)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f, g = torch.zeros(40, device=DEV), torch.zeros(50, device=DEV)
    out = torch.empty_like(x)
    for call in (lambda: lds.ot_transport_apply(x, y, f, g, 0.5, y, out),
                 lambda: lds.ot_barycentric_map(x, y, a, f, g, 0.5, out),
                 lambda: lds.ot_cost_gradient_x(x, y, f, g, 0.5, out),
                 lambda: lds.ot_sinkhorn_solve(x, y, a, b, 0.5, 3, f, g)):
        with pytest.raises(lds.OTError) as ei:
            call()
        assert ei.value.status == lds.OT_ERROR_NOT_SUPPORTED
