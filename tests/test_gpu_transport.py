"""GPU parity of the transport application and what is built on it, against
the fp64 oracle: out_i = sum_j P_ij v_j, the barycentric map
sum_j P_ij y_j / a_i and the x-gradient 2 sum_j P_ij (x_i - y_j)
("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodik
section 3).

Potentials come from the oracle's own solver (reduced sizes) or from a seeded
synthetic recipe (full sizes), never from the HIP path; both sides get the
same fp32 potentials.

Tolerance (normwise, max|out - ref| / max|ref| over the whole output): each
P_ij carries a relative error of a few fp32 ulps (log2 P is formed in fp32 on
the matrix cores, in fp64 on the d < 32 path, then one exp2), and the sums are
fp32 within one workgroup's column range (up to 16384 columns on the matrix
cores, 256 on the d < 32 path) and fp64 across ranges. A random-walk estimate
u*sqrt(K) is 8e-6 for K = 16384; TOL_APPLY = 5e-5 leaves a factor ~6.
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
import oracle
from workloads import make_clouds, random_clouds, random_values

from gpu_helpers import DEV, dev, rel_inf

pytestmark = pytest.mark.gpu

TOL_APPLY = 5e-5


def _oracle_potentials(c, eps, iters):
    f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps, iters)
    return f.astype(np.float32), g.astype(np.float32)


def _synthetic_potentials(c, eps, seed=3):
    """f_i = |x_i|^2 - eps log m + eps z_i / 4, g_j = |y_j|^2 + eps w_j / 4
    (z, w ~ N(0,1)): log P_ij = (2 x_i.y_j)/eps - log m + noise, so the large
    |x|^2 and |y|^2 terms cancel inside the kernel as they do for solver
    potentials, and every row of P sums to O(1)."""
    rng = np.random.default_rng(seed)
    x = c["x"].astype(np.float64)
    y = c["y"].astype(np.float64)
    m = y.shape[0]
    f = (x * x).sum(1) - eps * np.log(m) + 0.25 * eps * rng.normal(size=x.shape[0])
    g = (y * y).sum(1) + 0.25 * eps * rng.normal(size=m)
    return f.astype(np.float32), g.astype(np.float32)


def gpu_apply(c, f, g, eps, v):
    x, y = dev(c["x"]), dev(c["y"])
    out = torch.empty((x.shape[0], v.shape[1]), dtype=torch.float32, device=DEV)
    lds.ot_transport_apply(x, y, dev(f), dev(g), eps, dev(v), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_map(c, f, g, eps):
    x, y = dev(c["x"]), dev(c["y"])
    out = torch.empty_like(x)
    lds.ot_barycentric_map(x, y, dev(c["a"]), dev(f), dev(g), eps, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_grad(c, f, g, eps):
    x, y = dev(c["x"]), dev(c["y"])
    out = torch.empty_like(x)
    lds.ot_cost_gradient_x(x, y, dev(f), dev(g), eps, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# --------------------------------------------------------------------------- #
# reduced workloads: oracle potentials, whole outputs                           #
# --------------------------------------------------------------------------- #

REDUCED = [("gauss3d_1k", 1024, 1024, 30), ("cube_gauss3d_16k", 2000, 1500, 30),
           ("feature64_64k", 1500, 2100, 20), ("mixture_sphere3d_eps_scaling", 1800, 1300, 30)]


@pytest.mark.parametrize("name,n,m,iters", REDUCED)
def test_reduced_workload_apply_map_grad(name, n, m, iters):
    c = make_clouds(name, n=n, m=m)
    eps = c["eps"][-1] if name != "mixture_sphere3d_eps_scaling" else 0.05
    print(f"{name} n={n} m={m} eps={eps}", flush=True)
    f, g = _oracle_potentials(c, eps, iters)
    d = c["x"].shape[1]
    for dv in (1, d, 2 * d + 3):
        v = random_values(m, dv, seed=dv)
        out = gpu_apply(c, f, g, eps, v)
        ref = oracle.transport_apply(c["x"], c["y"], f, g, eps, v)
        e = rel_inf(out, ref)
        print(f"  apply dv={dv}: rel err {e:.2e}", flush=True)
        assert e <= TOL_APPLY
    em = rel_inf(gpu_map(c, f, g, eps), oracle.barycentric_map(c["x"], c["y"], c["a"], f, g, eps))
    eg = rel_inf(gpu_grad(c, f, g, eps), oracle.grad_x(c["x"], c["y"], f, g, eps))
    print(f"  map rel err {em:.2e}  grad rel err {eg:.2e}", flush=True)
    assert em <= TOL_APPLY and eg <= TOL_APPLY


# --------------------------------------------------------------------------- #
# shapes: every kernel boundary in d, ragged n and m, value widths             #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("n,m,d", [
    (1, 1, 3), (1, 700, 3), (700, 1, 3), (333, 517, 5), (257, 255, 17), (300, 600, 31),
    (300, 600, 32), (257, 513, 33), (400, 350, 48), (1, 900, 64), (900, 1, 64),
    (513, 1025, 64), (300, 700, 100), (260, 300, 128),
    # above 128 coordinates: 64-column tiles, hi operands read twice, one
    # 32-channel value block per pass; the map and the x-gradient (dv = d >
    # 128) take the one-pass kernel
    (300, 400, 160), (257, 300, 192), (1, 500, 192),
])
def test_shapes(n, m, d):
    c = random_clouds(n, m, d, seed=n + m + d, spread=1.0 / np.sqrt(d))
    eps = 0.2
    f, g = _oracle_potentials(c, eps, 8)
    for dv in (1, 3, 32, 33, 64, 65):
        v = random_values(m, dv, seed=dv + 1)
        e = rel_inf(gpu_apply(c, f, g, eps, v), oracle.transport_apply(c["x"], c["y"], f, g, eps, v))
        assert e <= TOL_APPLY, (n, m, d, dv, e)
    em = rel_inf(gpu_map(c, f, g, eps), oracle.barycentric_map(c["x"], c["y"], c["a"], f, g, eps))
    eg = rel_inf(gpu_grad(c, f, g, eps), oracle.grad_x(c["x"], c["y"], f, g, eps))
    print(f"n={n} m={m} d={d}: map {em:.2e} grad {eg:.2e}", flush=True)
    assert em <= TOL_APPLY and eg <= TOL_APPLY


@pytest.mark.parametrize("d,offset", [(64, 30.0), (33, -50.0), (3, 30.0)])
def test_offset_clouds(d, offset):
    # Both clouds far from the origin: the plan comes from scores of the
    # centred points (d >= 32) or fp64 scores (d < 32), so P.v keeps its
    # precision.
    c = random_clouds(300, 600, d, seed=d + 21, spread=1.0 / np.sqrt(d))
    c["x"] = c["x"] + np.float32(offset)
    c["y"] = c["y"] + np.float32(offset)
    eps = 0.2
    f, g = _oracle_potentials(c, eps, 8)
    for dv in (3, 64):
        v = random_values(600, dv, seed=dv + 5)
        e = rel_inf(gpu_apply(c, f, g, eps, v), oracle.transport_apply(c["x"], c["y"], f, g, eps, v))
        print(f"offset {offset:g} d={d} dv={dv}: apply rel err {e:.2e}", flush=True)
        assert e <= TOL_APPLY
    em = rel_inf(gpu_map(c, f, g, eps), oracle.barycentric_map(c["x"], c["y"], c["a"], f, g, eps))
    print(f"offset {offset:g} d={d}: map rel err {em:.2e}", flush=True)
    assert em <= TOL_APPLY


@pytest.mark.parametrize("d,dv", [(3, 1024), (64, 1024), (64, 200), (3, 17), (192, 200)])
def test_wide_values(d, dv):
    c = random_clouds(300, 400, d, seed=d + dv, spread=1.0 / np.sqrt(d))
    f, g = _oracle_potentials(c, 0.3, 5)
    v = random_values(400, dv, seed=9)
    e = rel_inf(gpu_apply(c, f, g, 0.3, v), oracle.transport_apply(c["x"], c["y"], f, g, 0.3, v))
    print(f"d={d} dv={dv}: rel err {e:.2e}", flush=True)
    assert e <= TOL_APPLY


@pytest.mark.parametrize("d,dv", [(160, 128), (160, 129), (192, 128), (192, 129), (192, 256),
                                  (192, 257), (160, 1024)])
def test_one_pass_boundary(d, dv):
    # At 160 and 192 coordinates up to 128 value channels go through the
    # 32x32 kernel's passes, from 129 on through the one-pass kernel; both
    # sides of the switch and the channel padding to 256 against the oracle.
    c = random_clouds(257, 600, d, seed=d * 7 + dv, spread=1.0 / np.sqrt(d))
    f, g = _oracle_potentials(c, 0.3, 5)
    v = random_values(600, dv, seed=dv + 2)
    e = rel_inf(gpu_apply(c, f, g, 0.3, v), oracle.transport_apply(c["x"], c["y"], f, g, 0.3, v))
    print(f"d={d} dv={dv}: rel err {e:.2e}", flush=True)
    assert e <= TOL_APPLY


def test_single_source_point_closed_form():
    # n = 1 after one f half-step from any g: P_1j = exp((g_j - C_1j)/eps) /
    # sum_k exp((g_k - C_1k)/eps) * a_1, so the map is the softmax-weighted
    # mean of y (closed form, independent of the oracle's transport code).
    rng = np.random.default_rng(11)
    c = {"x": rng.normal(size=(1, 64)).astype(np.float32) / 8,
         "y": rng.normal(size=(2000, 64)).astype(np.float32) / 8,
         "a": np.ones(1, np.float32), "b": np.full(2000, 1 / 2000, np.float32)}
    eps = 0.1
    g = (0.05 * rng.normal(size=2000)).astype(np.float32)
    C = ((c["x"].astype(np.float64) - c["y"].astype(np.float64)) ** 2).sum(1)
    s = (g.astype(np.float64) - C) / eps
    w = np.exp(s - s.max())
    w /= w.sum()
    f = np.array([-eps * (s.max() + np.log(np.exp(s - s.max()).sum()))], np.float32)
    T = gpu_map(c, f, g, eps)[0]
    ref = w @ c["y"].astype(np.float64)
    assert rel_inf(T, ref) <= 1e-5


def test_deterministic():
    c = random_clouds(700, 1900, 64, seed=5, spread=0.125)
    f, g = _oracle_potentials(c, 0.25, 4)
    v = random_values(1900, 65, seed=1)
    a = gpu_apply(c, f, g, 0.25, v)
    b = gpu_apply(c, f, g, 0.25, v)
    assert np.array_equal(a, b)
    assert np.array_equal(gpu_grad(c, f, g, 0.25), gpu_grad(c, f, g, 0.25))


# --------------------------------------------------------------------------- #
# full sizes: synthetic potentials, sampled rows                                #
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("name", ["feature64_64k", "cube_gauss3d_64k", "feature1024_50k"])
def test_full_size_sampled_rows(name):
    c = make_clouds(name)
    eps = c["eps"][0]
    n, m, d = c["n"], c["m"], c["d"]
    f, g = _synthetic_potentials(c, eps)
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 48, replace=False)]))
    print(f"{name}: full-size transport apply (v = y) and gradient", flush=True)
    out = gpu_apply(c, f, g, eps, c["y"])
    sub = {"x": c["x"][rows], "y": c["y"]}
    ref = oracle.transport_apply(sub["x"], c["y"], f[rows], g, eps, c["y"])
    e = rel_inf(out[rows], ref)
    grad = gpu_grad(c, f, g, eps)
    eg = rel_inf(grad[rows], oracle.grad_x(sub["x"], c["y"], f[rows], g, eps))
    print(f"{name}: sampled rows apply rel err {e:.2e}, grad rel err {eg:.2e}", flush=True)
    assert e <= TOL_APPLY and eg <= TOL_APPLY
