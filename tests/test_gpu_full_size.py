"""GPU parity at the workloads' full sizes, end to end, against stored fp64
oracle results.

Each fixture under ``tests/golden/`` was written by
``tests/golden/make_full_size.py`` (which calls only the oracle and the input
generators): the oracle's potentials after the workload's whole iteration
count (every stage of its eps schedule) from a cold start, and the oracle's
plan statistics of those potentials. Here the same inputs are redrawn (their
hash must match the fixture's), the GPU runs the same solve in the launch
configuration the benchmark uses, and:

* f, g are compared normwise with the fixture's (``max|v - v*| / max|v*|
  <= 1e-4``);
* the GPU's plan statistics of its own potentials are compared with the
  oracle's of its own (cost relative ``<= 1e-5``, each marginal L1 error
  absolute ``<= 1e-5``): the whole path, error accumulated over every
  iteration included;
* the GPU's plan statistics of the oracle's potentials rounded to fp32 are
  compared with the oracle's statistics of the same fp32 potentials (the
  statistics kernels alone, identical inputs).

This is the check of the claim that the streamed log-sum-exp reductions are
exact ("FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU", Methodik
section 2, and "Bedeutung und Behauptungen"): the fp32 GPU iterate stays on
the fp64 iterate at the benchmarked sizes.
"""
import glob
import os
import sys

import numpy as np
import pytest

from gpu_helpers import (TOL_COST, TOL_MARG, TOL_POT, gpu_plan_stats, gpu_solve,
                         gpu_solve_schedule, rel_inf)
from workloads import make_clouds

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
from make_full_size import input_key  # noqa: E402  (hashing only, no oracle call)

FIXTURES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(GOLDEN, "*.npz")))


def _load(fname):
    z = np.load(os.path.join(GOLDEN, fname))
    fx = {k: z[k] for k in z.files}
    name = str(fx["name"])
    n = int(fx["n"]) if "n" in fx else None
    m = int(fx["m"]) if "m" in fx else None
    c = make_clouds(name, n=n, m=m)
    assert input_key(c) == str(fx["key"]), f"{fname}: inputs differ from the fixture's"
    return c, fx


@pytest.mark.parametrize("fname", FIXTURES)
def test_full_size_solve_matches_oracle(fname):
    print(f"[{fname}] solve", flush=True)
    c, fx = _load(fname)
    eps_list = [float(e) for e in fx["eps"]]
    iters = int(fx["iters"])
    if len(eps_list) == 1:
        f, g = gpu_solve(c, eps_list[0], iters)
    else:
        f, g = gpu_solve_schedule(c, eps_list[0], eps_list[-1], len(eps_list), iters)
    eps = eps_list[-1]
    ef, eg = rel_inf(f, fx["f"], eps), rel_inf(g, fx["g"], eps)
    st = gpu_plan_stats(c, f, g, eps)
    ec = abs(st["cost"] - float(fx["cost"])) / abs(float(fx["cost"]))
    er = abs(st["marg_row"] - float(fx["marg_row"]))
    el = abs(st["marg_col"] - float(fx["marg_col"]))
    print(f"[{fname}] {c['n']}x{c['m']}x{c['d']}, {iters * len(eps_list)} iterations: rel err "
          f"f {ef:.2e} g {eg:.2e}; cost {st['cost']:.10g} vs {float(fx['cost']):.10g} "
          f"(rel {ec:.1e}); marg row {st['marg_row']:.3e} vs {float(fx['marg_row']):.3e} "
          f"(abs {er:.1e}), col {st['marg_col']:.3e} vs {float(fx['marg_col']):.3e} "
          f"(abs {el:.1e})", flush=True)
    assert ef <= TOL_POT and eg <= TOL_POT
    assert ec <= TOL_COST
    assert er <= TOL_MARG and el <= TOL_MARG


@pytest.mark.parametrize("fname", FIXTURES)
def test_full_size_plan_stats_on_oracle_potentials(fname):
    print(f"[{fname}] plan statistics", flush=True)
    c, fx = _load(fname)
    eps = float(fx["eps"][-1])
    st = gpu_plan_stats(c, fx["f"].astype(np.float32), fx["g"].astype(np.float32), eps)
    ec = abs(st["cost"] - float(fx["cost32"])) / abs(float(fx["cost32"]))
    er = abs(st["marg_row"] - float(fx["marg_row32"]))
    el = abs(st["marg_col"] - float(fx["marg_col32"]))
    print(f"[{fname}] statistics of the fixture's fp32 potentials: cost rel {ec:.1e}, "
          f"marg row abs {er:.1e} ({st['marg_row']:.3e}), col abs {el:.1e} "
          f"({st['marg_col']:.3e})", flush=True)
    assert ec <= TOL_COST
    assert er <= TOL_MARG and el <= TOL_MARG
