"""The stored full-size oracle results (``tests/golden/*.npz``, written by
``tests/golden/make_full_size.py`` from the oracle alone) against what must
hold for them without a GPU:

* the inputs the workload generator draws today hash to the fixture's key
  (a changed generator or schedule invalidates the fixture);
* the potentials are finite;
* the last half-step of every schedule is a g update, which makes the column
  sums of the plan equal b: the fixture's column marginal error (fp64
  potentials) is zero up to fp64 rounding ("FlashSinkhorn: IO-Aware Entropic
  Optimal Transport on GPU", Methodik section 1: each half-step matches one
  marginal);
* the statistics of the fp64 and of the fp32-rounded potentials differ only
  by what rounding the potentials moves.
"""
import glob
import os
import sys

import numpy as np
import pytest

from workloads import make_clouds

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
from make_full_size import input_key  # noqa: E402

FIXTURES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(GOLDEN, "*.npz")))


@pytest.mark.parametrize("fname", FIXTURES)
def test_fixture_is_consistent(fname):
    z = np.load(os.path.join(GOLDEN, fname))
    name = str(z["name"])
    n = int(z["n"]) if "n" in z.files else None
    m = int(z["m"]) if "m" in z.files else None
    c = make_clouds(name, n=n, m=m)
    assert input_key(c) == str(z["key"])
    f, g = z["f"], z["g"]
    assert f.shape == (c["n"],) and g.shape == (c["m"],)
    assert np.all(np.isfinite(f)) and np.all(np.isfinite(g))
    assert float(z["marg_col"]) <= 1e-11, float(z["marg_col"])
    assert float(z["cost"]) > 0.0
    assert abs(float(z["cost32"]) - float(z["cost"])) <= 1e-5 * abs(float(z["cost"]))
    assert np.allclose(np.asarray(z["eps"]), np.asarray(c["eps"]))
