"""Seeded synthetic inputs for log-domain Sinkhorn workloads.

This module only draws random inputs. It holds none of the method's
arithmetic, so both the fp64 oracle (under ``oracle/``) and the HIP path can be
fed the very same fp32 arrays from here without sharing any computation.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64), seed 0 unless stated.
* Values are drawn in fp64 in the order the workload text lists them, then
  rounded to nearest fp32.
* Dirichlet(1) weights are drawn in fp64, cast to fp32, renormalised in fp64
  and cast to fp32 again, so they sum to 1 up to one fp32 rounding each.
* Uniform weights are ``1/n`` rounded to fp32.

The point-cloud workloads come from the squared-Euclidean entropic OT problem
of "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU" (gist.science,
technical summary, "Problemstellung" and "Methodik"). The batched 4x4 logits
come from the Birkhoff-projection page ("Aceleración de la Proyección de
Birkhoff ...", §1 and §4: N(0,1) and N(0,10^2) inputs).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "CloudWorkload",
    "BirkhoffWorkload",
    "CLOUD_WORKLOADS",
    "BIRKHOFF_WORKLOADS",
    "make_clouds",
    "make_logits",
    "geometric_eps_schedule",
    "random_clouds",
    "random_values",
]


@dataclasses.dataclass(frozen=True)
class CloudWorkload:
    """A point-cloud entropic OT workload.

    ``eps`` is a list of regularisation values, one per stage; every stage runs
    ``iters`` alternating (f, g) iterations and warm-starts from the previous
    stage. A single-stage workload has a one-element list.
    """

    name: str
    n: int
    m: int
    d: int
    eps: tuple
    iters: int
    x_dist: str
    y_dist: str
    weights: str
    description: str

    @property
    def total_iters(self) -> int:
        return self.iters * len(self.eps)


@dataclasses.dataclass(frozen=True)
class BirkhoffWorkload:
    name: str
    batch: int
    sigmas: tuple  # one sigma per contiguous equal-sized part of the batch
    eps: float
    max_iters: int
    tol: float
    description: str


def geometric_eps_schedule(eps0: float, eps_end: float, stages: int) -> tuple:
    """``stages`` values from eps0 down to eps_end with a constant ratio, both ends
    included. This is input data (the schedule), drawn once here."""
    if stages == 1:
        return (float(eps0),)
    r = (eps_end / eps0) ** (1.0 / (stages - 1))
    return tuple(float(eps0 * r**s) for s in range(stages))


CLOUD_WORKLOADS: Dict[str, CloudWorkload] = {
    w.name: w
    for w in [
        CloudWorkload(
            "gauss3d_1k", 1024, 1024, 3, (0.1,), 100,
            "normal(0, I)", "normal(0.5*1, I)", "uniform",
            "n=m=1024, d=3, x~N(0,I), y~N(0.5*1,I), uniform weights, eps=0.1, 100 iterations",
        ),
        CloudWorkload(
            "cube_gauss3d_16k", 16384, 16384, 3, (0.05,), 200,
            "uniform[0,1]^3", "normal(0.5*1, 0.1^2 I)", "uniform",
            "n=m=16384, d=3, x~U[0,1]^3, y~N(0.5*1,0.1^2 I), uniform weights, eps=0.05, 200 iterations",
        ),
        CloudWorkload(
            "feature64_64k", 65536, 65536, 64, (0.5,), 100,
            "normal(0, I/64)", "normal(0, I/64) + 0.3*u", "dirichlet",
            "n=m=65536, d=64, x,y~N(0,I/64), y shifted by 0.3 along a random unit vector, "
            "Dirichlet(1) weights, eps=0.5, 100 iterations",
        ),
        CloudWorkload(
            "mixture_sphere3d_eps_scaling", 131072, 98304, 3,
            geometric_eps_schedule(1.0, 0.01, 8), 50,
            "4-component gaussian mixture, sigma=0.05", "uniform on unit sphere", "uniform",
            "n=131072, m=98304, d=3, x from a 4-component Gaussian mixture (sigma=0.05), "
            "y uniform on the unit sphere, uniform weights, eps 1.0 -> 0.01 over 8 geometric "
            "stages, 50 iterations per stage, warm start",
        ),
        # The feature workload's distributions at d=192, the largest on the
        # 32x32-tile kernels.
        CloudWorkload(
            "feature192_64k", 65536, 65536, 192, (0.5,), 100,
            "normal(0, I/192)", "normal(0, I/192) + 0.3*u", "dirichlet",
            "n=m=65536, d=192, x,y~N(0,I/192), y shifted by 0.3 along a random unit vector, "
            "Dirichlet(1) weights, eps=0.5, 100 iterations",
        ),
        # The feature workload's distributions at d=256, on the 16x16-tile
        # kernels of wide feature dimensions.
        CloudWorkload(
            "feature256_64k", 65536, 65536, 256, (0.5,), 100,
            "normal(0, I/256)", "normal(0, I/256) + 0.3*u", "dirichlet",
            "n=m=65536, d=256, x,y~N(0,I/256), y shifted by 0.3 along a random unit vector, "
            "Dirichlet(1) weights, eps=0.5, 100 iterations",
        ),
        # The feature distributions at the size and the largest feature dimension
        # of the pages' dimension sweep (n = 50,000, d up to 1024; "FlashSinkhorn:
        # IO-Aware Entropic Optimal Transport on GPU", "Experimentelle
        # Ergebnisse"); the pages fix no iteration count there, 20 is this
        # workload's.
        CloudWorkload(
            "feature1024_50k", 50000, 50000, 1024, (0.5,), 20,
            "normal(0, I/1024)", "normal(0, I/1024) + 0.3*u", "dirichlet",
            "n=m=50000, d=1024, x,y~N(0,I/1024), y shifted by 0.3 along a random unit vector, "
            "Dirichlet(1) weights, eps=0.5, 20 iterations",
        ),
        # Same distributions as cube_gauss3d_16k at n=m=65536: the d=3 point at the
        # 65536 x 65536 size.
        CloudWorkload(
            "cube_gauss3d_64k", 65536, 65536, 3, (0.05,), 100,
            "uniform[0,1]^3", "normal(0.5*1, 0.1^2 I)", "uniform",
            "n=m=65536, d=3, x~U[0,1]^3, y~N(0.5*1,0.1^2 I), uniform weights, eps=0.05, 100 iterations",
        ),
    ]
}

BIRKHOFF_WORKLOADS: Dict[str, BirkhoffWorkload] = {
    w.name: w
    for w in [
        BirkhoffWorkload(
            "birkhoff4x4_1m", 1 << 20, (1.0, 10.0), 1.0, 200, 1e-6,
            "B=1,048,576 fp32 4x4 logits, first half N(0,1), second half N(0,10^2); "
            "eps=1, until max row/col-sum error <= 1e-6, capped at 200 iterations",
        ),
        BirkhoffWorkload(
            "birkhoff4x4_1m_fixed20", 1 << 20, (1.0, 10.0), 1.0, 20, -1.0,
            "as birkhoff4x4_1m but exactly 20 iterations",
        ),
    ]
}


def _f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def _weights(kind: str, size: int, rng: np.random.Generator) -> np.ndarray:
    if kind == "uniform":
        return np.full(size, 1.0 / size, dtype=np.float32)
    if kind == "dirichlet":
        w = _f32(rng.dirichlet(np.ones(size)))
        w64 = w.astype(np.float64)
        return _f32(w64 / w64.sum())
    raise ValueError(f"unknown weight kind {kind!r}")


def _mixture(rng: np.random.Generator, size: int, d: int, comps: int, sigma: float) -> np.ndarray:
    # Equal-weight components; centres i.i.d. Uniform([-1,1]^d) drawn first,
    # then component labels, then the isotropic noise.
    centres = rng.uniform(-1.0, 1.0, size=(comps, d))
    labels = rng.integers(0, comps, size=size)
    noise = rng.normal(0.0, sigma, size=(size, d))
    return centres[labels] + noise


def _sphere(rng: np.random.Generator, size: int, d: int) -> np.ndarray:
    z = rng.normal(size=(size, d))
    return z / np.linalg.norm(z, axis=1, keepdims=True)


def make_clouds(name: str, seed: int = 0, n: Optional[int] = None, m: Optional[int] = None,
                d: Optional[int] = None) -> dict:
    """Draw the inputs of a point-cloud workload.

    ``n`` and ``m`` override the workload's sizes (same distributions, same
    recipe) for smaller test cases; ``d`` overrides the feature dimension
    (meant for ``feature64_64k``, whose distributions are defined for any d).
    Returns a dict with fp32 ``x`` (n x d), ``y`` (m x d), ``a`` (n), ``b``
    (m) and the schedule ``eps`` (tuple) and ``iters`` (per stage).
    """
    w = CLOUD_WORKLOADS[name]
    n = w.n if n is None else int(n)
    m = w.m if m is None else int(m)
    d = w.d if d is None else int(d)
    rng = np.random.default_rng(seed)
    if name == "gauss3d_1k":
        x = rng.normal(0.0, 1.0, size=(n, d))
        y = rng.normal(0.5, 1.0, size=(m, d))
    elif name in ("cube_gauss3d_16k", "cube_gauss3d_64k"):
        x = rng.uniform(0.0, 1.0, size=(n, d))
        y = rng.normal(0.5, 0.1, size=(m, d))
    elif name in ("feature64_64k", "feature192_64k", "feature256_64k", "feature1024_50k"):
        x = rng.normal(0.0, 1.0 / math.sqrt(d), size=(n, d))
        y = rng.normal(0.0, 1.0 / math.sqrt(d), size=(m, d))
        z = rng.normal(size=d)
        y = y + 0.3 * (z / np.linalg.norm(z))
    elif name == "mixture_sphere3d_eps_scaling":
        x = _mixture(rng, n, d, comps=4, sigma=0.05)
        y = _sphere(rng, m, d)
    else:  # pragma: no cover - table and branches are kept in step
        raise KeyError(name)
    a = _weights(w.weights, n, rng)
    b = _weights(w.weights, m, rng)
    return {"x": _f32(x), "y": _f32(y), "a": a, "b": b, "eps": tuple(w.eps), "iters": w.iters,
            "name": name, "n": n, "m": m, "d": d}


def random_clouds(n: int, m: int, d: int, seed: int = 0, spread: float = 1.0,
                  weights: str = "dirichlet") -> dict:
    """Generic small clouds for edge-case tests: x ~ N(0, spread^2 I),
    y ~ N(0.25, spread^2 I), weights uniform or Dirichlet(1)."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, spread, size=(n, d))
    y = rng.normal(0.25, spread, size=(m, d))
    a = _weights(weights, n, rng)
    b = _weights(weights, m, rng)
    return {"x": _f32(x), "y": _f32(y), "a": a, "b": b}


def random_values(count: int, dv: int, seed: int = 0) -> np.ndarray:
    """Value matrix (count x dv, fp32) for the transport application: N(0, 1)."""
    rng = np.random.default_rng(seed)
    return _f32(rng.normal(size=(count, dv)))


def make_logits(batch: int, sigmas=(1.0, 10.0), seed: int = 0) -> np.ndarray:
    """Batched 4x4 logits, fp32, shape (batch, 4, 4). The batch is cut into
    ``len(sigmas)`` contiguous equal parts (the last takes the remainder); part
    ``p`` is N(0, sigmas[p]^2)."""
    rng = np.random.default_rng(seed)
    parts: List[np.ndarray] = []
    base = batch // len(sigmas)
    for p, s in enumerate(sigmas):
        cnt = base if p < len(sigmas) - 1 else batch - base * (len(sigmas) - 1)
        parts.append(rng.normal(0.0, s, size=(cnt, 4, 4)))
    return _f32(np.concatenate(parts, axis=0) if parts else np.zeros((0, 4, 4)))
