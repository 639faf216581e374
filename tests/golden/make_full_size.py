"""Write the full-size oracle fixtures the GPU parity tests compare against.

Calls only the fp64 oracle (``oracle/``) and the seeded input generators
(``workloads/``); nothing here touches the HIP library.

For each point-cloud workload named on the command line it draws the inputs,
runs the oracle's alternating log-domain Sinkhorn iterations over the whole
workload (every stage of an eps schedule, warm-started) from a cold start,
and stores in ``tests/golden/full_<workload>.npz``
(``tests/golden/<workload>_<n>x<m>.npz`` when the workload is named as
``<workload>@<n>x<m>``: the same distributions, schedule and iteration count
at a smaller size):

* ``f``, ``g``      the oracle's final potentials (fp64);
* ``cost``, ``marg_row``, ``marg_col``  the oracle's plan statistics of those
  potentials at the last eps ("transport cost" = sum_ij P_ij C_ij, marginal
  errors = L1 norms of row and column sums minus a and b);
* ``cost32``, ``marg_row32``, ``marg_col32``  the same statistics of the
  potentials rounded to fp32 (the inputs a GPU statistics call takes), so the
  statistics kernels can be compared on identical inputs;
* ``key``           sha256 of the inputs and the schedule; the tests redraw
  the inputs and refuse a fixture whose key does not match.

The update followed is the one of "FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU" (Methodik, section 1), in the oracle's convention; the eps
schedule is the workload's own (not on the pages).

The run is long (hours for the 65536 x 65536 x 64 and 131072 x 98304
workloads), so it checkpoints (f, g, position in the schedule) every
``--chunk`` iterations into ``--ckpt-dir`` and resumes from there. Running a
schedule in chunks is exactly the same computation as one long run: the
oracle updates f and g in place, half-step after half-step.

Usage:  python tests/golden/make_full_size.py cube_gauss3d_16k feature64_64k \
            mixture_sphere3d_eps_scaling@65536x49152
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import tempfile
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import make_clouds  # noqa: E402


def input_key(c: dict) -> str:
    """sha256 over the fp32 inputs, the eps schedule and the iteration count."""
    h = hashlib.sha256()
    for k in ("x", "y", "a", "b"):
        arr = np.ascontiguousarray(c[k])
        h.update(k.encode())
        h.update(str(arr.shape).encode())
        h.update(arr.tobytes())
    h.update(repr(tuple(float(e) for e in c["eps"])).encode())
    h.update(str(int(c["iters"])).encode())
    return h.hexdigest()


def fixture_path(name: str, n=None, m=None) -> str:
    if n is None:
        return os.path.join(HERE, f"full_{name}.npz")
    return os.path.join(HERE, f"{name}_{n}x{m}.npz")


def parse_spec(spec: str):
    """``name`` or ``name@NxM`` -> (name, n or None, m or None)."""
    if "@" not in spec:
        return spec, None, None
    name, size = spec.split("@", 1)
    n, m = size.lower().split("x")
    return name, int(n), int(m)


def _save_atomic(path: str, **arrays) -> None:
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrays)
    os.replace(tmp, path)


def run(spec: str, ckpt_dir: str, chunk: int) -> None:
    name, n_over, m_over = parse_spec(spec)
    c = make_clouds(name, n=n_over, m=m_over)
    out_path = fixture_path(name, n_over, m_over)
    tag = os.path.splitext(os.path.basename(out_path))[0]
    key = input_key(c)
    eps_list = [float(e) for e in c["eps"]]
    iters = int(c["iters"])
    total = iters * len(eps_list)
    os.makedirs(ckpt_dir, exist_ok=True)
    ck = os.path.join(ckpt_dir, f"ckpt_{tag}.npz")
    done, f, g = 0, np.zeros(c["n"]), np.zeros(c["m"])
    if os.path.exists(ck):
        z = np.load(ck)
        if str(z["key"]) == key:
            done, f, g = int(z["done"]), z["f"].copy(), z["g"].copy()
            print(f"[{name}] resuming at iteration {done}/{total}", flush=True)
    t0 = time.time()
    while done < total:
        stage, it = divmod(done, iters)
        k = min(chunk, iters - it)
        f, g = oracle.sinkhorn(c["x"], c["y"], c["a"], c["b"], eps_list[stage], k, f, g)
        done += k
        _save_atomic(ck, key=key, done=done, f=f, g=g)
        print(f"[{name}] {done}/{total} iterations (stage {stage}, eps {eps_list[stage]:.6g}), "
              f"{time.time() - t0:.0f} s", flush=True)
    eps = eps_list[-1]
    s64 = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f, g, eps)
    f32 = f.astype(np.float32).astype(np.float64)
    g32 = g.astype(np.float32).astype(np.float64)
    s32 = oracle.plan_stats(c["x"], c["y"], c["a"], c["b"], f32, g32, eps)
    _save_atomic(out_path, key=key, name=name, n=c["n"], m=c["m"], f=f, g=g,
                 eps=np.array(eps_list),
                 iters=iters, cost=s64["cost"], marg_row=s64["marg_row"],
                 marg_col=s64["marg_col"], cost32=s32["cost"], marg_row32=s32["marg_row"],
                 marg_col32=s32["marg_col"], oracle_threads=oracle.num_threads())
    print(f"[{name}] wrote {out_path}: cost {s64['cost']:.12g}, "
          f"marg {s64['marg_row']:.3e} + {s64['marg_col']:.3e}", flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--ckpt-dir", default=os.path.join(tempfile.gettempdir(), "ot_golden_ckpt"))
    ap.add_argument("--chunk", type=int, default=5, help="iterations between checkpoints")
    args = ap.parse_args()
    oracle.build(force=False)
    for spec in args.workloads:
        run(spec, args.ckpt_dir, args.chunk)
    return 0


if __name__ == "__main__":
    sys.exit(main())
