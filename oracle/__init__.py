"""fp64 CPU oracle for log-domain Sinkhorn -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package. The HIP library and its binding never do,
and the two share no code. Inputs are the fp32 arrays of ``workloads``,
upcast to fp64 here; every result is fp64.

The arithmetic lives in ``sinkhorn_oracle.c`` (plain C, OpenMP over rows),
which states the update it follows ("FlashSinkhorn: IO-Aware Entropic Optimal
Transport on GPU", Methodik section 1; the Birkhoff-projection page, section
2). This module only marshals arrays, plus thin compositions of those
functions: :func:`sinkhorn_schedule` runs stages of :func:`sinkhorn` one
after another (warm start); :func:`barycentric_map` and :func:`grad_x` combine
one :func:`transport_apply` with the weights or the points.

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``):

* ``half_update``, ``sinkhorn``: pinned (closed forms, marginal invariants,
  dual-solver fixed point, brute-force OT limit).
* ``plan_stats``: pinned (closed forms, product-coupling limit).
* ``sinkhorn_schedule``: pinned through properties only (stage composition,
  fixed point at the final eps); the schedule itself is not on the pages.
* ``birkhoff4``, ``birkhoff4_replay``: pinned (doubly-stochastic limit,
  cross-ratio invariant, constant and circulant logits, stopping rule).
* ``transport_apply``, ``barycentric_map``, ``grad_x``: pinned (n = 1 closed
  form, product-coupling limit, eps -> 0 permutation limit, finite
  differences of the converged dual value, marginal sums).
* ``sinkhorn_cosine``, ``plan_stats_cosine``: pinned (scale and rotation
  invariance, the unit-sphere identity with the squared Euclidean cost at
  twice the eps, n = 1 closed form, marginal invariants, cost range).
* ``birkhoff4_newton``: pinned (same limit as long Sinkhorn-Knopp runs,
  cross-ratio invariant, doubly stochastic, constant logits need no step,
  quadratic convergence).
* ``birkhoff4_backward``: pinned (central finite differences of <G, P(L)>
  with P from Sinkhorn-Knopp, zero row and column sums of dl/dL).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sinkhorn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile ``sinkhorn_oracle.c`` into ``liboracle.so`` with gcc (fp64, no
    fast-math, OpenMP). Returns the library path."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_half_update.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_double, _i64p, ctypes.c_int64, _dp]
        lib.oracle_sinkhorn.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp, _dp]
        lib.oracle_plan_stats.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                          _dp, _dp, _dp, _dp]
        lib.oracle_sinkhorn_kind.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_int, _dp,
                                             _dp, ctypes.c_int]
        lib.oracle_plan_stats_kind.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                               _dp, _dp, _dp, _dp, ctypes.c_int]
        lib.oracle_transport_apply.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int, ctypes.c_double, _dp, ctypes.c_int,
                                               _dp]
        lib.oracle_birkhoff4.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                         ctypes.c_double, _dp, _i32p]
        lib.oracle_birkhoff4_replay.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, _i32p,
                                                _dp, _dp]
        lib.oracle_birkhoff4_newton.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                                ctypes.c_double, _dp, _i32p]
        lib.oracle_birkhoff4_backward.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_double, _dp]
        _lib = lib
        return lib


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, t=_dp):
    return a.ctypes.data_as(t)


def _points(a, name):
    a = _d(a)
    if a.ndim == 1:
        a = a.reshape(-1, 1)
    if a.ndim != 2:
        raise ValueError(f"{name} must be (count, d)")
    return a


def half_update(P, Q, w, other, eps: float, rows=None) -> np.ndarray:
    """One half-step for the side with points ``P`` and weights ``w``:
    ``eps*log w_i - eps*LSE_j((other_j - |P_i - Q_j|^2)/eps)``. With ``rows``
    (indices) only those rows are computed, in that order."""
    P = _points(P, "P")
    Q = _points(Q, "Q")
    w, other = _d(w), _d(other)
    if P.shape[1] != Q.shape[1] or w.shape != (P.shape[0],) or other.shape != (Q.shape[0],):
        raise ValueError("shape mismatch")
    if rows is None:
        out = np.empty(P.shape[0])
        _load().oracle_half_update(_ptr(P), _ptr(Q), _ptr(w), _ptr(other), P.shape[0],
                                   Q.shape[0], P.shape[1], float(eps), None, 0, _ptr(out))
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if r.size and (r.min() < 0 or r.max() >= P.shape[0]):
            raise ValueError("row index out of range")
        out = np.empty(r.size)
        _load().oracle_half_update(_ptr(P), _ptr(Q), _ptr(w), _ptr(other), P.shape[0],
                                   Q.shape[0], P.shape[1], float(eps), _ptr(r, _i64p), r.size,
                                   _ptr(out))
    return out


def sinkhorn(x, y, a, b, eps: float, iters: int, f0=None, g0=None):
    """``iters`` alternating iterations (f then g) at one eps from (f0, g0);
    g0 defaults to zeros (cold start) and f0 is only overwritten. Returns
    (f, g) as fp64 arrays."""
    x, y = _points(x, "x"), _points(y, "y")
    a, b = _d(a), _d(b)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    if y.shape[1] != d or a.shape != (n,) or b.shape != (m,):
        raise ValueError("shape mismatch")
    f = np.zeros(n) if f0 is None else _d(f0).copy()
    g = np.zeros(m) if g0 is None else _d(g0).copy()
    _load().oracle_sinkhorn(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps), int(iters),
                            _ptr(f), _ptr(g))
    return f, g


def sinkhorn_schedule(x, y, a, b, eps_list, iters_per_stage: int, f0=None, g0=None):
    """Stages of :func:`sinkhorn`, one per eps in ``eps_list``, each starting
    from the previous stage's (f, g)."""
    f, g = f0, g0
    for e in eps_list:
        f, g = sinkhorn(x, y, a, b, e, iters_per_stage, f, g)
    return f, g


def plan_stats(x, y, a, b, f, g, eps: float) -> dict:
    """cost = sum P*C; marg_row = sum_i |sum_j P_ij - a_i|; marg_col likewise;
    rowsum, colsum; marg = marg_row + marg_col."""
    x, y = _points(x, "x"), _points(y, "y")
    a, b, f, g = _d(a), _d(b), _d(f), _d(g)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    cost = np.zeros(1)
    marg = np.zeros(2)
    rs = np.empty(n)
    cs = np.empty(m)
    _load().oracle_plan_stats(_ptr(x), _ptr(y), _ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m, d,
                              float(eps), _ptr(cost), _ptr(marg), _ptr(rs), _ptr(cs))
    return {"cost": float(cost[0]), "marg_row": float(marg[0]), "marg_col": float(marg[1]),
            "marg": float(marg[0] + marg[1]), "rowsum": rs, "colsum": cs}


def transport_apply(x, y, f, g, eps: float, v) -> np.ndarray:
    """out_i = sum_j P_ij v_j with P_ij = exp((f_i + g_j - |x_i - y_j|^2)/eps);
    v is (m,) or (m, dv). Returns (n,) or (n, dv)."""
    x, y = _points(x, "x"), _points(y, "y")
    f, g = _d(f), _d(g)
    v = _d(v)
    flat = v.ndim == 1
    v2 = v.reshape(v.shape[0], -1)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    if y.shape[1] != d or f.shape != (n,) or g.shape != (m,) or v2.shape[0] != m:
        raise ValueError("shape mismatch")
    out = np.empty((n, v2.shape[1]))
    _load().oracle_transport_apply(_ptr(x), _ptr(y), _ptr(f), _ptr(g), n, m, d, float(eps),
                                   _ptr(np.ascontiguousarray(v2)), v2.shape[1], _ptr(out))
    return out[:, 0] if flat else out


def barycentric_map(x, y, a, f, g, eps: float) -> np.ndarray:
    """T(x_i) = sum_j P_ij y_j / a_i (Methodik section 3)."""
    return transport_apply(x, y, f, g, eps, y) / _d(a)[:, None]


def grad_x(x, y, f, g, eps: float) -> np.ndarray:
    """d/dx_i of sum_ij P_ij C_ij at the fixed plan P of (f, g):
    2 sum_j P_ij (x_i - y_j) = 2 (r_i x_i - sum_j P_ij y_j). At the
    optimal (f, g) this is the gradient of OT_eps with respect to x_i."""
    x, y = _points(x, "x"), _points(y, "y")
    ones = np.ones((y.shape[0], 1))
    w = transport_apply(x, y, f, g, eps, np.hstack([y, ones]))
    return 2.0 * (w[:, -1:] * x - w[:, :-1])


def birkhoff4(logits, eps: float = 1.0, max_iters: int = 200, tol: float = 1e-6):
    """Project each 4x4 logit matrix L to exp((f_i + g_j + L_ij)/eps), iterating
    from g = 0 until the plan's worst row/column-sum error is <= tol (tol >= 0)
    or for exactly max_iters iterations (tol < 0). Returns (P, iters)."""
    L = _d(logits).reshape(-1, 16)
    B = L.shape[0]
    P = np.empty((B, 16))
    it = np.empty(B, dtype=np.int32)
    _load().oracle_birkhoff4(_ptr(L), B, float(eps), int(max_iters), float(tol), _ptr(P),
                             _ptr(it, _i32p))
    return P.reshape(B, 4, 4), it


def birkhoff4_replay(logits, iters, eps: float = 1.0):
    """Exactly ``iters[b]`` iterations for matrix b. Returns (P, err) where err
    is each plan's worst row/column-sum deviation from 1."""
    L = _d(logits).reshape(-1, 16)
    B = L.shape[0]
    it = np.ascontiguousarray(np.broadcast_to(np.asarray(iters, dtype=np.int32), (B,)))
    P = np.empty((B, 16))
    err = np.empty(B)
    _load().oracle_birkhoff4_replay(_ptr(L), B, float(eps), _ptr(it, _i32p), _ptr(P), _ptr(err))
    return P.reshape(B, 4, 4), err


def birkhoff4_newton(logits, eps: float = 1.0, max_iters: int = 50, tol: float = 1e-12):
    """Projection by Newton's method on the 3-variable dual (Birkhoff page,
    section 2.1), from g = 0 with a backtracking line search; stops before a
    step once the worst column-sum error is <= tol (tol < 0: exactly
    max_iters steps). Returns (P, steps)."""
    L = _d(logits).reshape(-1, 16)
    B = L.shape[0]
    P = np.empty((B, 16))
    it = np.empty(B, dtype=np.int32)
    _load().oracle_birkhoff4_newton(_ptr(L), B, float(eps), int(max_iters), float(tol), _ptr(P),
                                    _ptr(it, _i32p))
    return P.reshape(B, 4, 4), it


def birkhoff4_backward(P, grad_P, eps: float = 1.0) -> np.ndarray:
    """dl/dL for the projection P of L and dl/dP = grad_P, by implicit
    differentiation at the solution (Birkhoff page, section 2.2)."""
    Pd = _d(P).reshape(-1, 16)
    G = _d(grad_P).reshape(-1, 16)
    if Pd.shape != G.shape:
        raise ValueError("shape mismatch")
    out = np.empty_like(Pd)
    _load().oracle_birkhoff4_backward(_ptr(Pd), _ptr(G), Pd.shape[0], float(eps), _ptr(out))
    return out.reshape(-1, 4, 4)


def sinkhorn_cosine(x, y, a, b, eps: float, iters: int, f0=None, g0=None):
    """:func:`sinkhorn` with the cosine cost C_ij = 1 - x_i.y_j / (|x_i| |y_j|)
    (FlashSinkhorn page, significance section)."""
    x, y = _points(x, "x"), _points(y, "y")
    a, b = _d(a), _d(b)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    if y.shape[1] != d or a.shape != (n,) or b.shape != (m,):
        raise ValueError("shape mismatch")
    f = np.zeros(n) if f0 is None else _d(f0).copy()
    g = np.zeros(m) if g0 is None else _d(g0).copy()
    _load().oracle_sinkhorn_kind(_ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps),
                                 int(iters), _ptr(f), _ptr(g), 1)
    return f, g


def plan_stats_cosine(x, y, a, b, f, g, eps: float) -> dict:
    """:func:`plan_stats` with the cosine cost."""
    x, y = _points(x, "x"), _points(y, "y")
    a, b, f, g = _d(a), _d(b), _d(f), _d(g)
    n, m, d = x.shape[0], y.shape[0], x.shape[1]
    cost = np.zeros(1)
    marg = np.zeros(2)
    rs = np.empty(n)
    cs = np.empty(m)
    _load().oracle_plan_stats_kind(_ptr(x), _ptr(y), _ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m,
                                   d, float(eps), _ptr(cost), _ptr(marg), _ptr(rs), _ptr(cs), 1)
    return {"cost": float(cost[0]), "marg_row": float(marg[0]), "marg_col": float(marg[1]),
            "marg": float(marg[0] + marg[1]), "rowsum": rs, "colsum": cs}
