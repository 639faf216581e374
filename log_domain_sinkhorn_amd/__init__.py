"""Python binding of the gfx950 log-domain Sinkhorn library (``libotsinkhorn.so``).

Each function has the name of the C entry point it wraps (declared in
``include/ot_sinkhorn.h``) and only marshals arguments: it checks that the
tensors are contiguous fp32 (int32 / fp64 where stated) CUDA tensors of the
right sizes, passes their data pointers and the current HIP stream of their
device, and raises :class:`OTError` on a non-success status. Every step of the
computation runs in the library's HIP kernels; there is no other path. If the
library has not been built, importing a function's first use raises
:class:`RuntimeError` instead of falling back to anything.

The math follows "FlashSinkhorn: IO-Aware Entropic Optimal Transport on GPU"
(Methodik sections 1-3) and, for the 4x4 case, the Birkhoff-projection page
(sections 1-2); see the header for the exact conventions.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

__all__ = [
    "OTError",
    "library_path",
    "load_library",
    "declared_functions",
    "ot_status_string",
    "ot_sinkhorn_solve",
    "ot_sinkhorn_solve_eps_scaling",
    "ot_sinkhorn_solve_no_alloc",
    "ot_plan_stats",
    "ot_plan_cost",
    "ot_marginal_error",
    "ot_sinkhorn_solve_cosine",
    "ot_plan_stats_cosine",
    "ot_transport_apply",
    "ot_barycentric_map",
    "ot_cost_gradient_x",
    "ot_birkhoff_project_batched",
    "ot_birkhoff_project_newton_batched",
    "ot_birkhoff_projection_backward_batched",
    "OT_MAX_DIM",
    "OT_MAX_TRANSPORT_DIM",
    "OT_MAX_VALUE_DIM",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_HEADER = os.path.join(_ROOT, "include", "ot_sinkhorn.h")
_LIB = os.path.join(_HERE, "libotsinkhorn.so")

OT_SUCCESS = 0
OT_ERROR_INVALID_VALUE = 1
OT_ERROR_NOT_SUPPORTED = 2
OT_ERROR_OUT_OF_MEMORY = 3
OT_ERROR_LAUNCH_FAILURE = 4
OT_MAX_DIM = 1024
OT_MAX_TRANSPORT_DIM = 1024
OT_MAX_VALUE_DIM = 1024
OT_NO_ALLOC_SCRATCH_BYTES = 128 << 20

_lock = threading.Lock()
_handle = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float

_SIGNATURES = {
    "ot_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "ot_sinkhorn_solve": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _i32, _p, _p, _p], ctypes.c_int),
    "ot_sinkhorn_solve_no_alloc": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _i32, _p, _p, _p],
                                   ctypes.c_int),
    "ot_sinkhorn_solve_eps_scaling": (
        [_p, _p, _p, _p, _i64, _i64, _i32, _f32, _f32, _i32, _i32, _p, _p, _p], ctypes.c_int),
    "ot_plan_stats": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p, _p], ctypes.c_int),
    "ot_plan_cost": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p], ctypes.c_int),
    "ot_marginal_error": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p], ctypes.c_int),
    "ot_sinkhorn_solve_cosine": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _i32, _p, _p, _p],
                                 ctypes.c_int),
    "ot_plan_stats_cosine": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p, _p],
                             ctypes.c_int),
    "ot_transport_apply": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _i32, _p, _p],
                           ctypes.c_int),
    "ot_barycentric_map": ([_p, _p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p], ctypes.c_int),
    "ot_cost_gradient_x": ([_p, _p, _p, _p, _i64, _i64, _i32, _f32, _p, _p], ctypes.c_int),
    "ot_birkhoff_project_batched": ([_p, _i64, _f32, _i32, _f32, _p, _p, _p], ctypes.c_int),
    "ot_birkhoff_project_newton_batched": ([_p, _i64, _f32, _i32, _f32, _p, _p, _p],
                                           ctypes.c_int),
    "ot_birkhoff_projection_backward_batched": ([_p, _p, _i64, _f32, _p, _p], ctypes.c_int),
}


class OTError(RuntimeError):
    """A library call returned a status other than OT_SUCCESS."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {_status_name(status)} ({status})")


def library_path() -> str:
    return _LIB


def declared_functions():
    """Names of the functions ``include/ot_sinkhorn.h`` declares."""
    text = open(_HEADER).read()
    return sorted(set(re.findall(r"^(?:const\s+char\s*\*|ot_status)\s*\**\s*(ot_\w+)\s*\(",
                                 text, flags=re.M)))


def load_library():
    """Load ``libotsinkhorn.so`` (built in-tree) and set the C signatures."""
    global _handle
    with _lock:
        if _handle is not None:
            return _handle
        if not os.path.exists(_LIB):
            raise RuntimeError(
                f"{_LIB} is missing: build it with `python -m log_domain_sinkhorn_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(_LIB)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _handle = lib
        return lib


def _status_name(status: int) -> str:
    try:
        return load_library().ot_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - only when the library itself is absent
        return f"status {status}"


def ot_status_string(status: int) -> str:
    return load_library().ot_status_string(int(status)).decode()


def _call(name: str, *args) -> None:
    st = getattr(load_library(), name)(*args)
    if st != OT_SUCCESS:
        raise OTError(name, st)


# --------------------------------------------------------------------------- #
# argument marshalling                                                         #
# --------------------------------------------------------------------------- #

def _torch():
    import torch

    return torch


def _dev_tensor(t, name: str, dtype_name: str, shape=None):
    torch = _torch()
    dtype = {"f32": torch.float32, "f64": torch.float64, "i32": torch.int32}[dtype_name]
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_of(t, stream) -> Optional[int]:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _clouds(x, y):
    x = _dev_tensor(x, "x", "f32")
    y = _dev_tensor(y, "y", "f32")
    if x.dim() != 2 or y.dim() != 2 or x.shape[1] != y.shape[1]:
        raise ValueError("x and y must be (n, d) and (m, d)")
    if x.device != y.device:
        raise ValueError("x and y must be on one device")
    return x.shape[0], y.shape[0], x.shape[1]


# --------------------------------------------------------------------------- #
# entry points                                                                 #
# --------------------------------------------------------------------------- #

def ot_sinkhorn_solve(x, y, a, b, eps: float, iters: int, f, g, stream=None) -> None:
    """``iters`` alternating log-domain Sinkhorn iterations; f and g are in/out."""
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _call("ot_sinkhorn_solve", _ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps),
          int(iters), _ptr(f), _ptr(g), _stream_of(x, stream))


def ot_sinkhorn_solve_no_alloc(x, y, a, b, eps: float, iters: int, f, g, stream=None) -> None:
    """:func:`ot_sinkhorn_solve` with its scratch in the library's static device
    array (no allocation); NOT_SUPPORTED when the problem's scratch exceeds
    ``OT_NO_ALLOC_SCRATCH_BYTES``. Calls on one GPU must not overlap."""
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _call("ot_sinkhorn_solve_no_alloc", _ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d,
          float(eps), int(iters), _ptr(f), _ptr(g), _stream_of(x, stream))


def ot_sinkhorn_solve_eps_scaling(x, y, a, b, eps0: float, eps_end: float, stages: int,
                                  iters_per_stage: int, f, g, stream=None) -> None:
    """Geometric eps schedule eps0 -> eps_end over ``stages`` warm-started solves."""
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _call("ot_sinkhorn_solve_eps_scaling", _ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d,
          float(eps0), float(eps_end), int(stages), int(iters_per_stage), _ptr(f), _ptr(g),
          _stream_of(x, stream))


def ot_plan_stats(x, y, a, b, f, g, eps: float, cost=None, marg=None, stream=None) -> None:
    """Write cost (fp64 [1]) and/or marg (fp64 [2]) of the plan of (f, g)."""
    n, m, d = _clouds(x, y)
    if a is not None:
        _dev_tensor(a, "a", "f32", (n,))
    if b is not None:
        _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    if cost is not None:
        _dev_tensor(cost, "cost", "f64", (1,))
    if marg is not None:
        _dev_tensor(marg, "marg", "f64", (2,))
    _call("ot_plan_stats", _ptr(x), _ptr(y), _ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m, d,
          float(eps), _ptr(cost), _ptr(marg), _stream_of(x, stream))


def ot_plan_cost(x, y, f, g, eps: float, cost, stream=None) -> None:
    n, m, d = _clouds(x, y)
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _dev_tensor(cost, "cost", "f64", (1,))
    _call("ot_plan_cost", _ptr(x), _ptr(y), _ptr(f), _ptr(g), n, m, d, float(eps), _ptr(cost),
          _stream_of(x, stream))


def ot_marginal_error(x, y, a, b, f, g, eps: float, marg, stream=None) -> None:
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _dev_tensor(marg, "marg", "f64", (2,))
    _call("ot_marginal_error", _ptr(x), _ptr(y), _ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m, d,
          float(eps), _ptr(marg), _stream_of(x, stream))


def ot_sinkhorn_solve_cosine(x, y, a, b, eps: float, iters: int, f, g, stream=None) -> None:
    """:func:`ot_sinkhorn_solve` with the cosine cost 1 - cos(x_i, y_j)."""
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _call("ot_sinkhorn_solve_cosine", _ptr(x), _ptr(y), _ptr(a), _ptr(b), n, m, d, float(eps),
          int(iters), _ptr(f), _ptr(g), _stream_of(x, stream))


def ot_plan_stats_cosine(x, y, a, b, f, g, eps: float, cost=None, marg=None,
                         stream=None) -> None:
    """:func:`ot_plan_stats` with the cosine cost."""
    n, m, d = _clouds(x, y)
    if a is not None:
        _dev_tensor(a, "a", "f32", (n,))
    if b is not None:
        _dev_tensor(b, "b", "f32", (m,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    if cost is not None:
        _dev_tensor(cost, "cost", "f64", (1,))
    if marg is not None:
        _dev_tensor(marg, "marg", "f64", (2,))
    _call("ot_plan_stats_cosine", _ptr(x), _ptr(y), _ptr(a), _ptr(b), _ptr(f), _ptr(g), n, m, d,
          float(eps), _ptr(cost), _ptr(marg), _stream_of(x, stream))


def ot_transport_apply(x, y, f, g, eps: float, v, out, stream=None) -> None:
    """out (n, dv) = P v for v (m, dv), P_ij = exp((f_i + g_j - |x_i - y_j|^2)/eps)."""
    n, m, d = _clouds(x, y)
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _dev_tensor(v, "v", "f32")
    if v.dim() != 2 or v.shape[0] != m:
        raise ValueError("v must be (m, dv)")
    dv = v.shape[1]
    _dev_tensor(out, "out", "f32", (n, dv))
    _call("ot_transport_apply", _ptr(x), _ptr(y), _ptr(f), _ptr(g), n, m, d, float(eps), _ptr(v),
          dv, _ptr(out), _stream_of(x, stream))


def ot_barycentric_map(x, y, a, f, g, eps: float, out, stream=None) -> None:
    """out (n, d): T(x_i) = sum_j P_ij y_j / a_i."""
    n, m, d = _clouds(x, y)
    _dev_tensor(a, "a", "f32", (n,))
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _dev_tensor(out, "out", "f32", (n, d))
    _call("ot_barycentric_map", _ptr(x), _ptr(y), _ptr(a), _ptr(f), _ptr(g), n, m, d, float(eps),
          _ptr(out), _stream_of(x, stream))


def ot_cost_gradient_x(x, y, f, g, eps: float, out, stream=None) -> None:
    """out (n, d): 2 (r_i x_i - sum_j P_ij y_j) with r_i = sum_j P_ij."""
    n, m, d = _clouds(x, y)
    _dev_tensor(f, "f", "f32", (n,))
    _dev_tensor(g, "g", "f32", (m,))
    _dev_tensor(out, "out", "f32", (n, d))
    _call("ot_cost_gradient_x", _ptr(x), _ptr(y), _ptr(f), _ptr(g), n, m, d, float(eps),
          _ptr(out), _stream_of(x, stream))


def ot_birkhoff_project_batched(logits, eps: float, max_iters: int, tol: float, out,
                                iters_out=None, stream=None) -> None:
    """Project each 4x4 matrix of ``logits`` (batch, 4, 4) into ``out`` (may be
    ``logits`` itself); ``iters_out`` (int32 [batch]) gets the iterations run."""
    _dev_tensor(logits, "logits", "f32")
    if logits.dim() != 3 or tuple(logits.shape[1:]) != (4, 4):
        raise ValueError("logits must be (batch, 4, 4)")
    batch = logits.shape[0]
    _dev_tensor(out, "out", "f32", (batch, 4, 4))
    if iters_out is not None:
        _dev_tensor(iters_out, "iters_out", "i32", (batch,))
    _call("ot_birkhoff_project_batched", _ptr(logits), batch, float(eps), int(max_iters),
          float(tol), _ptr(out), _ptr(iters_out), _stream_of(logits, stream))


def ot_birkhoff_project_newton_batched(logits, eps: float, max_iters: int, tol: float, out,
                                       iters_out=None, stream=None) -> None:
    """Newton's method on the 3-variable dual; same arguments as
    :func:`ot_birkhoff_project_batched` (``iters_out`` gets Newton steps)."""
    _dev_tensor(logits, "logits", "f32")
    if logits.dim() != 3 or tuple(logits.shape[1:]) != (4, 4):
        raise ValueError("logits must be (batch, 4, 4)")
    batch = logits.shape[0]
    _dev_tensor(out, "out", "f32", (batch, 4, 4))
    if iters_out is not None:
        _dev_tensor(iters_out, "iters_out", "i32", (batch,))
    _call("ot_birkhoff_project_newton_batched", _ptr(logits), batch, float(eps), int(max_iters),
          float(tol), _ptr(out), _ptr(iters_out), _stream_of(logits, stream))


def ot_birkhoff_projection_backward_batched(plan, grad_plan, eps: float, grad_logits,
                                            stream=None) -> None:
    """dl/dL (batch, 4, 4) from the projection ``plan`` and dl/dP ``grad_plan``."""
    _dev_tensor(plan, "plan", "f32")
    if plan.dim() != 3 or tuple(plan.shape[1:]) != (4, 4):
        raise ValueError("plan must be (batch, 4, 4)")
    batch = plan.shape[0]
    _dev_tensor(grad_plan, "grad_plan", "f32", (batch, 4, 4))
    _dev_tensor(grad_logits, "grad_logits", "f32", (batch, 4, 4))
    _call("ot_birkhoff_projection_backward_batched", _ptr(plan), _ptr(grad_plan), batch,
          float(eps), _ptr(grad_logits), _stream_of(plan, stream))
