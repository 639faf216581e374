"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device.
Only calls that fail host validation are made here (no device is needed)."""
import ctypes
import math

import pytest

import log_domain_sinkhorn_amd as lds

INVALID = lds.OT_ERROR_INVALID_VALUE
UNSUPPORTED = lds.OT_ERROR_NOT_SUPPORTED

# Distinct fake, non-overlapping, 256-byte aligned addresses: never dereferenced
# because every call below fails validation first.
X, Y, A, B, F, G, C, MG = (0x10000000 * k for k in range(1, 9))


@pytest.fixture(scope="module")
def lib():
    return lds.load_library()


def test_header_declares_expected_functions():
    assert lds.declared_functions() == sorted([
        "ot_status_string", "ot_sinkhorn_solve", "ot_sinkhorn_solve_eps_scaling",
        "ot_plan_stats", "ot_plan_cost", "ot_marginal_error", "ot_birkhoff_project_batched",
        "ot_transport_apply", "ot_barycentric_map", "ot_cost_gradient_x",
        "ot_birkhoff_project_newton_batched", "ot_birkhoff_projection_backward_batched",
        "ot_sinkhorn_solve_cosine", "ot_plan_stats_cosine", "ot_sinkhorn_solve_no_alloc",
    ])


def test_every_declared_function_is_exported(lib):
    for name in lds.declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_header_max_dim_matches_binding():
    text = open(lds._HEADER).read()
    assert f"#define OT_MAX_DIM {lds.OT_MAX_DIM}" in text
    assert f"#define OT_MAX_TRANSPORT_DIM {lds.OT_MAX_TRANSPORT_DIM}" in text
    assert f"#define OT_MAX_VALUE_DIM {lds.OT_MAX_VALUE_DIM}" in text
    assert "#define OT_NO_ALLOC_SCRATCH_BYTES (128ull << 20)" in text
    assert lds.OT_NO_ALLOC_SCRATCH_BYTES == 128 << 20


def test_no_alloc_refuses_scratch_beyond_the_array_on_the_host(lib):
    # 65536 x 65536 at d = 128 needs 133.5 MiB of scratch, more than the
    # 128 MiB array: refused by the host-side size check before any HIP
    # call, so placeholder addresses (far apart, never dereferenced) suffice.
    n, d = 65536, 128
    base = 1 << 44
    step = 1 << 36
    ptrs = [ctypes.c_void_p(base + k * step) for k in range(6)]
    st = lib.ot_sinkhorn_solve_no_alloc(ptrs[0], ptrs[1], ptrs[2], ptrs[3], n, n, d,
                                        ctypes.c_float(0.5), 1, ptrs[4], ptrs[5], None)
    assert st == UNSUPPORTED
    # 65536 x 65536 at d = 64 fits (69.25 MiB): with iters = 0 the call
    # returns success without touching the device
    st = lib.ot_sinkhorn_solve_no_alloc(ptrs[0], ptrs[1], ptrs[2], ptrs[3], n, n, 64,
                                        ctypes.c_float(0.5), 0, ptrs[4], ptrs[5], None)
    assert st == 0


def test_status_strings(lib):
    assert lds.ot_status_string(0) == "OT_SUCCESS"
    assert lds.ot_status_string(INVALID) == "OT_ERROR_INVALID_VALUE"
    assert lds.ot_status_string(UNSUPPORTED) == "OT_ERROR_NOT_SUPPORTED"
    assert lds.ot_status_string(3) == "OT_ERROR_OUT_OF_MEMORY"
    assert lds.ot_status_string(4) == "OT_ERROR_LAUNCH_FAILURE"
    assert lds.ot_status_string(99) == "OT_ERROR_UNKNOWN"


def solve(lib, x=X, y=Y, a=A, b=B, n=10, m=12, d=3, eps=0.1, iters=5, f=F, g=G):
    return lib.ot_sinkhorn_solve(x, y, a, b, n, m, d, eps, iters, f, g, None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(y=None), dict(a=None), dict(b=None), dict(f=None), dict(g=None),
    dict(n=0), dict(m=0), dict(n=-3), dict(d=0), dict(eps=0.0), dict(eps=-1.0),
    dict(eps=math.inf), dict(eps=math.nan), dict(iters=-1),
    dict(f=A), dict(g=X), dict(f=G),            # outputs alias inputs / each other
])
def test_solve_rejects_invalid(lib, kw):
    assert solve(lib, **kw) == INVALID


def test_solve_invalid_beats_unsupported(lib):
    assert solve(lib, d=lds.OT_MAX_DIM + 1, eps=-1.0) == INVALID


def test_solve_unsupported_dim(lib):
    assert solve(lib, d=lds.OT_MAX_DIM + 1) == UNSUPPORTED


def test_eps_scaling_rejects_invalid(lib):
    f = lib.ot_sinkhorn_solve_eps_scaling
    assert f(X, Y, A, B, 10, 12, 3, 1.0, 0.01, 0, 5, F, G, None) == INVALID   # stages < 1
    assert f(X, Y, A, B, 10, 12, 3, 1.0, 0.0, 8, 5, F, G, None) == INVALID    # eps_end
    assert f(X, Y, A, B, 10, 12, 3, math.nan, 0.1, 8, 5, F, G, None) == INVALID
    assert f(X, Y, A, B, 10, 12, 3, 1.0, 0.1, 8, -1, F, G, None) == INVALID
    assert f(X, Y, A, B, 10, 12, lds.OT_MAX_DIM + 1, 1.0, 0.1, 8, 5, F, G, None) == UNSUPPORTED


def test_plan_stats_rejects_invalid(lib):
    ps = lib.ot_plan_stats
    assert ps(X, Y, A, B, F, G, 10, 12, 3, 0.1, None, None, None) == INVALID   # no output
    assert ps(X, Y, None, B, F, G, 10, 12, 3, 0.1, None, MG, None) == INVALID  # marg needs a
    assert ps(X, Y, A, B, None, G, 10, 12, 3, 0.1, C, None, None) == INVALID
    assert ps(X, Y, A, B, F, G, 10, 12, 3, 0.0, C, None, None) == INVALID
    assert ps(X, Y, A, B, F, G, 10, 12, lds.OT_MAX_DIM + 1, 0.1, C, None, None) == UNSUPPORTED
    assert lib.ot_plan_cost(X, Y, F, G, 10, 12, 3, 0.1, None, None) == INVALID
    assert lib.ot_marginal_error(X, Y, A, B, F, G, 10, 12, 3, 0.1, None, None) == INVALID
    assert lib.ot_marginal_error(X, Y, None, B, F, G, 10, 12, 3, 0.1, MG, None) == INVALID


V, OUT = 0x90000000, 0xA0000000


def test_transport_apply_rejects_invalid(lib):
    ta = lib.ot_transport_apply
    ok = dict(x=X, y=Y, f=F, g=G, n=10, m=12, d=3, eps=0.1, v=V, dv=5, out=OUT)

    def call(**kw):
        a = {**ok, **kw}
        return ta(a["x"], a["y"], a["f"], a["g"], a["n"], a["m"], a["d"], a["eps"], a["v"],
                  a["dv"], a["out"], None)

    for kw in [dict(x=None), dict(f=None), dict(g=None), dict(v=None), dict(out=None),
               dict(n=0), dict(m=-1), dict(d=0), dict(dv=0), dict(eps=0.0), dict(eps=math.nan),
               dict(out=X), dict(out=V + 8), dict(out=F - 16)]:
        assert call(**kw) == INVALID, kw
    assert call(d=lds.OT_MAX_DIM + 1) == UNSUPPORTED
    assert call(d=lds.OT_MAX_TRANSPORT_DIM + 1) == UNSUPPORTED
    assert call(dv=lds.OT_MAX_VALUE_DIM + 1) == UNSUPPORTED
    assert call(dv=lds.OT_MAX_VALUE_DIM + 1, eps=-1.0) == INVALID


def test_map_and_gradient_reject_invalid(lib):
    bm, gx = lib.ot_barycentric_map, lib.ot_cost_gradient_x
    assert bm(X, Y, None, F, G, 10, 12, 3, 0.1, OUT, None) == INVALID      # map needs a
    assert bm(X, Y, A, F, G, 10, 12, 3, 0.1, None, None) == INVALID
    assert bm(X, Y, A, F, G, 10, 12, 3, 0.1, A, None) == INVALID           # out aliases a
    assert bm(X, Y, A, F, G, 0, 12, 3, 0.1, OUT, None) == INVALID
    assert bm(X, Y, A, F, G, 10, 12, lds.OT_MAX_DIM + 1, 0.1, OUT, None) == UNSUPPORTED
    assert gx(X, Y, None, G, 10, 12, 3, 0.1, OUT, None) == INVALID
    assert gx(X, Y, F, G, 10, 12, 3, 0.1, Y + 4, None) == INVALID          # out overlaps y
    assert gx(X, Y, F, G, 10, 12, 3, -0.1, OUT, None) == INVALID
    assert gx(X, Y, F, G, 10, 12, lds.OT_MAX_DIM + 1, 0.1, OUT, None) == UNSUPPORTED
    # the transport calls cover the solve's whole range of d
    assert lds.OT_MAX_TRANSPORT_DIM == lds.OT_MAX_DIM


def test_birkhoff_rejects_invalid(lib):
    bp = lib.ot_birkhoff_project_batched
    assert bp(None, 4, 1.0, 20, -1.0, F, None, None) == INVALID
    assert bp(X, 4, 1.0, 20, -1.0, None, None, None) == INVALID
    assert bp(X, -1, 1.0, 20, -1.0, F, None, None) == INVALID
    assert bp(X, 4, 0.0, 20, -1.0, F, None, None) == INVALID
    assert bp(X, 4, 1.0, -1, -1.0, F, None, None) == INVALID
    assert bp(X, 4, 1.0, 20, math.nan, F, None, None) == INVALID
    assert bp(X + 4, 4, 1.0, 20, -1.0, F, None, None) == INVALID          # misaligned
    assert bp(X, 4, 1.0, 20, -1.0, X + 64, None, None) == INVALID         # partial overlap
    assert bp(X, 4, 1.0, 20, -1.0, F, X + 16, None) == INVALID            # counts overlap
    # batch == 0 is a valid no-op that never touches the device
    assert bp(X, 0, 1.0, 20, -1.0, F, None, None) == 0


def test_birkhoff_newton_rejects_invalid(lib):
    bn = lib.ot_birkhoff_project_newton_batched
    assert bn(None, 4, 1.0, 20, 1e-6, F, None, None) == INVALID
    assert bn(X, 4, 1.0, 20, 1e-6, None, None, None) == INVALID
    assert bn(X, -2, 1.0, 20, 1e-6, F, None, None) == INVALID
    assert bn(X, 4, math.inf, 20, 1e-6, F, None, None) == INVALID
    assert bn(X, 4, 1.0, -1, 1e-6, F, None, None) == INVALID
    assert bn(X, 4, 1.0, 20, math.nan, F, None, None) == INVALID
    assert bn(X + 8, 4, 1.0, 20, 1e-6, F, None, None) == INVALID
    assert bn(X, 4, 1.0, 20, 1e-6, X + 32, None, None) == INVALID
    assert bn(X, 4, 1.0, 20, 1e-6, F, F + 4, None) == INVALID
    assert bn(X, 0, 1.0, 20, 1e-6, F, None, None) == 0


def test_birkhoff_backward_rejects_invalid(lib):
    bw = lib.ot_birkhoff_projection_backward_batched
    assert bw(None, G, 4, 1.0, F, None) == INVALID
    assert bw(X, None, 4, 1.0, F, None) == INVALID
    assert bw(X, G, 4, 1.0, None, None) == INVALID
    assert bw(X, G, -1, 1.0, F, None) == INVALID
    assert bw(X, G, 4, 0.0, F, None) == INVALID
    assert bw(X + 4, G, 4, 1.0, F, None) == INVALID
    assert bw(X, G, 4, 1.0, X + 16, None) == INVALID      # partial overlap with plan
    assert bw(X, G, 4, 1.0, G - 16, None) == INVALID      # partial overlap with grad_plan
    assert bw(X, G, 0, 1.0, F, None) == 0
    assert bw(X, G, 0, 1.0, X, None) == 0                 # exact aliasing is allowed


def test_cosine_entries_reject_invalid(lib):
    sc, pc = lib.ot_sinkhorn_solve_cosine, lib.ot_plan_stats_cosine
    assert sc(None, Y, A, B, 10, 12, 3, 0.1, 5, F, G, None) == INVALID
    assert sc(X, Y, A, B, 10, 12, 3, 0.0, 5, F, G, None) == INVALID
    assert sc(X, Y, A, B, 10, 12, 3, 0.1, -1, F, G, None) == INVALID
    assert sc(X, Y, A, B, 10, 12, 3, 0.1, 5, A, G, None) == INVALID    # f aliases a
    assert sc(X, Y, A, B, 10, 12, lds.OT_MAX_DIM + 1, 0.1, 5, F, G, None) == UNSUPPORTED
    assert sc(X, Y, A, B, 10, 12, 3, 3e38, 5, F, G, None) == UNSUPPORTED  # 2 eps overflows
    assert sc(X, Y, A, B, 10, 12, 3, 0.1, 0, F, G, None) == 0           # host no-op
    assert pc(X, Y, A, B, F, G, 10, 12, 3, 0.1, None, None, None) == INVALID
    assert pc(X, Y, None, B, F, G, 10, 12, 3, 0.1, None, MG, None) == INVALID
    assert pc(X, Y, A, B, F, G, 10, 12, 200, 0.1, C, None, None) == UNSUPPORTED


def test_solve_zero_iters_is_a_host_noop(lib):
    # valid arguments with iters == 0 return before any device call
    assert solve(lib, iters=0) == 0
