"""Graph capture: a call enqueues its work (and its temporary memory, as
stream-ordered allocations) on the caller's stream, so it can be captured
into a HIP graph. Each case captures a call once, then replays the graph
several times with other eager work and synchronisations in between; every
replay must reproduce the eager call bit for bit (the kernels are
deterministic: fixed reduction orders, no atomics).

The eager result itself is checked against the fp64 oracle by the other GPU
tests; here only capture and replay are under test.
"""
import numpy as np
import pytest
import torch

import log_domain_sinkhorn_amd as lds
from workloads import make_logits, random_clouds

from gpu_helpers import DEV, dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replays_match(run, outputs, reset):
    """Run eagerly, capture one call, replay REPLAYS times; compare each
    replay's outputs with the eager ones."""
    reset()
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    reset()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 16, device=DEV)
    for rep in range(REPLAYS):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        # unrelated eager work between replays
        scratch.mul_(1.5).add_(1.0)
        float(scratch.sum().item())
        for e, o in zip(eager, outputs):
            assert torch.equal(o, e), f"replay {rep} differs from the eager call"
    print(f"{REPLAYS} replays identical to the eager call", flush=True)


@pytest.mark.parametrize("d", [3, 64, 256, 1024])
def test_solve_and_plan_stats_capture(d):
    c = random_clouds(1500, 1100, d, seed=d)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    eps = 0.5 * d ** 0.5
    f = torch.zeros(1500, device=DEV)
    g = torch.zeros(1100, device=DEV)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)

    def reset():
        for t in (f, g, cost, marg):
            t.zero_()

    def run():
        lds.ot_sinkhorn_solve(x, y, a, b, eps, 7, f, g)
        lds.ot_plan_stats(x, y, a, b, f, g, eps, cost, marg)

    _replays_match(run, [f, g, cost, marg], reset)


@pytest.mark.parametrize("d", [3, 64, 256, 1024])
def test_transport_capture(d):
    c = random_clouds(700, 900, d, seed=10 + d, spread=1.0 / np.sqrt(d))
    x, y = dev(c["x"]), dev(c["y"])
    eps = 0.2
    f = torch.linspace(-1.0, 0.0, 700, device=DEV)
    g = torch.linspace(0.0, 0.5, 900, device=DEV)
    out = torch.zeros(700, d, device=DEV)

    def reset():
        out.zero_()

    def run():
        lds.ot_transport_apply(x, y, f, g, eps, y, out)

    _replays_match(run, [out], reset)


def test_birkhoff_capture():
    L = dev(make_logits(4099, (1.0, 10.0), seed=3))
    out = torch.zeros_like(L)
    it = torch.zeros(L.shape[0], dtype=torch.int32, device=DEV)

    def reset():
        out.zero_()
        it.zero_()

    def run():
        lds.ot_birkhoff_project_batched(L, 1.0, 200, 1e-6, out, it)

    _replays_match(run, [out, it], reset)


def test_calls_refused_under_capture():
    # The calls of the sequence that faulted under capture and whose cause is
    # not known return OT_ERROR_NOT_SUPPORTED on a capturing stream and
    # enqueue nothing; outside a capture they run.
    c = random_clouds(300, 200, 40, seed=6, spread=0.3)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(300, device=DEV)
    g = torch.zeros(200, device=DEV)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    out = torch.zeros(300, 40, device=DEV)
    calls = {
        "ot_sinkhorn_solve_cosine": lambda: lds.ot_sinkhorn_solve_cosine(x, y, a, b, 0.1, 3, f, g),
        "ot_plan_stats_cosine": lambda: lds.ot_plan_stats_cosine(x, y, a, b, f, g, 0.1, cost,
                                                                 marg),
        "ot_barycentric_map": lambda: lds.ot_barycentric_map(x, y, a, f, g, 0.2, out),
        "ot_cost_gradient_x": lambda: lds.ot_cost_gradient_x(x, y, f, g, 0.2, out),
    }
    marker = torch.zeros(1, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    status = {}
    with torch.cuda.graph(graph, stream=side):
        marker.add_(1.0)  # keeps the captured graph non-empty
        for name, call in calls.items():
            try:
                call()
                status[name] = 0
            except lds.OTError as e:
                status[name] = e.status
    torch.cuda.synchronize()
    print("status under capture:", status, flush=True)
    assert all(v == 2 for v in status.values()), status
    for name, call in calls.items():
        call()
    torch.cuda.synchronize()
    assert torch.isfinite(f).all() and torch.isfinite(out).all()


@pytest.mark.skip(reason="replaying this graph faulted the GPU (illegal address reported in "
                         "prep_h3_kernel) after the same sequence ran correctly eagerly; reading "
                         "the kernels' index ranges and the scratch layout found no out-of-range "
                         "access, so the cause is unknown and the case stays off the GPU; the "
                         "cosine calls, the barycentric map and the x-gradient refuse capture "
                         "(test_calls_refused_under_capture)")
def test_other_entry_points_capture():
    # eps schedule, cosine cost, barycentric map, x-gradient, 4x4 Newton and
    # its backward, all in one captured sequence.
    c = random_clouds(800, 600, 40, seed=5, spread=0.3)
    x, y, a, b = dev(c["x"]), dev(c["y"]), dev(c["a"]), dev(c["b"])
    f = torch.zeros(800, device=DEV)
    g = torch.zeros(600, device=DEV)
    fc = torch.zeros(800, device=DEV)
    gc = torch.zeros(600, device=DEV)
    cost = torch.zeros(1, dtype=torch.float64, device=DEV)
    marg = torch.zeros(2, dtype=torch.float64, device=DEV)
    bary = torch.zeros(800, 40, device=DEV)
    grad = torch.zeros(800, 40, device=DEV)
    L = dev(make_logits(1000, (1.0, 10.0), seed=4))
    P = torch.zeros_like(L)
    it = torch.zeros(1000, dtype=torch.int32, device=DEV)
    dP = dev(np.random.default_rng(2).normal(size=(1000, 4, 4)).astype(np.float32))
    dL = torch.zeros_like(L)
    outs = [f, g, fc, gc, cost, marg, bary, grad, P, it, dL]

    def reset():
        for t in outs:
            t.zero_()

    def run():
        lds.ot_sinkhorn_solve_eps_scaling(x, y, a, b, 2.0, 0.2, 3, 4, f, g)
        lds.ot_barycentric_map(x, y, a, f, g, 0.2, bary)
        lds.ot_cost_gradient_x(x, y, f, g, 0.2, grad)
        lds.ot_sinkhorn_solve_cosine(x, y, a, b, 0.1, 5, fc, gc)
        lds.ot_plan_stats_cosine(x, y, a, b, fc, gc, 0.1, cost, marg)
        lds.ot_birkhoff_project_newton_batched(L, 1.0, 50, 1e-6, P, it)
        lds.ot_birkhoff_projection_backward_batched(P, dP, 1.0, dL)

    _replays_match(run, outs, reset)
