"""GPU parity: recorded PowerSGD steps (gc_powersgd_plan once, then
gc_powersgd_run per step: kernel launches only) against the direct calls
(gc_powersgd_ef_step; the deferred form's memory written out by
gc_powersgd_materialize), bit for bit; one plan
replayed inside a captured HIP graph too.  The direct calls are themselves
checked against the float64 oracle in test_gpu_powersgd*.py."""
import numpy as np
import pytest
import torch

import gen
from gpu_util import DEV, lib, require_gpu, to_dev
from test_gpu_powersgd_deferred import Set, bits_equal, compare_bitwise

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def ws_for(S, grads):
    return torch.empty(lib().gc_powersgd_workspace_bytes(S.mats(grads)), dtype=torch.uint8, device=DEV)


def compare_all(A, B, label):
    torch.cuda.synchronize()
    for i in range(len(A.shapes)):
        r = A.ranks[i]
        for name, x, y in [("out", A.out[i], B.out[i]), ("P", A.p[i][:r], B.p[i][:r]), ("Q", A.q[i][:r], B.q[i][:r]),
                           ("mem", A.mem[i], B.mem[i])]:
            assert bits_equal(x, y), f"{label}: matrix {i} {A.shapes[i]} {name} differs"


def grad_buffers(shapes, dtype):
    return [torch.zeros(n, m, dtype=dtype, device=DEV) for n, m in shapes]


def fill(bufs, grads_h):
    for b, g in zip(bufs, grads_h):
        b.copy_(to_dev(g).view(b.shape))


@pytest.mark.parametrize("case", ["resnet18", "random", "many"])
def test_explicit_plan_matches_direct(case):
    gc = lib()
    if case == "resnet18":
        shapes, ranks, gfn = gen.RESNET18_MATS, [2] * len(gen.RESNET18_MATS), gen.c2_grads
    elif case == "random":
        rs = np.random.default_rng(77)
        shapes = [(int(rs.integers(1, 400)), int(rs.choice([27, 64, 576, 1030, 2048, 4096, 4608]))) for _ in range(10)]
        ranks = [int(rs.integers(1, min(4, n, m) + 1)) for n, m in shapes]
        gfn = lambda t: [gen.gaussian_mat(n, m, 1400 + 11 * t + i, 1e-2) for i, (n, m) in enumerate(shapes)]
    else:
        shapes = [(3 + i % 5, 8 if i % 3 else 5) for i in range(4100)]
        ranks = [1 + i % 3 for i in range(4100)]
        gfn = lambda t: [gen.gaussian_mat(n, m, 1500 + 7 * t + i, 1e-2) for i, (n, m) in enumerate(shapes)]
    print(f"case: explicit plan vs direct, {case}", flush=True)
    A, B = Set(shapes, ranks, 3), Set(shapes, ranks, 3)
    ga, gb = grad_buffers(shapes, torch.float32), grad_buffers(shapes, torch.float32)
    wsb = ws_for(B, gb)
    plan = gc.gc_powersgd_plan(B.mats(gb), None, wsb)
    for t in range(3):
        g = gfn(t)
        fill(ga, g)
        fill(gb, g)
        A.explicit(ga, 0.9)
        gc.gc_powersgd_run(plan, 0.9, wsb)
        compare_all(A, B, f"{case} explicit step {t}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deferred_plan_matches_direct(dtype):
    """The first deferred step direct (prev_rank 0), then one plan with
    prev_rank = rank for every later step; eta changes per run."""
    gc = lib()
    shapes = [(300, 1024), (64, 27), (33, 4608), (128, 2048), (40, 4096)]
    ranks = [4, 2, 3, 1, 4]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"case: deferred plan vs direct {dtype}", flush=True)

    def grads(t):
        out = [gen.gaussian_mat(n, m, 1600 + 13 * t + i, 1e-2) for i, (n, m) in enumerate(shapes)]
        return [gen.f32_to_bf16_bits(g).reshape(g.shape) for g in out] if dtype == "bf16" else out

    A, B = Set(shapes, ranks, 4), Set(shapes, ranks, 4)
    ga, gb = grad_buffers(shapes, tdt), grad_buffers(shapes, tdt)
    wsb = ws_for(B, gb)
    fill(ga, grads(0))
    fill(gb, grads(0))
    A.explicit(ga, 1.0)
    B.deferred(gb, 1.0)
    plan = gc.gc_powersgd_plan(B.mats(gb), ranks, wsb)
    for t, eta in zip(range(1, 5), [1.0, 0.5, 0.25, 1.0]):
        fill(ga, grads(t))
        fill(gb, grads(t))
        A.explicit(ga, eta)
        gc.gc_powersgd_run(plan, eta, wsb)
        B.prev = list(ranks)
        compare_bitwise(A, B, f"deferred plan step {t}")


@pytest.mark.parametrize("case", ["deferred-bf16", "explicit-f32", "many-deferred"])
def test_phases_match_run(case):
    """gc_powersgd_run_phases: the encode, unrelated work on the same stream
    and on a second stream, then the decode, against gc_powersgd_run of an
    identical set, bit for bit.  "many": 4100 matrices, so the plan holds
    several batches and all their encodes run before all their decodes."""
    gc = lib()
    deferred = case != "explicit-f32"
    if case.startswith("many"):
        shapes = [(3 + i % 5, 8 if i % 3 else 5) for i in range(4100)]
        ranks = [1 + i % 3 for i in range(4100)]
        tdt = torch.float32
    else:
        shapes = [(300, 1024), (64, 27), (33, 4608), (128, 2048), (40, 4096), (1024, 1024)]
        ranks = [4, 2, 3, 1, 4, 4]
        tdt = torch.bfloat16 if case.endswith("bf16") else torch.float32
    print(f"case: phases vs run, {case}", flush=True)

    def grads(t):
        out = [gen.gaussian_mat(n, m, 1700 + 17 * t + i, 1e-2) for i, (n, m) in enumerate(shapes)]
        return [gen.f32_to_bf16_bits(g).reshape(g.shape) for g in out] if tdt == torch.bfloat16 else out

    A, B = Set(shapes, ranks, 5), Set(shapes, ranks, 5)
    ga, gb = grad_buffers(shapes, tdt), grad_buffers(shapes, tdt)
    wsa, wsb = ws_for(A, ga), ws_for(B, gb)
    fill(ga, grads(0))
    fill(gb, grads(0))
    if deferred:
        A.deferred(ga, 1.0)
        B.deferred(gb, 1.0)
    prev = list(ranks) if deferred else None
    pa = gc.gc_powersgd_plan(A.mats(ga), prev, wsa)
    pb = gc.gc_powersgd_plan(B.mats(gb), prev, wsb)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    x = torch.randn(1 << 22, device=DEV)
    ev = torch.cuda.Event()
    for t, eta in zip(range(1, 4), [1.0, 0.5, 1.0]):
        fill(ga, grads(t))
        fill(gb, grads(t))
        gc.gc_powersgd_run(pa, eta, wsa)
        gc.gc_powersgd_run_phases(pb, eta, wsb, gc.PHASE_ENCODE)
        y = x * 2.0                       # unrelated work between the phases
        ev.record(main)
        side.wait_event(ev)
        with torch.cuda.stream(side):     # and beside the decode
            z = x + 1.0
        gc.gc_powersgd_run_phases(pb, eta, wsb, gc.PHASE_DECODE)
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(y, x * 2.0) and torch.equal(z, x + 1.0)
        # identical sets, identical calls: every buffer (deferred: mem holds M) equal
        compare_all(A, B, f"{case} step {t}")


@pytest.mark.parametrize("split", [False, True], ids=["run", "phases"])
def test_plan_replayed_in_graph(split):
    """A deferred plan captured in a HIP graph on the ResNet-18 set: each
    replay is one step; new gradients are copied in eagerly between replays,
    and every replay is compared with the direct deferred call.  "phases":
    the capture holds the encode, a torch kernel, then the decode."""
    gc = lib()
    gc.gc_timing_enable(None)   # no timing events in the capture
    shapes, ranks = gen.RESNET18_MATS, [2] * len(gen.RESNET18_MATS)
    print(f"case: deferred plan in a captured graph, ResNet-18, split={split}", flush=True)
    A, B = Set(shapes, ranks, gen.CFG_C2), Set(shapes, ranks, gen.CFG_C2)
    ga, gb = grad_buffers(shapes, torch.float32), grad_buffers(shapes, torch.float32)
    wsb = ws_for(B, gb)
    fill(ga, gen.c2_grads(0))
    fill(gb, gen.c2_grads(0))
    A.explicit(ga, 1.0)
    B.deferred(gb, 1.0)
    plan = gc.gc_powersgd_plan(B.mats(gb), ranks, wsb)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    # the capture records the launches only; what it computes is checked on replay
    snapshot = [[t.clone() for t in lst] for lst in (B.mem, B.q, B.p, B.out)]
    x = torch.arange(4096, dtype=torch.float32, device=DEV)
    y = torch.zeros_like(x)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            if split:
                gc.gc_powersgd_run_phases(plan, 1.0, wsb, gc.PHASE_ENCODE)
                y.copy_(x * 3.0)
                gc.gc_powersgd_run_phases(plan, 1.0, wsb, gc.PHASE_DECODE)
            else:
                gc.gc_powersgd_run(plan, 1.0, wsb)
    torch.cuda.synchronize()
    for lst, snap in zip((B.mem, B.q, B.p, B.out), snapshot):
        for t, s0 in zip(lst, snap):
            t.copy_(s0)
    for t in range(1, 4):
        g = gen.c2_grads(t)
        fill(ga, g)
        fill(gb, g)
        torch.cuda.synchronize()
        A.explicit(ga, 1.0)
        graph.replay()
        torch.cuda.synchronize()
        B.prev = list(ranks)
        compare_bitwise(A, B, f"graph replay {t}")
        if split:
            assert torch.equal(y, x * 3.0)


def test_run_refuses_another_workspace():
    gc = lib()
    shapes, ranks = [(64, 576)], [2]
    S = Set(shapes, ranks)
    g = grad_buffers(shapes, torch.float32)
    ws1, ws2 = ws_for(S, g), ws_for(S, g)
    plan = gc.gc_powersgd_plan(S.mats(g), None, ws1)
    torch.cuda.synchronize()
    with pytest.raises(gc.GCError):
        gc.gc_powersgd_run(plan, 1.0, ws2)
    with pytest.raises(gc.GCError):
        gc.gc_powersgd_run(plan[:16].copy(), 1.0, ws1)
