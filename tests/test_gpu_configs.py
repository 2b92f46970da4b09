"""GPU parity of whole configurations, through the code the benchmark runs.

Each test drives the benchmark's own step objects (bench.py: PowersgdPart's
recorded deferred plans, TopkEncoder's deferred top-k, the uncompressed
vectors) and compares every checked step with the float64 oracle from the
state the GPU held before that step: the deferred memories are written out
(gc_powersgd_materialize / gc_topk_materialize on copies) and fed to the
oracle step together with Q and the step's gradient.  PowerSGD results (P^,
Q, out, memory) must agree within a relative Frobenius error of 1e-4 per
matrix (an absolute 1e-4 * ||M|| where the oracle's value is ~0); top-k and
the uncompressed vectors must agree bit for bit.

  * ResNet-18 (CIFAR-100): 21 matrices at rank 1 and at rank 2 plus the 41
    BN/bias vectors sent uncompressed, the 20 steps of the protocol with a
    fresh draw each step.
  * VGG-19 with Accordion: the norm trajectory over the 300 steps of the
    protocol, one gradient buffer refilled per step (as a training loop
    would), the per-layer norms taken on the GPU every 10 steps, the levels
    chosen by gc_accordion_select (l_low = rank 4, l_high = rank 2), the plan
    recorded again at each switch and Q's new columns refilled on rank growth.
    Every step of 100..120 and 200..220 (both jumps) and 290..299 is compared
    with the oracle;
    the decisions at every check equal the closed-form schedule, and at the
    window checks the oracle's own norms give the same decisions.
  * BERT-large: the benchmark's C5 step (all 144 matrices in one recorded
    plan, the embedding's top-k 1%), the 5 steps of the protocol; encoder layers 0 and 23 (12
    matrices) and the embedding are compared every step.
  * Determinism: two instances of each configuration's step (C1-C5), built
    from the same seeds, hold the same bits in every output and state buffer
    after every step (C4 across a rank switch).
  * The ResNet-50-sized flat gradient over the 50 steps of its protocol
    (fresh gradient each step, deferred top-k 1%): every step against the
    properties that fix an exact top-k EF step, on the device at full size;
    four steps against the oracle from the GPU's state.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, f32_bits, lib, rel_err, require_gpu, to_dev
from topk_props import check_topk_step_properties

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
import bench  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 1e-4
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Snapshot:
    """The state a PowerSGD step starts from, for the chosen matrices: the
    memory the method carries (the deferred memory written out into copies)
    and the first `rank` columns of Q."""

    def __init__(self, part, layers, ws):
        gc = lib()
        copies = [part.mem[i].clone() for i in layers]
        mats = [gc.Mat(grad=None, mem=c, q=part.q[i], rank=max(1, part.ranks[i]), p=part.p[i])
                for c, i in zip(copies, layers)]
        gc.gc_powersgd_materialize(mats, [part.prev[i] for i in layers], ws)
        torch.cuda.synchronize()
        self.mem = {i: c.cpu().numpy() for c, i in zip(copies, layers)}
        self.q = {i: part.q[i][: part.ranks[i]].cpu().numpy().T.copy() for i in layers}


def materialize_ws(part, layers):
    gc = lib()
    mats = [gc.Mat(grad=None, mem=part.mem[i], q=part.q[i], rank=1, p=part.p[i]) for i in layers]
    return torch.empty(gc.gc_powersgd_workspace_bytes(mats), dtype=torch.uint8, device=DEV)


def check_psgd_step(part, layers, before, after, grads_h, label):
    """The GPU step (before -> after, and its out / P^ / Q) against the oracle step from `before`."""
    worst = 0.0
    for i in layers:
        r = part.ranks[i]
        ref = oracle.powersgd_ef_step(grads_h[i], before.mem[i], before.q[i], 1.0, r)
        Mn = np.linalg.norm(ref["M"])
        checks = [("P", part.p[i][:r].cpu().numpy().T, ref["P"]), ("Q", after.q[i], ref["Q"]),
                  ("out", part.out[i].cpu().numpy(), ref["out"]), ("mem", after.mem[i], ref["mem"])]
        for name, got, want in checks:
            if name in ("mem", "out") and np.linalg.norm(want) < 1e-6 * Mn:
                err = float(np.linalg.norm(got.astype(np.float64) - want) / Mn)
            else:
                err = rel_err(got, want)
            worst = max(worst, err)
            assert err <= TOL, f"{label}: matrix {i} {part.shapes[i]} r={r} {name}: rel err {err:.3e}"
    return worst


@pytest.mark.parametrize("rank", [1, 2])
def test_c2_resnet18_with_vectors(rank):
    """The ResNet-18 step of the benchmark: PowerSGD (recorded deferred plan) on
    the 21 matrices and the BN/bias vectors uncompressed, for the 20 steps of
    the configuration's protocol with a fresh gradient draw every step (copied
    into the benchmark's two alternating buffers), at rank 1 and rank 2."""
    print(f"case: C2 ResNet-18 config, rank {rank}, 20 steps", flush=True)
    gc = lib()
    W = bench.C2(torch, gc, DEV, rank=rank)
    part = W.ps
    layers = list(range(len(part.shapes)))
    ws = materialize_ws(part, layers)
    for t in range(20):
        grads_h = gen.c2_grads(t)
        vecs_h = gen.c2_vectors(t)
        for view, g in zip(W.sets[t % 2], grads_h):
            view.copy_(torch.from_numpy(g.ravel()))
        for view, v in zip(W.vsets[t % 2], vecs_h):
            view.copy_(torch.from_numpy(v))
        before = Snapshot(part, layers, ws)
        W.step(t)
        torch.cuda.synchronize()
        after = Snapshot(part, layers, ws)
        worst = check_psgd_step(part, layers, before, after, grads_h, f"C2 r{rank} step {t}")
        for v, h in enumerate(vecs_h):
            assert np.array_equal(f32_bits(W.vout[v]), f32_bits(oracle.passthrough_step(h, 1.0))), \
                f"C2 step {t} vector {v}"
        if t % 5 == 4:
            print(f"C2 r{rank} step {t}: worst PowerSGD relative error {worst:.2e}", flush=True)


WINDOWS = list(range(100, 121)) + list(range(200, 221)) + list(range(290, 300))


def test_c4_vgg19_accordion_end_to_end():
    print("case: C4 VGG-19 Accordion end to end, steps 0..299", flush=True)
    gc = lib()
    gold = json.load(open(os.path.join(GOLD, "c4_accordion_schedule.json")))
    thr = gold["threshold"]
    shapes = gen.VGG19_MATS
    sizes = [n * m for n, m in shapes]
    L = len(shapes)
    _, mem_views = bench._flat(torch, sizes, torch.float32, DEV, 64)
    _, gviews = bench._flat(torch, sizes, torch.float32, DEV, 64)
    part = bench.PowersgdPart(torch, gc, shapes, [gen.C4_RANK_LOW_COMPRESSION] * L, [gviews], mem_views, DEV,
                              gen.CFG_C4, deferred=True)
    layers = list(range(L))
    ws = materialize_ws(part, layers)
    norms = torch.empty(L, device=DEV)
    nws = torch.empty(gc.gc_grad_norm_workspace_bytes(gviews), dtype=torch.uint8, device=DEV)
    prev = np.zeros(L, np.float32)
    lows, worst, plans = [], 0.0, 0
    last_key = None
    for t in range(WINDOWS[-1] + 1):
        host = gen.c4_grads(t)
        for v, h in zip(gviews, host):
            v.copy_(torch.from_numpy(h.ravel()))
        if t % gold["check_every"] == 0:
            gc.gc_grad_norm(gviews, norms, nws)
            got = norms.cpu().numpy()
            prev_before = prev.copy()
            lv, prev = gc.gc_accordion_select(got, prev, thr, t > 0)
            assert len(set(lv.tolist())) == 1, f"check {t}: layers disagree {lv}"
            if lv[0] == gc.GC_LEVEL_LOW:
                lows.append(t)
            if t in WINDOWS:
                want = np.array([oracle.grad_norm(h) for h in host])
                assert np.all(np.abs(got - want) <= TOL * want), f"check {t}: norms"
                olv, _ = oracle.accordion_select(want.astype(np.float32), prev_before, True, thr)
                assert np.array_equal(olv, lv), f"check {t}: oracle decisions differ"
            new = [gen.C4_RANK_LOW_COMPRESSION if x == gc.GC_LEVEL_LOW else gen.C4_RANK_HIGH_COMPRESSION for x in lv]
            for l in layers:
                bench.refill_q(part, l, t, part.ranks[l], new[l], gen.CFG_C4)
            part.set_ranks(new)
        check = t in WINDOWS
        if check:
            before = Snapshot(part, layers, ws)
        part.step(0)
        if part.plan_keys[0] != last_key:
            plans += 1
            last_key = part.plan_keys[0]
        if check:
            torch.cuda.synchronize()
            after = Snapshot(part, layers, ws)
            worst = max(worst, check_psgd_step(part, layers, before, after, host, f"C4 step {t}"))
    assert lows == [c for c in gold["low_checks"] if c <= WINDOWS[-1]]
    # plans: the first step (prev 0), the steady rank-4 plan, then per switch the
    # switching step's plan and the steady plan after it
    assert plans >= 6
    print(f"C4 checks at l_low: {lows}; plans recorded: {plans}; worst relative error {worst:.2e}", flush=True)


def test_c5_bert_shipped_steps():
    print("case: C5 BERT-large shipped step (bench.C5), 5 steps", flush=True)
    gc = lib()
    W = bench.C5(torch, gc, DEV)
    part = W.ps
    layers = list(range(6)) + list(range(138, 144))
    ws = materialize_ws(part, layers)
    d, k = W.emb_mem.numel(), W.k
    for t in range(5):
        s = t % 2
        grads_h = {i: gen.c5_matrix_bf16(s, i).reshape(part.shapes[i]) for i in layers}
        before = Snapshot(part, layers, ws)
        emb_before = W.emb_mem.clone()
        if W.enc.has_prev:
            gc.gc_topk_materialize(emb_before, W.enc.sel)
        W.step(t)
        torch.cuda.synchronize()
        after = Snapshot(part, layers, ws)
        worst = check_psgd_step(part, layers, before, after, grads_h, f"C5 step {t}")
        emb_after = W.emb_mem.clone()
        gc.gc_topk_materialize(emb_after, W.enc.sel)
        ref = oracle.topk_ef_step(emb_before.cpu().numpy(), gen.c5_embedding_bf16(s), 1.0, k)
        torch.cuda.synchronize()
        assert np.array_equal(W.idx.cpu().numpy(), ref["idx"]), f"C5 step {t}: embedding top-k indices"
        assert np.array_equal(f32_bits(W.val), f32_bits(ref["val"])), f"C5 step {t}: embedding top-k values"
        assert np.array_equal(f32_bits(emb_after), f32_bits(ref["mem"])), f"C5 step {t}: embedding memory"
        out = W.emb_out.cpu().numpy()
        assert np.array_equal(out, oracle.topk_decode(ref["idx"], ref["val"], d)), f"C5 step {t}: decode"
        print(f"C5 step {t}: worst PowerSGD relative error {worst:.2e}", flush=True)
    del W
    torch.cuda.empty_cache()


def _c2_state(W):
    ps = W.ps
    return ([t.clone() for t in ps.out] + [t.clone() for t in ps.mem] + [t.clone() for t in ps.q] +
            [t.clone() for t in ps.p] + [W.vout_buf.clone()])


def _c3_state(W):
    return [W.idx.clone(), W.val.clone(), W.out.clone(), W.mem.clone(), W.enc.sel.clone()]


def _c4_state(W):
    ps = W.ps
    return ([t.clone() for t in ps.out] + [t.clone() for t in ps.mem] + [t.clone() for t in ps.q] +
            [t.clone() for t in ps.p] + [W.norms.clone()])


def _c5_state(W):
    ps = W.ps
    return ([ps.out_buf.clone()] + [t.clone() for t in ps.mem] + [t.clone() for t in ps.q] +
            [t.clone() for t in ps.p] + [W.idx.clone(), W.val.clone(), W.emb_out.clone(), W.emb_mem.clone(),
                                         W.enc.sel.clone()])


def _make_c4(torch_, gc, dev):
    W = bench.C4(torch_, gc, dev)
    # trajectory steps 100..111: the checks at 100 (l_high) and 110 (l_low, ranks 2 -> 4)
    W.prepare(0, 12)
    return W


CONFIGS = {
    "c1": (bench.C1, _c3_state, 10),
    "c2": (bench.C2, _c2_state, 4),
    "c3": (bench.C3, _c3_state, 4),
    "c4": (_make_c4, _c4_state, 12),
    "c5": (bench.C5, _c5_state, 3),
}


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_config_determinism(name):
    """Two instances of a configuration's step, from the same seeds, hold the same
    bits after every step: outputs, memories, Q, P^, the norms and the
    selection record (compaction order and every reduction order included)."""
    make, state, steps = CONFIGS[name]
    print(f"case: determinism of the {name} step, two instances, {steps} steps", flush=True)
    gc = lib()
    A, B = make(torch, gc, DEV), make(torch, gc, DEV)
    for t in range(steps):
        A.step(t)
        B.step(t)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(state(A), state(B))):
            assert torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32)), \
                f"{name} step {t}: buffer {i} differs between the two instances"
    del A, B
    torch.cuda.empty_cache()


def test_c3_fifty_steps_deferred():
    """The ResNet-50-sized flat gradient for the 50 steps of its protocol, a
    fresh heavy-tailed gradient each step, k = 1%, through the benchmark's
    deferred top-k encoder and decode: every step against the properties that
    fix an exact top-k EF step (checked on the device, at full size), and
    steps 0, 1, 25 and 49 against the float64 oracle from the memory the GPU
    held before them."""
    print("case: C3 50 steps, deferred top-k, d=25.6M k=1%", flush=True)
    gc = lib()
    d, k = gen.C3_D, gen.C3_KS[1]
    enc = bench.TopkEncoder(torch, gc, DEV)
    assert enc.deferred
    mem = torch.zeros(d, device=DEV)
    idx = torch.empty(k, dtype=torch.int32, device=DEV)
    val = torch.empty(k, device=DEV)
    out = torch.empty(d, device=DEV)
    ws = torch.empty(gc.gc_topk_workspace_bytes(d, k), dtype=torch.uint8, device=DEV)
    oracle_steps = {0, 1, 25, 49}
    for t in range(50):
        g_h = gen.c3_grad(t)
        g = to_dev(g_h)
        before = mem.clone()
        if enc.has_prev:
            gc.gc_topk_materialize(before, enc.sel)
        acc = before + g                       # fl32(m + fl32(1 * g)): eta = 1
        enc.encode(g, mem, 1.0, k, idx, val, ws)
        gc.gc_topk_decode(idx, val, out)
        after = mem.clone()
        gc.gc_topk_materialize(after, enc.sel)
        torch.cuda.synchronize()
        check_topk_step_properties(acc, idx, val, out, after, k, f"C3 step {t}")
        if t in oracle_steps:
            ref = oracle.topk_ef_step(before.cpu().numpy(), g_h, 1.0, k)
            assert np.array_equal(idx.cpu().numpy(), ref["idx"]), f"C3 step {t}: indices vs oracle"
            assert np.array_equal(f32_bits(val), f32_bits(ref["val"])), f"C3 step {t}: values vs oracle"
            assert np.array_equal(f32_bits(after), f32_bits(ref["mem"])), f"C3 step {t}: memory vs oracle"
        if t % 10 == 9:
            print(f"C3 step {t}: ok", flush=True)
    del mem, out, ws
    torch.cuda.empty_cache()
