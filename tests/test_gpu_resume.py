"""GPU: a run checkpointed and resumed equals the run straight through, bit for bit.

With the memories in deferred form, what a checkpoint must hold is the memory
the method carries (written out with gc_powersgd_materialize /
gc_topk_materialize), Q, the ranks in use and the Accordion state (the
previous check's norms).  After a restore into fresh buffers the first step
takes the restored memory as explicit (previous rank 0, no selection record);
every later step is deferred again.

  * PowerSGD with Accordion on the VGG-19 set, steps 100..109 of the norm
    trajectory with a check every 2 steps: rank 4 at the first check, 2 after
    it, 4 again after the jump at 105 (Q's new columns refilled), then 2.  Run
    A goes straight through; run B stops after step 104, checkpoints to host
    arrays, frees every device buffer, restores and runs 105..109.
  * Top-k 1% with its memory in deferred form (d = 2^22 + 77), steps 0..9, the
    checkpoint after step 4.

Every output of the resumed steps (PowerSGD out, P^ and Q; top-k indices,
values and decode) and the final memory equal run A's bit for bit.
"""
import numpy as np
import pytest
import torch

import gen
from gpu_util import DEV, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def bits(t):
    return t.contiguous().view(torch.int32)


# ----------------------------------------------------------------------------- PowerSGD + Accordion

SHAPES = gen.VGG19_MATS
T0, T_SPLIT, T_END, EVERY = 100, 105, 110, 2
LOW, HIGH = gen.C4_RANK_LOW_COMPRESSION, gen.C4_RANK_HIGH_COMPRESSION


class PsRun:
    """Device state of one run: memories, Q, P, outputs, ranks and the Accordion state."""

    def __init__(self, mem=None, q=None, ranks=None, prev_norms=None, has_prev=False):
        L = len(SHAPES)
        self.mem = [torch.zeros(n, m, device=DEV) if mem is None else to_dev(mem[i]) for i, (n, m) in enumerate(SHAPES)]
        self.q = [to_dev(gen.q_init(gen.CFG_C4, l, m)) if q is None else to_dev(q[l]) for l, (n, m) in enumerate(SHAPES)]
        self.p = [torch.zeros(4, n, device=DEV) for n, m in SHAPES]
        self.out = [torch.zeros(n, m, device=DEV) for n, m in SHAPES]
        self.ranks = [LOW] * L if ranks is None else list(ranks)
        self.prev = [0] * L                  # memory held explicitly
        self.prev_norms = np.zeros(L, np.float32) if prev_norms is None else prev_norms.copy()
        self.has_prev = has_prev
        self.ws = None
        self.nws = None

    def mats(self, grads, mem=None):
        gc = lib()
        mem = self.mem if mem is None else mem
        return [gc.Mat(grad=g, mem=mem[i], q=self.q[i], rank=self.ranks[i], p=self.p[i], out=self.out[i])
                for i, g in enumerate(grads)]

    def _ws(self, mats):
        need = lib().gc_powersgd_workspace_bytes(mats)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        return self.ws

    def step(self, t):
        gc = lib()
        grads = [to_dev(g.ravel()).view(n, m) for g, (n, m) in zip(gen.c4_grads(t), SHAPES)]
        if (t - T0) % EVERY == 0:
            flat = [g.view(-1) for g in grads]
            if self.nws is None:
                self.nws = torch.empty(gc.gc_grad_norm_workspace_bytes(flat), dtype=torch.uint8, device=DEV)
            norms = torch.empty(len(flat), device=DEV)
            gc.gc_grad_norm(flat, norms, self.nws)
            lv, self.prev_norms = gc.gc_accordion_select(norms.cpu().numpy(), self.prev_norms,
                                                          gen.C4_THRESHOLD, self.has_prev)
            self.has_prev = True
            new = [LOW if x == gc.GC_LEVEL_LOW else HIGH for x in lv]
            for l, (n, m) in enumerate(SHAPES):
                old = self.ranks[l]
                if new[l] > old:
                    self.q[l][old:new[l]].copy_(torch.from_numpy(gen.q_refill(gen.CFG_C4, l, t, m, 4)[old:new[l]]))
            self.ranks = new
        mats = self.mats(grads)
        gc.gc_powersgd_ef_step_deferred(mats, self.prev, 1.0, self._ws(mats))
        self.prev = list(self.ranks)

    def memory(self):
        copies = [t.clone() for t in self.mem]
        mats = self.mats([None] * len(copies), mem=copies)
        lib().gc_powersgd_materialize(mats, self.prev, self._ws(mats))
        return copies

    def checkpoint(self):
        mem = [c.cpu().numpy() for c in self.memory()]
        q = [t.cpu().numpy() for t in self.q]
        return dict(mem=mem, q=q, ranks=list(self.ranks), prev_norms=self.prev_norms.copy(), has_prev=self.has_prev)

    def outputs(self):
        return [(o.clone(), p[:r].clone(), q[:r].clone()) for o, p, q, r in zip(self.out, self.p, self.q, self.ranks)]


def test_powersgd_accordion_resume():
    print("case: PowerSGD + Accordion on VGG-19, steps 100..109, checkpoint after 104", flush=True)
    A = PsRun()
    ref, ranks_seen = {}, []
    for t in range(T0, T_END):
        A.step(t)
        ranks_seen.append(A.ranks[0])
        if t >= T_SPLIT:
            ref[t] = A.outputs()
    assert ranks_seen == [LOW, LOW, HIGH, HIGH, HIGH, HIGH, LOW, LOW, HIGH, HIGH], ranks_seen
    memA = A.memory()
    torch.cuda.synchronize()

    B = PsRun()
    for t in range(T0, T_SPLIT):
        B.step(t)
    ck = B.checkpoint()
    del B
    torch.cuda.empty_cache()
    C = PsRun(mem=ck["mem"], q=ck["q"], ranks=ck["ranks"], prev_norms=ck["prev_norms"], has_prev=ck["has_prev"])
    for t in range(T_SPLIT, T_END):
        C.step(t)
        got = C.outputs()
        torch.cuda.synchronize()
        for l, ((oa, pa, qa), (oc, pc, qc)) in enumerate(zip(ref[t], got)):
            assert torch.equal(bits(oa), bits(oc)), f"step {t} layer {l}: out differs after the resume"
            assert torch.equal(bits(pa), bits(pc)), f"step {t} layer {l}: P^ differs after the resume"
            assert torch.equal(bits(qa), bits(qc)), f"step {t} layer {l}: Q differs after the resume"
    memC = C.memory()
    torch.cuda.synchronize()
    for l in range(len(SHAPES)):
        assert torch.equal(bits(memA[l]), bits(memC[l])), f"layer {l}: final memory differs"


# ----------------------------------------------------------------------------- top-k

D = (1 << 22) + 77
K = D // 100
STEPS, SPLIT = 10, 5


class TkRun:
    def __init__(self, mem=None):
        gc = lib()
        self.mem = torch.zeros(D, device=DEV) if mem is None else to_dev(mem)
        self.sel = torch.zeros(4, dtype=torch.int32, device=DEV)
        self.idx = torch.empty(K, dtype=torch.int32, device=DEV)
        self.val = torch.empty(K, device=DEV)
        self.out = torch.empty(D, device=DEV)
        self.ws = torch.empty(gc.gc_topk_workspace_bytes(D, K), dtype=torch.uint8, device=DEV)
        self.has_prev = False

    def step(self, s):
        gc = lib()
        g = to_dev(gen.c3_grad(s, D))
        gc.gc_topk_ef_encode_deferred(g, self.mem, 1.0, K, self.idx, self.val, self.sel, self.has_prev, self.ws)
        gc.gc_topk_decode(self.idx, self.val, self.out)
        self.has_prev = True

    def memory(self):
        m = self.mem.clone()
        if self.has_prev:
            lib().gc_topk_materialize(m, self.sel)
        return m


def test_topk_deferred_resume():
    print(f"case: top-k deferred, d={D} k={K}, steps 0..9, checkpoint after 4", flush=True)
    A = TkRun()
    ref = {}
    for s in range(STEPS):
        A.step(s)
        if s >= SPLIT:
            ref[s] = (A.idx.clone(), A.val.clone(), A.out.clone())
    memA = A.memory()
    B = TkRun()
    for s in range(SPLIT):
        B.step(s)
    saved = B.memory().cpu().numpy()
    del B
    torch.cuda.empty_cache()
    C = TkRun(mem=saved)
    for s in range(SPLIT, STEPS):
        C.step(s)
        torch.cuda.synchronize()
        for name, a, c in zip(("idx", "val", "out"), ref[s], (C.idx, C.val, C.out)):
            assert torch.equal(bits(a), bits(c)), f"step {s}: {name} differs after the resume"
    memC = C.memory()
    torch.cuda.synchronize()
    assert torch.equal(bits(memA), bits(memC)), "final memory differs"
