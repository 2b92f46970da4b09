"""GPU: top-k steps replayed from captured HIP graphs equal eager calls.

The top-k encode (deferred memory) and decode only launch kernels and clear
their counters with kernels, so a step can be captured once per gradient
buffer and replayed.  Two sets of buffers run the same steps: one through
eager calls, one through two captured graphs (one per gradient buffer,
alternating).  Between replays the stream carries unrelated eager work and
the host synchronises; after every replay the indices, values, decode,
selection record and memory equal the eager run's bit for bit.  The uncompressed
vector call is replayed the same way."""
import numpy as np
import pytest
import torch

import gen
from gpu_util import DEV, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Path:
    def __init__(self, d, k):
        gc = lib()
        self.k = k
        self.mem = torch.zeros(d, device=DEV)
        self.sel = torch.zeros(4, dtype=torch.int32, device=DEV)
        self.idx = torch.empty(k, dtype=torch.int32, device=DEV)
        self.val = torch.empty(k, device=DEV)
        self.out = torch.empty(d, device=DEV)
        self.ws = torch.empty(gc.gc_topk_workspace_bytes(d, k), dtype=torch.uint8, device=DEV)

    def step(self, g, has_prev=True):
        gc = lib()
        gc.gc_topk_ef_encode_deferred(g, self.mem, 1.0, self.k, self.idx, self.val, self.sel, has_prev, self.ws)
        gc.gc_topk_decode(self.idx, self.val, self.out)


def same(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def test_topk_deferred_graph_replays():
    d = (1 << 22) + 77
    k = d // 100
    print(f"case: top-k deferred step as HIP graphs, d={d} k={k}", flush=True)
    grads = [to_dev(gen.c3_grad(s, d)) for s in range(2)]
    A, B = Path(d, k), Path(d, k)
    A.step(grads[0], has_prev=False)
    B.step(grads[0], has_prev=False)
    torch.cuda.synchronize()
    graphs = []
    for s in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            B.step(grads[s])
        graphs.append(g)
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, device=DEV)
    for i in range(1, 7):
        s = i % 2
        A.step(grads[s])
        junk.normal_()
        graphs[s].replay()
        junk.mul_(2.0)
        torch.cuda.synchronize()
        for name in ("idx", "val", "out", "sel", "mem"):
            assert same(getattr(A, name), getattr(B, name)), f"replay {i}: {name} differs from the eager step"


def test_passthrough_graph_replays():
    print("case: uncompressed vectors as a HIP graph", flush=True)
    gc = lib()
    vecs = [to_dev(v) for v in gen.c2_vectors(0)]
    outs_e = [torch.empty_like(v) for v in vecs]
    outs_g = [torch.empty_like(v) for v in vecs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gc.gc_passthrough(vecs, outs_g, 0.5)
    for i in range(3):
        for v in vecs:
            v.mul_(1.5)
        gc.gc_passthrough(vecs, outs_e, 0.5)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs_e, outs_g):
            assert same(a, b), f"replay {i} differs"
