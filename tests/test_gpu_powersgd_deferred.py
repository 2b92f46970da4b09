"""GPU parity: the PowerSGD step with the error-feedback memory held in
deferred form (mem keeps M, p keeps P^, q keeps Q; the next step rebuilds
m' = M - P^ Q^T in its first pass).

Two checks:
  * bit for bit against the explicit step (gc_powersgd_ef_step) from the same
    start, over several steps, rank switches included: out, P^ and Q after
    every step, and the memory after gc_powersgd_materialize on a copy.  Both
    paths form every value with the same float32 operations in the same order.
  * against the float64 oracle, step by step from the same state, at the
    1e-4 relative Frobenius bar of the explicit step's tests.
The explicit step is itself checked against the oracle in test_gpu_powersgd.py.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, lib, rel_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Set:
    """Device buffers of a matrix list (Q and P with 4 columns of capacity)."""

    def __init__(self, shapes, ranks, q_cfg=0):
        self.shapes, self.ranks = list(shapes), list(ranks)
        self.mem = [torch.zeros(n, m, device=DEV) for n, m in self.shapes]
        self.q = [to_dev(gen.q_init(q_cfg, l, m)) for l, (n, m) in enumerate(self.shapes)]
        self.p = [torch.zeros(4, n, device=DEV) for n, m in self.shapes]
        self.out = [torch.zeros(n, m, device=DEV) for n, m in self.shapes]
        self.prev = [0] * len(self.shapes)
        self.ws = None

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

    def explicit(self, grads, eta):
        mats = self.mats(grads)
        lib().gc_powersgd_ef_step(mats, eta, self._ws(mats))

    def deferred(self, grads, eta):
        mats = self.mats(grads)
        lib().gc_powersgd_ef_step_deferred(mats, self.prev, eta, self._ws(mats))
        self.prev = list(self.ranks)

    def memory(self):
        """The memory m' the method carries, written out into copies of mem."""
        copies = [t.clone() for t in self.mem]
        mats = self.mats([None] * len(copies), mem=copies)
        lib().gc_powersgd_materialize(mats, self.prev, self._ws(mats))
        return copies


def bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def compare_bitwise(A, B, label):
    memB = B.memory()
    torch.cuda.synchronize()
    for i, (n, m) in enumerate(A.shapes):
        r = A.ranks[i]
        for name, x, y in [("out", A.out[i], B.out[i]), ("P", A.p[i][:r], B.p[i][:r]), ("Q", A.q[i][:r], B.q[i][:r]),
                           ("mem", A.mem[i], memB[i])]:
            assert bits_equal(x, y), f"{label}: matrix {i} ({n}x{m}, r={r}) {name} differs from the explicit step"


def run_pair(shapes, ranks, grads_fn, steps, eta=1.0, q_cfg=0, label=""):
    A, B = Set(shapes, ranks, q_cfg), Set(shapes, ranks, q_cfg)
    for t in range(steps):
        g = [to_dev(x) for x in grads_fn(t)]
        A.explicit(g, eta)
        B.deferred(g, eta)
        compare_bitwise(A, B, f"{label} step {t}")


def test_single_classes_fp32():
    """One matrix per launch: each psgd_pq class kernel alone (row lengths 1024,
    2048, 4096) and the split path (m % 4 != 0, m > 4096)."""
    for (n, m), r in [((300, 1024), 4), ((130, 2048), 3), ((77, 4096), 2), ((64, 27), 2), ((33, 4608), 4),
                      ((5, 1030), 1)]:
        print(f"case: deferred vs explicit {n}x{m} r={r} fp32", flush=True)
        run_pair([(n, m)], [r], lambda t: [gen.gaussian_mat(n, m, 900 + t, 1e-2)], 3, eta=0.8,
                 label=f"{n}x{m}")


def test_single_classes_bf16():
    for (n, m), r in [((1024, 1024), 4), ((96, 4096), 4), ((64, 27), 2)]:
        print(f"case: deferred vs explicit {n}x{m} r={r} bf16", flush=True)
        run_pair([(n, m)], [r], lambda t: [gen.f32_to_bf16_bits(gen.gaussian_mat(n, m, 950 + t, 1e-3))], 3,
                 label=f"{n}x{m} bf16")


@pytest.mark.parametrize("rank", [1, 2])
def test_resnet18_set(rank):
    """The ResNet-18 set: one launch of the team kernel for its fused classes, plus the split path."""
    print(f"case: deferred vs explicit ResNet-18 r={rank}", flush=True)
    run_pair(gen.RESNET18_MATS, [rank] * len(gen.RESNET18_MATS), gen.c2_grads, 4, q_cfg=gen.CFG_C2,
             label=f"ResNet-18 r{rank}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wide_classes(dtype):
    """Each wide fused class alone (4096 < m <= 6144 on 768 threads with two
    float4 per thread, 6144 < m <= 8192 on 1024 threads) at its edges, three
    steps, deferred against explicit bit for bit."""
    for (n, m), r in [((300, 4100), 4), ((96, 4608), 2), ((33, 6144), 3), ((130, 6148), 4), ((40, 8192), 1),
                      ((7, 8188), 4)]:
        print(f"case: deferred vs explicit wide {n}x{m} r={r} {dtype}", flush=True)

        def grads(t, n=n, m=m):
            g = gen.gaussian_mat(n, m, 1400 + t, 1e-2)
            return [gen.f32_to_bf16_bits(g).reshape(n, m) if dtype == "bf16" else g]
        run_pair([(n, m)], [r], grads, 3, eta=0.9, label=f"{n}x{m} {dtype}")


def test_small_class():
    """Matrices with n, m <= 1024 whose rows are not float4-wide (any m) are
    done whole by one workgroup: alone (their own launch) and beside fused
    classes (inside the team launch), with a rank switch, deferred against
    explicit bit for bit."""
    alone = [(1024, 1023), (1000, 3), (1, 1), (64, 27), (2, 999)]
    mixed = alone + [(300, 1024), (64, 576), (33, 2048)]
    for shapes in (alone, mixed):
        sched = [[min(4, n, m) for n, m in shapes], [min(2, n, m) for n, m in shapes],
                 [min(4, n, m) for n, m in shapes], [min(3, n, m) for n, m in shapes]]
        A, B = Set(shapes, sched[0], gen.CFG_C4), Set(shapes, sched[0], gen.CFG_C4)
        for t, ranks in enumerate(sched):
            print(f"case: deferred small class {len(shapes)} matrices step {t} ranks={ranks}", flush=True)
            for S in (A, B):
                for i, r in enumerate(ranks):
                    if r > S.ranks[i]:
                        fresh = gen.q_refill(gen.CFG_C4, i, t, shapes[i][1], 4)
                        S.q[i][S.ranks[i]:r] = to_dev(fresh[S.ranks[i]:r])
                S.ranks = list(ranks)
            g = [to_dev(gen.gaussian_mat(n, m, 1600 + 10 * t + i, 1e-2)) for i, (n, m) in enumerate(shapes)]
            A.explicit(g, 1.0)
            B.deferred(g, 1.0)
            compare_bitwise(A, B, f"small class step {t}")


def test_wide_rank_switches():
    """Accordion-style switches on wide rows: 4 -> 2 (the previous Q columns 2,
    3 still rebuild the residual), 2 -> 4 with refilled columns, 4 -> 1 -> 3."""
    shapes = [(96, 4608), (40, 8192), (130, 6148), (64, 1024)]
    sched = [[4, 4, 4, 4], [2, 2, 2, 2], [4, 4, 2, 4], [1, 2, 4, 1], [3, 1, 3, 4]]
    A, B = Set(shapes, sched[0], gen.CFG_C4), Set(shapes, sched[0], gen.CFG_C4)
    for t, ranks in enumerate(sched):
        print(f"case: deferred wide rank switch step {t} ranks={ranks}", flush=True)
        for S in (A, B):
            for i, r in enumerate(ranks):
                if r > S.ranks[i]:
                    fresh = gen.q_refill(gen.CFG_C4, i, t, shapes[i][1], 4)
                    S.q[i][S.ranks[i]:r] = to_dev(fresh[S.ranks[i]:r])
            S.ranks = list(ranks)
        g = [to_dev(gen.gaussian_mat(n, m, 1500 + 10 * t + i, 1e-2)) for i, (n, m) in enumerate(shapes)]
        A.explicit(g, 1.0)
        B.deferred(g, 1.0)
        compare_bitwise(A, B, f"wide rank switch step {t}")


def test_max_size_wide_rows():
    """One 262143 x 8192 matrix (n*m = 2^31 - 8192, the largest of the widest
    fused class), bf16 gradients drawn on the device, rank 4: two deferred
    steps against two explicit ones, bit for bit on the device."""
    n, m, r = 262143, 8192, 4
    print(f"case: deferred vs explicit, wide max size {n}x{m} r={r} bf16", flush=True)
    rng_t = torch.Generator(device=DEV)
    rng_t.manual_seed(94)
    A, B = Set([(n, m)], [r], gen.CFG_C5), Set([(n, m)], [r], gen.CFG_C5)
    for t in range(2):
        g = (torch.randn(n, m, generator=rng_t, dtype=torch.float32, device=DEV) * 1e-3).to(torch.bfloat16)
        A.explicit([g], 1.0)
        B.deferred([g], 1.0)
        del g
        compare_bitwise(A, B, f"wide max size step {t}")
    del A, B
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed,dtype", [(4, "f32"), (5, "bf16")])
def test_random_shape_sets(seed, dtype):
    rs = np.random.default_rng(200 + seed)
    shapes, ranks = [], []
    for _ in range(12):
        n = int(rs.integers(1, 500))
        m = int(rs.choice([rs.integers(1, 64), rs.integers(64, 1025), rs.integers(1025, 2049),
                           rs.integers(2049, 4097), rs.integers(4097, 6145), rs.integers(6145, 8300)]))
        if rs.uniform() < 0.7:
            m = max(4, m - m % 4)
        shapes.append((n, m))
        ranks.append(int(rs.integers(1, min(4, n, m) + 1)))
    print(f"case: deferred random set seed={seed} {dtype} {shapes} ranks={ranks}", flush=True)

    def grads(t):
        out = []
        for l, (n, m) in enumerate(shapes):
            g = gen.gaussian_mat(n, m, 1000 + 17 * seed + 31 * t + l, 1e-2)
            out.append(gen.f32_to_bf16_bits(g).reshape(n, m) if dtype == "bf16" else g)
        return out

    run_pair(shapes, ranks, grads, 3, q_cfg=7, label=f"random set {seed}")


def test_rank_switches():
    """Accordion-style switches on mixed shapes: 4 -> 2 (the old columns 2, 3
    of Q and P still rebuild the residual), 2 -> 4 (columns 2, 3 of Q refilled
    before the call), 4 -> 1 -> 3, in both paths."""
    shapes = [(256, 2304), (64, 27), (128, 1024), (40, 4608)]
    sched = [[4, 2, 4, 4], [4, 2, 4, 4], [2, 2, 2, 1], [2, 2, 1, 1], [4, 2, 2, 3], [4, 1, 4, 3]]
    A, B = Set(shapes, sched[0], gen.CFG_C4), Set(shapes, sched[0], gen.CFG_C4)
    for t, ranks in enumerate(sched):
        print(f"case: deferred rank switch step {t} ranks={ranks}", flush=True)
        for S in (A, B):
            for i, r in enumerate(ranks):
                if r > S.ranks[i]:
                    fresh = gen.q_refill(gen.CFG_C4, i, t, shapes[i][1], 4)
                    S.q[i][S.ranks[i]:r] = to_dev(fresh[S.ranks[i]:r])
            S.ranks = list(ranks)
        g = [to_dev(gen.gaussian_mat(n, m, 1100 + 10 * t + i, 1e-2)) for i, (n, m) in enumerate(shapes)]
        A.explicit(g, 1.0)
        B.deferred(g, 1.0)
        compare_bitwise(A, B, f"rank switch step {t}")


def test_materialize_then_explicit_and_prev_zero():
    """Materialize in place, then continue with the explicit step (and a
    deferred call with prev_rank 0): the memory is then the memory itself."""
    shapes = [(100, 512), (7, 30)]
    A, B = Set(shapes, [3, 2]), Set(shapes, [3, 2])
    g = [[to_dev(gen.gaussian_mat(n, m, 1200 + 10 * t + i, 1e-2)) for i, (n, m) in enumerate(shapes)]
         for t in range(4)]
    A.explicit(g[0], 1.0)
    B.deferred(g[0], 1.0)
    B.deferred(g[1], 1.0)
    A.explicit(g[1], 1.0)
    # B's memory written out in place; B continues with the explicit step
    mats = B.mats([None, None])
    lib().gc_powersgd_materialize(mats, B.prev, B._ws(mats))
    B.prev = [0, 0]
    A.explicit(g[2], 1.0)
    B.explicit(g[2], 1.0)
    compare_bitwise(A, B, "after materialize + explicit")
    A.explicit(g[3], 1.0)
    B.deferred(g[3], 1.0)          # prev_rank 0: mem holds the memory itself
    compare_bitwise(A, B, "deferred from prev_rank 0")
    # a materialize call with prev_rank 0 leaves mem alone
    before = [t.clone() for t in A.mem]
    mats = A.mats([None, None])
    lib().gc_powersgd_materialize(mats, [0, 0], A._ws(mats))
    torch.cuda.synchronize()
    for x, y in zip(before, A.mem):
        assert bits_equal(x, y)


def test_oracle_parity_chain():
    """Deferred steps on the ResNet-18 set (rank 2) against the float64 oracle,
    each step from the GPU's state before it (materialized memory and Q)."""
    shapes = gen.RESNET18_MATS
    S = Set(shapes, [2] * len(shapes), gen.CFG_C2)
    for t in range(3):
        print(f"case: deferred vs oracle ResNet-18 step {t}", flush=True)
        mem_before = [x.cpu().numpy() for x in S.memory()]
        q_before = [x.cpu().numpy() for x in S.q]
        grads_h = gen.c2_grads(t)
        S.deferred([to_dev(x) for x in grads_h], 1.0)
        mem_after = [x.cpu().numpy() for x in S.memory()]
        torch.cuda.synchronize()
        for i, (n, m) in enumerate(shapes):
            ref = oracle.powersgd_ef_step(grads_h[i], mem_before[i], q_before[i].T, 1.0, 2)
            Mn = np.linalg.norm(ref["M"])
            for name, got, want in [("mem", mem_after[i], ref["mem"]), ("out", S.out[i].cpu().numpy(), ref["out"]),
                                    ("Q", S.q[i].cpu().numpy()[:2].T, ref["Q"]),
                                    ("P", S.p[i].cpu().numpy()[:2].T, ref["P"])]:
                if name in ("mem", "out") and np.linalg.norm(want) < 1e-6 * Mn:
                    err = np.linalg.norm(got.astype(np.float64) - want) / Mn
                else:
                    err = rel_err(got, want)
                assert err <= TOL, f"step {t} matrix {i} ({n}x{m}) {name}: rel err {err:.3e}"


def test_bert_large_set():
    """All 144 BERT-large matrices (bf16 gradients, rank 4): the separate class
    launches of the benchmark's launch shape, two steps, bit for bit."""
    print("case: deferred vs explicit BERT-large 144 matrices", flush=True)
    shapes = gen.BERT_MATS
    grads = [[to_dev(gen.c5_matrix_bf16(s, l)) for l in range(len(shapes))] for s in range(2)]
    A, B = Set(shapes, [4] * len(shapes), gen.CFG_C5), Set(shapes, [4] * len(shapes), gen.CFG_C5)
    for t in range(3):
        A.explicit(grads[t % 2], 1.0)
        B.deferred(grads[t % 2], 1.0)
        compare_bitwise(A, B, f"BERT-large step {t}")
    del grads, A, B
    torch.cuda.empty_cache()


def test_several_launch_groups():
    """4100 small matrices (more than one launch group of 4096), fused and split
    shapes mixed, mixed ranks: the per-group tables and decode tiles."""
    print("case: deferred vs explicit, 4100 matrices", flush=True)
    shapes = [(3 + i % 5, 8 if i % 3 else 5) for i in range(4100)]
    ranks = [1 + i % 3 for i in range(4100)]
    run_pair(shapes, ranks, lambda t: [gen.gaussian_mat(n, m, 1300 + 7 * t + i, 1e-2) for i, (n, m) in
                                       enumerate(shapes)], 2, label="4100 matrices")


def test_max_size_one_matrix():
    """One 524287 x 4096 matrix (n*m = 2^31 - 4096, the largest the ABI takes),
    bf16 gradients drawn on the device, rank 4: three deferred steps against
    three explicit ones, compared on the device bit for bit (out, P^, Q, and
    the memory written out by gc_powersgd_materialize)."""
    n, m, r = 524287, 4096, 4
    print(f"case: deferred vs explicit, max size {n}x{m} r={r} bf16", flush=True)
    rng_t = torch.Generator(device=DEV)
    rng_t.manual_seed(93)
    A, B = Set([(n, m)], [r], gen.CFG_C5), Set([(n, m)], [r], gen.CFG_C5)
    for t in range(3):
        g = (torch.randn(n, m, generator=rng_t, dtype=torch.float32, device=DEV) * 1e-3).to(torch.bfloat16)
        A.explicit([g], 1.0)
        B.deferred([g], 1.0)
        del g
        compare_bitwise(A, B, f"max size step {t}")
    del A, B
    torch.cuda.empty_cache()
