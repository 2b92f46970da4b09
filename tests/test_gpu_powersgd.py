"""GPU parity: PowerSGD EF steps vs the float64 oracle.

Tolerance (from the float32 arithmetic): relative Frobenius error <= 1e-4 for
P^, Q, the decoded matrix and the new memory, per matrix and per step.  Each
GPU step is compared with an oracle step from the same input state (the GPU's
memory and Q before the step), so float32-vs-float64 drift through the warm
start cannot fail a correct kernel.  When a reference is ~0 (full-rank
residual) the error is measured against ||M|| instead.
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


class PsgdSet:
    """Device buffers for a list of (n, m) matrices with Q capacity 4 columns."""

    def __init__(self, shapes, ranks, q_cfg=0, with_p=True, with_out=True):
        self.shapes = list(shapes)
        self.ranks = list(ranks)
        self.mem = [torch.zeros(n, m, device=DEV) for n, m in self.shapes]
        self.q = [to_dev(gen.q_init(q_cfg, l, m)) for l, (n, m) in enumerate(self.shapes)]
        self.p = [torch.zeros(4, n, device=DEV) if with_p else None for n, m in self.shapes]
        self.out = [torch.zeros(n, m, device=DEV) if with_out else None for n, m in self.shapes]
        self.ws = None

    def mats(self, grads):
        gc = lib()
        return [gc.Mat(grad=g, mem=self.mem[i], q=self.q[i], rank=self.ranks[i], p=self.p[i], out=self.out[i])
                for i, g in enumerate(grads)]

    def step(self, grads_dev, eta):
        gc = lib()
        mats = self.mats(grads_dev)
        need = gc.gc_powersgd_workspace_bytes(mats)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        gc.gc_powersgd_ef_step(mats, eta, self.ws)


def cond_p(grad_h, mem_h, q_h, eta, r):
    """Condition number of P = M Q_in (float64) for one matrix."""
    M = mem_h.astype(np.float64) + np.float64(np.float32(eta)) * oracle.grad_to_f64(grad_h).reshape(mem_h.shape)
    return float(np.linalg.cond(M @ q_h[:r].T.astype(np.float64)))


def check_step(ps, grads_h, eta, label="", cond_scaled=False):
    """One GPU step compared with the oracle from the same state; returns max error.

    cond_scaled: allow max(1e-4, 10 * 2^-24 * cond(P)) per matrix -- the float32
    limit of any method on a nearly rank-deficient P.  Only
    test_conditioning_limit_near_degenerate_p uses it; every other case holds
    the flat 1e-4 of the method statement."""
    mem_before = [t.cpu().numpy() for t in ps.mem]
    q_before = [t.cpu().numpy() for t in ps.q]
    ps.step([to_dev(g) for g in grads_h], eta)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (n, m) in enumerate(ps.shapes):
        r = ps.ranks[i]
        ref = oracle.powersgd_ef_step(grads_h[i], mem_before[i], q_before[i].T, eta, r)
        tol = TOL
        if cond_scaled:
            tol = max(TOL, 10.0 * 2.0 ** -24 * cond_p(grads_h[i], mem_before[i], q_before[i], eta, r))
        Mn = np.linalg.norm(ref["M"])
        checks = [("mem", ps.mem[i].cpu().numpy(), ref["mem"]), ("Q", ps.q[i].cpu().numpy()[:r].T, ref["Q"])]
        if ps.out[i] is not None:
            checks.append(("out", ps.out[i].cpu().numpy(), ref["out"]))
        if ps.p[i] is not None:
            checks.append(("P", ps.p[i].cpu().numpy()[:r].T, ref["P"]))
        for name, got, want in checks:
            wn = np.linalg.norm(want)
            if name in ("mem", "out") and wn < 1e-6 * Mn:
                err = np.linalg.norm(got.astype(np.float64) - want) / Mn
            else:
                err = rel_err(got, want)
            worst = max(worst, err)
            assert err <= tol, f"{label} matrix {i} ({n}x{m}, r={r}) {name}: rel err {err:.3e} (tol {tol:.1e})"
        # columns of Q beyond the rank are untouched
        if r < 4:
            assert np.array_equal(ps.q[i].cpu().numpy()[r:], q_before[i][r:])
    return worst


SHAPES = [(64, 27, 1), (64, 27, 4), (7, 2, 2), (2, 9, 2), (1, 1, 1), (100, 512, 4), (128, 576, 2),
          (33, 1030, 3), (1000, 3, 3), (4, 4608, 4), (513, 4608, 4), (17, 64, 4), (300, 2304, 1),
          (37, 8192, 4), (5, 8196, 2), (3, 4100, 1), (600, 6144, 3),
          # the wide fused classes (4096 < m <= 6144 and <= 8192) at and around their edges,
          # and the first widths past them (split path)
          (300, 4100, 4), (200, 5000, 3), (1, 6144, 1), (70, 6148, 4), (9, 8188, 2), (64, 8192, 1),
          (45, 4102, 2), (12, 8200, 4),
          # the small class (n, m <= 1024, any m) at its limits, and just past them (split path)
          (1024, 1023, 4), (2, 999, 2), (1025, 27, 2), (7, 1030, 3)]


@pytest.mark.parametrize("n,m,r", SHAPES)
def test_shapes_fp32(n, m, r):
    print(f"case: psgd {n}x{m} r={r} fp32", flush=True)
    ps = PsgdSet([(n, m)], [r])
    for t in range(3):
        g = gen.gaussian_mat(n, m, 100 + t, 1e-2)
        check_step(ps, [g], 0.8, f"step {t}")


@pytest.mark.parametrize("n,m,r", [(64, 27, 2), (513, 4608, 4), (1024, 1024, 4), (33, 1030, 3), (129, 6148, 4),
                                   (40, 8192, 3)])
def test_shapes_bf16(n, m, r):
    print(f"case: psgd {n}x{m} r={r} bf16", flush=True)
    ps = PsgdSet([(n, m)], [r])
    for t in range(2):
        g = gen.f32_to_bf16_bits(gen.gaussian_mat(n, m, 200 + t, 1e-3))
        check_step(ps, [g], 1.0, f"step {t}")


@pytest.mark.parametrize("rank", [1, 2])
def test_c2_resnet18(rank):
    print(f"case: C2 ResNet-18 r={rank}", flush=True)
    ps = PsgdSet(gen.RESNET18_MATS, [rank] * len(gen.RESNET18_MATS), q_cfg=gen.CFG_C2)
    for t in range(3):
        check_step(ps, gen.c2_grads(t), 1.0, f"C2 step {t}")


# Parity sets at the flat 1e-4 bar avoid near-degenerate P: a matrix whose
# P = M Q_in (predicted with the oracle for every step the test runs) has a
# condition number above COND_MAX is drawn again.  float32 rounding of P moves
# its column space by about eps32 * cond(P), which at cond(P) <= 100 stays far
# below 1e-4; larger condition numbers are the subject of
# test_conditioning_limit_near_degenerate_p alone.
COND_MAX = 100.0


def well_conditioned(grad_h, q_h, r, steps, eta=1.0):
    """cond(P) <= COND_MAX at each of `steps` oracle steps from m = 0 and Q_in = q_h (cols, m)."""
    mem = np.zeros(grad_h.shape, np.float32)
    q = q_h[:r].T.astype(np.float32)
    for _ in range(steps):
        M = mem.astype(np.float64) + np.float64(np.float32(eta)) * oracle.grad_to_f64(grad_h).reshape(mem.shape)
        if np.linalg.cond(M @ q.astype(np.float64)) > COND_MAX:
            return False
        ref = oracle.powersgd_ef_step(grad_h, mem, q, eta, r)
        mem, q = ref["mem"].astype(np.float32), ref["Q"].astype(np.float32)
    return True


def draw_well_conditioned(n, m, r, q_h, seed, scale, steps, bf16=False):
    """The first of the seeded draws seed, seed + 100000, ... with well-conditioned P."""
    for a in range(50):
        g = gen.gaussian_mat(n, m, seed + 100_000 * a, scale)
        if bf16:
            g = gen.f32_to_bf16_bits(g).reshape(n, m)
        if well_conditioned(g, q_h, r, steps):
            return g
    raise AssertionError(f"no well-conditioned draw for {n}x{m} r={r}")


def test_more_matrices_than_one_launch_group():
    """4100 matrices: more than one launch group (4096), fused and split shapes
    mixed, at the flat 1e-4 bar (draws with near-degenerate P replaced)."""
    print("case: 4100 small matrices", flush=True)
    shapes = [(3 + i % 5, 8 if i % 3 else 5) for i in range(4100)]
    ranks = [1 + i % 3 for i in range(4100)]
    ps = PsgdSet(shapes, ranks)
    q0 = [t.cpu().numpy() for t in ps.q]
    grads = [draw_well_conditioned(n, m, ranks[i], q0[i], 7000 + i, 1e-2, 1) for i, (n, m) in enumerate(shapes)]
    check_step(ps, grads, 1.0, "4100 matrices")


def test_conditioning_limit_near_degenerate_p():
    """The float32 limit on nearly rank-deficient P, on its own.

    The same 4100 tiny random matrices without the redraw: some P are nearly
    singular (cond(P) up to about 1.2e4).  Orthonormalising such a P in any
    float32 method moves its column space by about eps32 * cond(P), so each
    matrix is held to max(1e-4, 10 * 2^-24 * cond(P)) -- the 1e-4 bar where
    cond(P) <= 167, proportionally more above it.  Every parity set elsewhere
    keeps cond(P) <= 100 and the flat 1e-4."""
    print("case: conditioning limit, 4100 small matrices", flush=True)
    shapes = [(3 + i % 5, 8 if i % 3 else 5) for i in range(4100)]
    ranks = [1 + i % 3 for i in range(4100)]
    ps = PsgdSet(shapes, ranks)
    grads = [gen.gaussian_mat(n, m, 7000 + i, 1e-2) for i, (n, m) in enumerate(shapes)]
    check_step(ps, grads, 1.0, "4100 matrices, raw draws", cond_scaled=True)


def test_many_matrices_multi_batch():
    """70 matrices of mixed ranks and widths in one launch group (all classes and the split path)."""
    print("case: 70 mixed matrices", flush=True)
    r = gen.rng(0, gen.KIND_MISC, 400)
    shapes = [(int(r.integers(1, 300)), int(r.choice([5, 64, 100, 576, 1030]))) for _ in range(70)]
    ranks = [int(min(4, n, m, r.integers(1, 5))) for n, m in shapes]
    ps = PsgdSet(shapes, ranks)
    for t in range(2):
        grads = [gen.gaussian_mat(n, m, 500 + 100 * t + i, 1e-2) for i, (n, m) in enumerate(shapes)]
        check_step(ps, grads, 1.0, f"step {t}")


def test_null_p_and_out():
    print("case: p=NULL out=NULL", flush=True)
    ps = PsgdSet([(128, 1152), (64, 27)], [2, 3], with_p=False, with_out=False)
    check_step(ps, [gen.gaussian_mat(128, 1152, 600), gen.gaussian_mat(64, 27, 601)], 1.0)


def test_rank_switch_in_place():
    """Accordion-style 4 -> 2 -> 4 on the same Q buffer; grown columns refilled from the host."""
    print("case: rank switch", flush=True)
    n, m = 256, 2304
    ps = PsgdSet([(n, m)], [4], q_cfg=gen.CFG_C4)
    for t, r in enumerate([4, 4, 2, 2, 4, 4]):
        if r > ps.ranks[0]:
            fresh = gen.q_refill(gen.CFG_C4, 0, t, m, 4)
            ps.q[0][ps.ranks[0]:r] = to_dev(fresh[ps.ranks[0]:r])
        ps.ranks[0] = r
        check_step(ps, [gen.gaussian_mat(n, m, 700 + t, 1e-2)], 1.0, f"step {t} r={r}")


def test_determinism():
    print("case: determinism", flush=True)
    shapes = [(512, 4608), (64, 27), (1024, 1024)]
    grads = [to_dev(gen.gaussian_mat(n, m, 800 + i)) for i, (n, m) in enumerate(shapes)]
    res = []
    for _ in range(2):
        ps = PsgdSet(shapes, [4, 2, 4])
        ps.step(grads, 1.0)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy().copy() for t in ps.mem + ps.q + ps.out + ps.p])
    for a, b in zip(*res):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_c5_bert_full():
    """All 144 BERT-large matrices, bf16 gradients, fp32 memory, rank 4, at the benchmark's launch shape."""
    print("case: C5 BERT-large 144 matrices r=4 bf16", flush=True)
    ps = PsgdSet(gen.BERT_MATS, [4] * len(gen.BERT_MATS), q_cfg=gen.CFG_C5)
    grads = [gen.c5_matrix_bf16(0, l) for l in range(len(gen.BERT_MATS))]
    worst = check_step(ps, grads, 1.0, "C5")
    print(f"C5 worst relative error {worst:.2e}")


def test_max_size_one_matrix():
    """One 524287 x 4096 matrix: n*m = 2^31 - 4096, the largest a matrix may be.
    bf16 gradient from a seeded draw on the device, m0 = 0, eta = 1 (so M is the
    gradient exactly), rank 4.  The oracle's steps at this size, in pieces:
    P = M Q_in as float64 row-chunk products, P^ by the oracle's Gram-Schmidt,
    Q = M^T P^ as float64 chunk products; out and mem compared at 2048 sampled rows
    (including the first and last).  Same 1e-4 relative bar as the other cases."""
    n, m, r = 524287, 4096, 4
    print(f"case: PowerSGD max size {n}x{m} r={r} bf16", flush=True)
    rng_t = torch.Generator(device=DEV)
    rng_t.manual_seed(92)
    g32 = torch.randn(n, m, generator=rng_t, dtype=torch.float32, device=DEV).mul_(1e-3)
    g_t = g32.to(torch.bfloat16)
    del g32
    ps = PsgdSet([(n, m)], [r], q_cfg=gen.CFG_C5)
    q_in = ps.q[0].clone()
    ps.step([g_t], 1.0)
    torch.cuda.synchronize()

    chunk = 1 << 16
    qd = q_in.double().t().contiguous()                   # m x 4
    P = torch.empty(n, 4, dtype=torch.float64, device=DEV)
    for i0 in range(0, n, chunk):
        P[i0:i0 + chunk] = g_t[i0:i0 + chunk].double() @ qd
    p_ref = oracle.orthonormalize_mgs(P.cpu().numpy())
    p_ref_t = torch.from_numpy(p_ref).to(DEV)
    Q = torch.zeros(m, 4, dtype=torch.float64, device=DEV)
    for i0 in range(0, n, chunk):
        Q += g_t[i0:i0 + chunk].double().t() @ p_ref_t[i0:i0 + chunk]
    q_ref = Q.cpu().numpy()

    rs = np.random.default_rng(6)
    rows = np.unique(np.concatenate([rs.integers(0, n, 2046), [0, n - 1]]))
    rows_t = torch.from_numpy(rows).to(DEV)
    out_ref = p_ref[rows] @ q_ref.T
    M_rows = g_t[rows_t].double().cpu().numpy()
    errs = {"P": rel_err(ps.p[0].cpu().numpy()[:r].T, p_ref),
            "Q": rel_err(ps.q[0].cpu().numpy()[:r].T, q_ref),
            "out": rel_err(ps.out[0][rows_t].cpu().numpy(), out_ref),
            "mem": rel_err(ps.mem[0][rows_t].cpu().numpy(), M_rows - out_ref)}
    print("max-size relative errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for name, err in errs.items():
        assert err <= TOL, f"{name}: rel err {err:.3e}"
    del P, Q, p_ref_t, g_t, ps
    torch.cuda.empty_cache()


@pytest.mark.parametrize("seed,dtype", [(1, "f32"), (2, "bf16"), (3, "f32")])
def test_random_shape_sets(seed, dtype):
    """Seeded random sets of 12 matrices mixing every row-length class and the
    split path (m from 1 to 8299, some m % 4 != 0), random ranks: the plan's
    class sort, balanced shares and partial counts on shapes no workload has."""
    rs = np.random.default_rng(100 + seed)
    shapes, ranks = [], []
    for _ in range(12):
        n = int(rs.integers(1, 600))
        m = int(rs.choice([rs.integers(1, 64), rs.integers(64, 1025), rs.integers(1025, 2049),
                           rs.integers(2049, 4097), rs.integers(4097, 6145), rs.integers(6145, 8300)]))
        if rs.uniform() < 0.7:
            m = max(4, m - m % 4)
        shapes.append((n, m))
        ranks.append(int(rs.integers(1, min(4, n, m) + 1)))
    print(f"case: random PowerSGD set seed={seed} {dtype} {shapes} ranks={ranks}", flush=True)
    ps = PsgdSet(shapes, ranks, q_cfg=7)
    q0 = [t.cpu().numpy() for t in ps.q]
    grads = [draw_well_conditioned(n, m, ranks[l], q0[l], 300 + 13 * seed + l, 10.0 ** rs.uniform(-4, -2), 2,
                                   bf16=dtype == "bf16") for l, (n, m) in enumerate(shapes)]
    for step in range(2):
        check_step(ps, grads, 1.0, f"random set {seed} step {step}")
