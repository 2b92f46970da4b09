"""GPU parity: the top-k step with the memory in deferred form (mem keeps
acc, a 16-byte selection record marks the selected entries, the next step's
accumulate pass takes them as +0.0).

Checked bit for bit, step by step, against the explicit step
(gc_topk_ef_encode): indices, values, the decode, and the memory after
gc_topk_materialize on a copy.  The explicit step itself is checked against
the oracle in test_gpu_topk.py; one chain here is also compared with the
oracle directly.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, TopkRunner, f32_bits, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Deferred:
    """A deferred top-k chain: memory, selection record and workspace."""

    def __init__(self, d, k, mem_h):
        self.d, self.k = d, k
        self.mem = to_dev(mem_h.copy())
        self.sel = torch.zeros(4, dtype=torch.int32, device=DEV)
        self.idx = torch.empty(k, dtype=torch.int32, device=DEV)
        self.val = torch.empty(k, dtype=torch.float32, device=DEV)
        self.out = torch.empty(d, dtype=torch.float32, device=DEV)
        self.ws = torch.empty(lib().gc_topk_workspace_bytes(d, k), dtype=torch.uint8, device=DEV)
        self.has_prev = False

    def step(self, grad_t, eta, k=None):
        k = self.k if k is None else k
        lib().gc_topk_ef_encode_deferred(grad_t, self.mem, eta, k, self.idx[:k], self.val[:k], self.sel,
                                         self.has_prev, self.ws)
        lib().gc_topk_decode(self.idx[:k], self.val[:k], self.out)
        self.has_prev = True

    def memory(self):
        m = self.mem.clone()
        lib().gc_topk_materialize(m, self.sel)
        return m


def chain(d, k, grads, mems0, eta, ks=None, label=""):
    """Explicit and deferred chains side by side; compare after every step."""
    ex = TopkRunner(d, k)
    mem_x = to_dev(mems0.copy())
    df = Deferred(d, k, mems0)
    for t, g in enumerate(grads):
        kk = k if ks is None else ks[t]
        gt = to_dev(g)
        lib().gc_topk_ef_encode(gt, mem_x, eta, kk, ex.idx[:kk], ex.val[:kk], ex.ws)
        lib().gc_topk_decode(ex.idx[:kk], ex.val[:kk], ex.out)
        df.step(gt, eta, kk)
        m = df.memory()
        torch.cuda.synchronize()
        where = f"{label} step {t} (d={d}, k={kk})"
        assert torch.equal(ex.idx[:kk], df.idx[:kk]), f"{where}: indices differ"
        assert torch.equal(ex.val[:kk].view(torch.int32), df.val[:kk].view(torch.int32)), f"{where}: values differ"
        assert torch.equal(ex.out.view(torch.int32), df.out.view(torch.int32)), f"{where}: decode differs"
        assert torch.equal(mem_x.view(torch.int32), m.view(torch.int32)), f"{where}: memory differs"
    return df


def test_tiny_ten_steps_against_oracle():
    """The tiny Mem-SGD case (d = 10,000, k = 100, eta = 0.1, 10 steps) in
    deferred form, each step against the oracle from the written-out memory."""
    d, k, eta = gen.C1_D, gen.C1_K, gen.C1_ETA
    print("case: deferred top-k tiny, 10 steps vs oracle", flush=True)
    df = Deferred(d, k, np.zeros(d, np.float32))
    mem_h = np.zeros(d, np.float32)
    for t in range(10):
        g = gen.c1_grad(t)
        df.step(to_dev(g), eta)
        ref = oracle.topk_ef_step(mem_h, g, eta, k)
        m = df.memory()
        torch.cuda.synchronize()
        assert np.array_equal(df.idx.cpu().numpy(), ref["idx"]), f"step {t}: indices"
        assert np.array_equal(f32_bits(df.val), f32_bits(ref["val"])), f"step {t}: values"
        assert np.array_equal(f32_bits(m), f32_bits(ref["mem"])), f"step {t}: memory"
        mem_h = ref["mem"]


@pytest.mark.parametrize("d,k", [(1, 1), (7, 3), (1000, 1000), (4097, 1), (16384, 16384), (16384, 700),
                                 (16385, 700), (65537, 600), (300_001, 3000)])
def test_edge_sizes(d, k):
    print(f"case: deferred top-k edge d={d} k={k}", flush=True)
    grads = [gen.gaussian_vector(d, 2000 + t + d % 97) for t in range(4)]
    chain(d, k, grads, gen.gaussian_vector(d, 3000 + d % 89, 0.5), 0.37, label="edge")


@pytest.mark.parametrize("d", [50_000, 16_384])
def test_tie_heavy(d):
    """Values on a coarse grid: many ties at the threshold, so the cut index
    (the last tie taken) decides which equal keys were selected (16384: the
    single-workgroup encode)."""
    print(f"case: deferred top-k tie-heavy d={d}", flush=True)
    grads = [gen.tie_heavy(d, 1000 + t) for t in range(5)]
    chain(d, 1234, grads, gen.tie_heavy(d, 7), 1.0, label="ties")
    chain(d, 1, grads, np.zeros(d, np.float32), 1.0, label="ties k=1")


def test_full_size_and_changing_k():
    """The 25.6M flat gradient (heavy-tailed) at k = 1% and 0.1%, and an
    Accordion-like k that changes from step to step."""
    d = gen.C3_D
    print("case: deferred top-k 25.6M", flush=True)
    grads = [gen.c3_grad(t) for t in range(3)]
    for k in gen.C3_KS:
        chain(d, k, grads, np.zeros(d, np.float32), 1.0, label=f"25.6M k={k}")
    k_hi, k_lo = max(gen.C3_KS), min(gen.C3_KS)
    chain(d, k_hi, grads, np.zeros(d, np.float32), 1.0, ks=[k_hi, k_lo, k_hi], label="25.6M switching k")


def test_bf16_embedding():
    """The BERT-large embedding (30522 x 1024, bf16 gradients, k = 1%)."""
    d = gen.BERT_EMB[0] * gen.BERT_EMB[1]
    print("case: deferred top-k BERT embedding bf16", flush=True)
    grads = [gen.c5_embedding_bf16(s) for s in (0, 1, 0)]
    chain(d, gen.C5_EMB_K, grads, np.zeros(d, np.float32), 1.0, label="embedding")


def test_guess_too_high_and_materialize_restart():
    """The re-reading capture path in deferred form, then a materialize in
    place and a fresh chain from it (has_prev = 0)."""
    d, k = 1 << 20, 1000
    print("case: deferred top-k, capture fallback and restart", flush=True)
    g = gen.gaussian_vector(d, 77, 1e-3)
    run0 = 5 * (d // 256)
    g[run0:run0 + 64] = 2.0
    grads = [g, gen.gaussian_vector(d, 78, 1e-3), g]
    df = chain(d, k, grads, np.zeros(d, np.float32), 1.0, label="fallback")
    # write the memory out in place and continue with has_prev = 0
    lib().gc_topk_materialize(df.mem, df.sel)
    df.has_prev = False
    ex_mem = df.mem.clone()
    ex = TopkRunner(d, k)
    g2 = to_dev(gen.gaussian_vector(d, 79, 1e-3))
    lib().gc_topk_ef_encode(g2, ex_mem, 1.0, k, ex.idx, ex.val, ex.ws)
    df.step(g2, 1.0)
    m = df.memory()
    torch.cuda.synchronize()
    assert torch.equal(ex.idx, df.idx) and torch.equal(ex_mem.view(torch.int32), m.view(torch.int32))


@pytest.mark.parametrize("k", [10])
def test_memsgd_loop_on_the_gpu(k):
    """Mem-SGD on the strongly convex quadratic of the oracle's convergence pin
    (d = 100, curvatures in [1, 10], noise 0.1, eta_t = 8 / (mu (a + t))), run
    in float32 with the top-k step on the GPU in deferred form and the
    iterate x updated on the host: every step's (idx, val) equals the float32
    oracle step's bit for bit, so the two trajectories are the same, the final
    written-out memory too, and the run converges (f(x_T) <= 1e-2 f(x_0))."""
    d, mu, L, sigma = 100, 1.0, 10.0, 0.1
    r = gen.rng(0, gen.KIND_MISC, 92, k)
    lam = np.exp(r.uniform(np.log(mu), np.log(L), d)).astype(np.float32)
    xstar = r.standard_normal(d).astype(np.float32)
    T = int(50 * (d / k) * np.sqrt(L / mu))
    noise = r.standard_normal((T, d)).astype(np.float32)
    a = max(d / k, 16 * L / mu)
    print(f"case: Mem-SGD loop on the GPU, d={d} k={k} T={T}", flush=True)
    f = lambda x: 0.5 * float(np.sum(lam.astype(np.float64) * (x.astype(np.float64) - xstar) ** 2))
    x_gpu = np.zeros(d, np.float32)
    x_orc = np.zeros(d, np.float32)
    mem_h = np.zeros(d, np.float32)
    df = Deferred(d, k, mem_h)
    grad_t = torch.empty(d, dtype=torch.float32, device=DEV)
    for t in range(T):
        eta = np.float32(8.0 / (mu * (a + t)))
        g_gpu = (lam * (x_gpu - xstar) + np.float32(sigma) * noise[t]).astype(np.float32)
        g_orc = (lam * (x_orc - xstar) + np.float32(sigma) * noise[t]).astype(np.float32)
        grad_t.copy_(torch.from_numpy(g_gpu))
        df.step(grad_t, float(eta))
        ref = oracle.topk_ef_step(mem_h, g_orc, float(eta), k)
        idx = df.idx.cpu().numpy()
        val = df.val.cpu().numpy()
        assert np.array_equal(idx, ref["idx"]) and np.array_equal(val.view(np.uint32), ref["val"].view(np.uint32)), \
            f"step {t}: the GPU step differs from the oracle"
        x_gpu[idx] -= val
        x_orc[ref["idx"]] -= ref["val"]
        mem_h = ref["mem"]
    m = df.memory()
    torch.cuda.synchronize()
    assert np.array_equal(x_gpu.view(np.uint32), x_orc.view(np.uint32))
    assert np.array_equal(f32_bits(m), f32_bits(mem_h))
    assert f(x_gpu) <= 1e-2 * f(np.zeros(d, np.float32)), f"no convergence: f(x_T) = {f(x_gpu):.3e}"
