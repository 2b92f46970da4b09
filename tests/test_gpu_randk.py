"""GPU parity: rand-k error-feedback encode vs the CPU oracle, bit for bit,
on the same seeded index subsets; decode through gc_topk_decode."""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, f32_bits, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def check(grad_h, mem_h, eta, idx_h, mem_t=None):
    gc = lib()
    d, k = mem_h.size, idx_h.size
    mem_t = to_dev(mem_h.copy()) if mem_t is None else mem_t
    idx_t = torch.from_numpy(idx_h).to(DEV)
    val_t = torch.empty(k, device=DEV)
    out_t = torch.empty(d, device=DEV)
    gc.gc_randk_ef_encode(to_dev(grad_h), mem_t, eta, idx_t, val_t)
    gc.gc_topk_decode(idx_t, val_t, out_t)
    ref = oracle.randk_ef_step(mem_h, grad_h, eta, idx_h)
    torch.cuda.synchronize()
    assert np.array_equal(f32_bits(val_t), f32_bits(ref["val"]))
    assert np.array_equal(f32_bits(mem_t), f32_bits(ref["mem"]))
    assert np.array_equal(f32_bits(out_t), f32_bits(ref["g"]))
    return ref, mem_t


@pytest.mark.parametrize("d,k", [(1, 1), (3, 2), (4095, 17), (4096, 4096), (4097, 5), (12289, 12289),
                                 (100_003, 1000), (300_001, 3)])
def test_sizes(d, k):
    print(f"case: rand-k d={d} k={k}", flush=True)
    g = gen.gaussian_vector(d, 21)
    mem = gen.gaussian_vector(d, 22, 0.3)
    check(g, mem, 0.1, gen.randk_indices(0, d, d, k))


def test_steps_memory_on_device():
    d, k = 100_003, 997
    print(f"case: rand-k 8 steps d={d} k={k}", flush=True)
    mem_h = np.zeros(d, np.float32)
    mem_t = None
    for t in range(8):
        g = gen.gaussian_vector(d, 100 + t)
        ref, mem_t = check(g, mem_h, 0.5, gen.randk_indices(1, t, d, k), mem_t)
        mem_h = ref["mem"]


def test_bf16_grad():
    d, k = 65_537, 655
    print(f"case: rand-k bf16 d={d}", flush=True)
    g = gen.f32_to_bf16_bits(gen.gaussian_vector(d, 31, 1e-3))
    check(g, gen.gaussian_vector(d, 32, 1e-3), 1.0, gen.randk_indices(2, 0, d, k))


def test_c3_full_size():
    d = gen.C3_D
    k = d // 100
    print(f"case: rand-k full size d={d} k={k}", flush=True)
    check(gen.c3_grad(0), np.zeros(d, np.float32), 1.0, gen.randk_indices(gen.CFG_C3, 0, d, k))
