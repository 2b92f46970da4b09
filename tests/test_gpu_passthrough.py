"""GPU parity: vectors sent uncompressed (gc_passthrough), out = fl32(eta * g),
bit for bit against the oracle: edge lengths around the 4-entry vector width
and the 4096-entry tile, float32 and bf16 gradients, more vectors than one
launch holds, and the ResNet-18 BN/bias set."""
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


def run(host, eta):
    gc = lib()
    grads = [to_dev(h) for h in host]
    outs = [torch.full((h.size,), float("nan"), device=DEV) for h in host]
    gc.gc_passthrough(grads, outs, eta)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("eta", [1.0, 0.1])
def test_edge_lengths(bf16, eta):
    print(f"case: passthrough edge lengths bf16={bf16} eta={eta}", flush=True)
    sizes = [1, 3, 4, 5, 63, 4095, 4096, 4097, 8193, 100_003]
    host = [gen.gaussian_vector(s, 60 + i, 1e-2) for i, s in enumerate(sizes)]
    if bf16:
        host = [gen.f32_to_bf16_bits(h) for h in host]
    outs = run(host, eta)
    for h, o in zip(host, outs):
        assert np.array_equal(f32_bits(o), f32_bits(oracle.passthrough_step(h, eta))), f"length {h.size}"


def test_more_vectors_than_one_launch():
    print("case: passthrough 250 vectors", flush=True)
    host = [gen.gaussian_vector(1 + (i * 37) % 700, 300 + i, 1.0) for i in range(250)]
    outs = run(host, 0.8)
    for h, o in zip(host, outs):
        assert np.array_equal(f32_bits(o), f32_bits(oracle.passthrough_step(h, 0.8)))


def test_resnet18_vectors():
    print("case: passthrough ResNet-18 BN/bias set", flush=True)
    for t in range(2):
        host = gen.c2_vectors(t)
        outs = run(host, 1.0)
        for h, o in zip(host, outs):
            assert np.array_equal(f32_bits(o), f32_bits(oracle.passthrough_step(h, 1.0)))


def test_prepared_call_equals_direct_call():
    print("case: passthrough prepared call, ResNet-18 set, 3 calls", flush=True)
    gc = lib()
    for t in range(2):
        host = gen.c2_vectors(t)
        grads = [to_dev(h) for h in host]
        direct = [torch.full((h.size,), float("nan"), device=DEV) for h in host]
        outs = [torch.full((h.size,), float("nan"), device=DEV) for h in host]
        call = gc.gc_passthrough_prepare(grads, outs)
        for eta in (1.0, 0.3, 1.0):
            gc.gc_passthrough(grads, direct, eta)
            call(eta)
            torch.cuda.synchronize()
            for h, a, b in zip(host, direct, outs):
                assert np.array_equal(f32_bits(a), f32_bits(b))
                assert np.array_equal(f32_bits(b), f32_bits(oracle.passthrough_step(h, eta)))
