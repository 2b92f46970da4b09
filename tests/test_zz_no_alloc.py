"""GPU: the allocation-free norm entry point against gc_grad_norm.

gc_grad_norm_noalloc keeps its tile partials in a fixed per-device scratch
array instead of a caller workspace.  Through the C ABI, two calls in a row on
the same device -- the second with a smaller input, so a stale partial of the
first call would show -- and a call at the scratch's full size: each result
must equal gc_grad_norm's bit for bit (same kernels, same summation order),
and the first call's norms are also checked against the float64 oracle at
the 1e-4 relative bar of the other norm tests.  A call past the scratch size
must fail before any launch and leave the output untouched.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def with_workspace(layers):
    gc = lib()
    norms = torch.full((len(layers),), -1.0, device=DEV)
    ws = torch.empty(gc.gc_grad_norm_workspace_bytes(layers), dtype=torch.uint8, device=DEV)
    gc.gc_grad_norm(layers, norms, ws)
    return norms


def without_workspace(layers):
    gc = lib()
    norms = torch.full((len(layers),), -1.0, device=DEV)
    gc.gc_grad_norm_noalloc(layers, norms)
    return norms


def bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_noalloc_matches_workspace_twice_then_smaller():
    print("case: noalloc norm, call 1: 30 bf16 layers", flush=True)
    sizes = [int(s) for s in np.linspace(1, 3_000_000, 30)]
    host1 = [gen.f32_to_bf16_bits(gen.gaussian_vector(s, 40 + i, 1e-3)) for i, s in enumerate(sizes)]
    dev1 = [to_dev(h) for h in host1]
    a = without_workspace(dev1)
    b = with_workspace(dev1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b)), "call 1 differs from gc_grad_norm"
    got = a.cpu().numpy()
    for l, h in enumerate(host1):
        want = oracle.grad_norm(h)
        assert abs(got[l] - want) <= 1e-4 * want, f"call 1 layer {l}"
    print("case: noalloc norm, call 2: 4 smaller fp32 layers", flush=True)
    host2 = [gen.gaussian_vector(s, 90 + i, 1e-2) for i, s in enumerate([7, 16384, 16385, 50_000])]
    dev2 = [to_dev(h) for h in host2]
    c = without_workspace(dev2)
    d = with_workspace(dev2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(c), bits(d)), "call 2 differs from gc_grad_norm"
    got = c.cpu().numpy()
    for l, h in enumerate(host2):
        want = oracle.grad_norm(h)
        assert abs(got[l] - want) <= 1e-4 * want, f"call 2 layer {l}"


def test_noalloc_full_scratch_and_over_limit():
    gc = lib()
    tiles = gc.GC_NORM_SCRATCH_TILES
    n = tiles * 16384                      # exactly the scratch: 2^30 entries
    print(f"case: noalloc norm at the scratch size, {n} bf16 entries in 3 layers", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    big = torch.randn(n, generator=g, device=DEV, dtype=torch.float32).mul_(1e-3).to(torch.bfloat16)
    layers = [big[: n // 2], big[n // 2: n // 2 + 16384], big[n // 2 + 16384:]]
    a = without_workspace(layers)
    b = with_workspace(layers)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b))
    print("case: noalloc norm one tile over the scratch (refused)", flush=True)
    over = layers + [big[:1]]
    norms = torch.full((4,), -1.0, device=DEV)
    with pytest.raises(gc.GCError) as e:
        gc.gc_grad_norm_noalloc(over, norms)
    assert e.value.status == gc.GC_ERR_ARG
    torch.cuda.synchronize()
    assert np.all(norms.cpu().numpy() == -1.0)
    del big, layers, over
    torch.cuda.empty_cache()
