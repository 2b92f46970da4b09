"""GPU parity: per-layer norms vs the oracle (relative error <= 1e-4) and the
Accordion decisions they drive on the VGG-19 trajectory."""
import json
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-4
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def gpu_norms(layers_dev):
    gc = lib()
    norms = torch.empty(len(layers_dev), device=DEV)
    ws = torch.empty(gc.gc_grad_norm_workspace_bytes(layers_dev), dtype=torch.uint8, device=DEV)
    gc.gc_grad_norm(layers_dev, norms, ws)
    torch.cuda.synchronize()
    return norms.cpu().numpy()


@pytest.mark.parametrize("bf16", [False, True])
def test_sizes(bf16):
    print(f"case: norm sizes bf16={bf16}", flush=True)
    sizes = [1, 3, 4095, 4096, 4097, 1_000_003, 17]
    host = [gen.gaussian_vector(s, s % 97, 1e-3) for s in sizes]
    if bf16:
        host = [gen.f32_to_bf16_bits(h) for h in host]
    got = gpu_norms([to_dev(h) for h in host])
    for l, h in enumerate(host):
        want = oracle.grad_norm(h)
        assert abs(got[l] - want) <= TOL * want, f"layer {l} size {sizes[l]}"
    const = gpu_norms([to_dev(np.full(16, 0.75, np.float32)), to_dev(np.zeros(5, np.float32))])
    assert const[0] == 3.0 and const[1] == 0.0


def test_many_layers():
    print("case: 200 layers", flush=True)
    host = [gen.gaussian_vector(int(s), i, 1e-2) for i, s in enumerate(np.linspace(1, 20000, 200))]
    got = gpu_norms([to_dev(h) for h in host])
    for l, h in enumerate(host):
        want = oracle.grad_norm(h)
        assert abs(got[l] - want) <= TOL * want


def test_c4_decisions_from_gpu_norms():
    """Every check of the 300-step VGG-19 trajectory: GPU norms -> host switch -> closed-form schedule;
    at three checks (quiet, up-jump, down-jump) the norms are also compared with the oracle."""
    print("case: C4 Accordion schedule", flush=True)
    gc = lib()
    gold = json.load(open(os.path.join(GOLD, "c4_accordion_schedule.json")))
    L = len(gen.VGG19_MATS)
    prev = np.zeros(L, np.float32)
    oprev = np.zeros(L, np.float32)
    lows = []
    for i, t in enumerate(range(0, gold["steps"], gold["check_every"])):
        host = gen.c4_grads(t)
        got = gpu_norms([to_dev(h) for h in host])
        lv, prev = gc.gc_accordion_select(got, prev, gold["threshold"], i > 0)
        assert len(set(lv.tolist())) == 1
        if lv[0] == gc.GC_LEVEL_LOW:
            lows.append(t)
        if t in (100, 110, 210):
            want = np.array([oracle.grad_norm(h) for h in host])
            assert np.all(np.abs(got - want) <= TOL * want)
            olv, oprev = oracle.accordion_select(want.astype(np.float32), oprev, True, gold["threshold"])
            assert np.array_equal(olv, lv)
        oprev = got.astype(np.float32)
    assert lows == gold["low_checks"]


def test_c5_all_tensors():
    print("case: C5 145 tensors bf16", flush=True)
    host = [gen.c5_matrix_bf16(0, l) for l in range(0, 144, 7)] + [gen.c5_embedding_bf16(0)]
    got = gpu_norms([to_dev(h) for h in host])
    for l, h in enumerate(host):
        want = oracle.grad_norm(h)
        assert abs(got[l] - want) <= TOL * want
