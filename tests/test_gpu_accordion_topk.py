"""GPU parity: Accordion on top-k -- the GPU norm drives the host level switch,
which picks k for the top-k error-feedback step (k = 1% at l_low, 0.1% at
l_high).  Every step's indices, values, memory and decode match the oracle bit
for bit; the decisions match the oracle's and the closed-form schedule."""
import json
import os

import numpy as np
import pytest
import torch

import gen
import oracle
from gpu_util import DEV, TopkRunner, f32_bits, lib, require_gpu, to_dev

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_accordion_topk_trajectory():
    gold = json.load(open(os.path.join(GOLD, "acc_topk_schedule.json")))
    d = 1 << 20
    k_low, k_high = gen.acc_topk_ks(d)
    print(f"case: Accordion top-k d={d} k={k_low}/{k_high} steps={gold['steps']}", flush=True)
    gc = lib()
    runners = {oracle.LEVEL_LOW: TopkRunner(d, k_low), oracle.LEVEL_HIGH: TopkRunner(d, k_high)}
    norms = torch.empty(1, device=DEV)
    mem_t = torch.zeros(d, device=DEV)
    mem_h = np.zeros(d, np.float32)
    g_t = torch.empty(d, device=DEV)
    nws = torch.empty(gc.gc_grad_norm_workspace_bytes([g_t]), dtype=torch.uint8, device=DEV)
    prev_gpu = np.zeros(1, np.float32)
    prev_orc = np.zeros(1, np.float32)
    low_checks, level = [], None
    for t in range(gold["steps"]):
        g = gen.acc_topk_grad(t, d)
        g_t.copy_(torch.from_numpy(g))
        if t % gold["check_every"] == 0:
            gc.gc_grad_norm([g_t], norms, nws)
            now = norms.cpu().numpy()
            want = oracle.grad_norm(g)
            assert abs(float(now[0]) - want) <= 1e-4 * want
            lv, prev_gpu = gc.gc_accordion_select(now, prev_gpu, gold["threshold"], t > 0)
            lv_o, prev_orc = oracle.accordion_select(np.array([want], np.float32), prev_orc, t > 0,
                                                     gold["threshold"])
            assert int(lv[0]) == int(lv_o[0]), f"level differs at t={t}"
            level = int(lv[0])
            if level == oracle.LEVEL_LOW:
                low_checks.append(t)
        r = runners[level]
        r.encode(g_t, mem_t, 1.0)
        r.decode()
        ref = oracle.topk_ef_step(mem_h, g, 1.0, r.k)
        torch.cuda.synchronize()
        assert np.array_equal(r.idx.cpu().numpy(), ref["idx"]), f"indices differ at t={t}"
        assert np.array_equal(f32_bits(r.val), f32_bits(ref["val"])), f"values differ at t={t}"
        assert np.array_equal(f32_bits(mem_t), f32_bits(ref["mem"])), f"memory differs at t={t}"
        assert np.array_equal(f32_bits(r.out), f32_bits(ref["g"])), f"decode differs at t={t}"
        mem_h = ref["mem"]
    assert low_checks == gold["low_checks"]
