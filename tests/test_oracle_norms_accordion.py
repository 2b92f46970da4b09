"""Pins for the per-layer norm and the Accordion switch oracles (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_norm_closed_forms():
    assert oracle.grad_norm(np.full(16, 0.75, np.float32)) == 3.0
    assert oracle.grad_norm(np.full(4, -2.5, np.float32)) == 5.0
    assert oracle.grad_norm(np.array([3.0, 4.0], np.float32)) == 5.0
    assert oracle.grad_norm(np.array([5.0, -12.0], np.float32)) == 13.0
    assert oracle.grad_norm(np.zeros(7, np.float32)) == 0.0
    # bf16 patterns: 0x3F80 = 1.0, 0xC040 = -3.0
    assert oracle.grad_norm(np.array([0x3F80] * 9, np.uint16)) == 3.0
    assert oracle.grad_norm(np.array([0xC040, 0x4080], np.uint16)) == 5.0


def test_norm_matches_library():
    for s, n in [(1, 1000), (2, 123457), (3, 1728)]:
        g = gen.gaussian_vector(n, s, 1e-3)
        ref = np.linalg.norm(g.astype(np.float64))
        assert abs(oracle.grad_norm(g) - ref) <= 1e-14 * ref


def test_norm_wrong_mutations_caught():
    g = np.array([3.0, 4.0], np.float32)
    assert math.fsum(g.astype(np.float64)) != 5.0            # a dropped square
    assert math.fsum(g.astype(np.float64) ** 2) != 5.0        # a dropped square root


def test_accordion_rules():
    L, H = oracle.LEVEL_LOW, oracle.LEVEL_HIGH
    lv, prev = oracle.accordion_select([1.0, 2.0], [0.0, 0.0], False, 0.5)
    assert lv.tolist() == [L, L] and prev.tolist() == [1.0, 2.0]
    # exact tie rho == threshold goes to l_low (both directions)
    lv, _ = oracle.accordion_select([1.0, 3.0, 3.0], [2.0, 2.0, 4.0], True, 0.5)
    assert lv.tolist() == [L, L, H]
    # N_prev = 0
    lv, _ = oracle.accordion_select([0.5, 0.0], [0.0, 0.0], True, 0.5)
    assert lv.tolist() == [L, H]
    # a drop is as critical as a rise
    lv, _ = oracle.accordion_select([0.1, 10.0, 1.04], [1.0, 1.0, 1.0], True, 0.5)
    assert lv.tolist() == [L, L, H]
    # threshold 0: every check critical except exact zero change
    lv, _ = oracle.accordion_select([1.0, 1.5], [1.0, 1.0], True, 0.0)
    assert lv.tolist() == [L, L]


def test_c4_schedule_closed_form():
    """Decisions on the VGG-19 trajectory, from the per-layer scale alone."""
    gold = json.load(open(os.path.join(GOLD, "c4_accordion_schedule.json")))
    checks = list(range(0, gold["steps"], gold["check_every"]))
    prev, lows = None, []
    for t in checks:
        now = np.array([gen.c4_scale(t)], np.float32)
        lv, newp = oracle.accordion_select(now, prev if prev is not None else now, prev is not None,
                                           gold["threshold"])
        if lv[0] == oracle.LEVEL_LOW:
            lows.append(t)
        prev = newp
    assert lows == gold["low_checks"]
    e = math.exp(-0.05)
    assert abs((1 - e) - gold["expected_rho_quiet"]) < 1e-5
    assert abs((4 * e - 1) - gold["expected_rho_t110"]) < 1e-5
    assert abs((1 - e / 4) - gold["expected_rho_t210"]) < 1e-5


def test_c4_schedule_on_sampled_layers():
    """Same schedule from real synthetic norms of the smallest and fc layers."""
    gold = json.load(open(os.path.join(GOLD, "c4_accordion_schedule.json")))
    layers = [0, 16, 17, 18]   # 64x27 and the three fc layers
    sig0 = gen.layer_sigmas(gen.CFG_C4, len(gen.VGG19_MATS))
    prev = None
    lows = []
    for t in range(0, gold["steps"], gold["check_every"]):
        norms = []
        for l in layers:
            n, m = gen.VGG19_MATS[l]
            g = gen.gaussian_matrix(gen.CFG_C4, t, l, n, m, sig0[l] * gen.c4_scale(t))
            norms.append(oracle.grad_norm(g))
        now = np.array(norms, np.float32)
        lv, newp = oracle.accordion_select(now, prev if prev is not None else now, prev is not None,
                                           gold["threshold"])
        assert len(set(lv.tolist())) == 1     # all layers agree on this trajectory
        if lv[0] == oracle.LEVEL_LOW:
            lows.append(t)
        prev = newp
    assert lows == gold["low_checks"]


def test_accordion_topk_schedule_closed_form():
    """Accordion on top-k (oracle only): the norm trajectory gives the closed-form
    schedule, and each step's top-k takes the k of the level chosen at the last check."""
    gold = json.load(open(os.path.join(GOLD, "acc_topk_schedule.json")))
    d = 1 << 18
    k_low, k_high = gen.acc_topk_ks(d)
    assert (k_low, k_high) == (int(d * gold["k_fraction_low"]), int(d * gold["k_fraction_high"]))
    prev = np.zeros(1, np.float32)
    low, high = [], []
    mem = np.zeros(d, np.float32)
    k = None
    for t in range(gold["steps"]):
        g = gen.acc_topk_grad(t, d)
        if t % gold["check_every"] == 0:
            norm = np.array([oracle.grad_norm(g)], np.float32)
            lv, prev = oracle.accordion_select(norm, prev, t > 0, gold["threshold"])
            (low if lv[0] == oracle.LEVEL_LOW else high).append(t)
            k = k_low if lv[0] == oracle.LEVEL_LOW else k_high
        if t in (0, 10, 20):   # a few full steps: k pairs, memory invariant
            r = oracle.topk_ef_step(mem, g, 1.0, k)
            assert r["idx"].size == k and np.count_nonzero(r["g"]) == k
            assert np.array_equal((r["mem"] + r["g"]).view(np.uint32), r["acc"].view(np.uint32))
            mem = r["mem"]
    assert low == gold["low_checks"] and high == gold["high_checks"]
