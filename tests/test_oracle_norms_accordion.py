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
