"""Pins for the top-k / error-feedback oracle (CPU only).

What fixes the oracle's results, independently of its own code:
  * a hand-worked example with ties (tests/golden/topk_hand_example.json);
  * float32 arithmetic done by NumPy's own float32 ops (a different route to
    the same two roundings) for the accumulate;
  * brute force: i is selected iff fewer than k entries precede it in the
    order (|acc| desc, index asc), checked pairwise on every C1 step and on
    tie-heavy vectors;
  * numpy.argmax for k = 1 (first maximum = lowest index), k = d, d = 1;
  * the memory invariant m_{t+1} + g_t = m_t + eta*grad of the method section,
    the k-contraction bound of top-k, the decode round trip.
A few mutation tests plant plausible mistakes in a copy of the selection and
check that the pins reject them.
"""
import json
import os

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def brute_force_selected(acc, k, chunk=512):
    """Boolean mask: i selected iff #{j : key_j > key_i or (key_j == key_i and j < i)} < k."""
    key = np.abs(acc.astype(np.float64))
    d = key.size
    j = np.arange(d)
    sel = np.zeros(d, bool)
    for s in range(0, d, chunk):
        i = np.arange(s, min(d, s + chunk))
        ki = key[i][:, None]
        before = (key[None, :] > ki) | ((key[None, :] == ki) & (j[None, :] < i[:, None]))
        sel[i] = before.sum(axis=1) < k
    return sel


def check_step(res, mem, grad, eta, k):
    acc = res["acc"]
    d = acc.size
    # accumulate: same value as NumPy float32 arithmetic (two separate roundings)
    if grad.dtype == np.uint16:
        g32 = gen.bf16_bits_as_f32(grad)
    else:
        g32 = grad
    ref = np.asarray(mem, np.float32) + np.float32(eta) * g32
    assert np.array_equal(bits(acc), bits(ref))
    # |acc - (m + eta*grad)| within the float32 rounding of two operations
    exact = mem.astype(np.float64) + np.float64(np.float32(eta)) * g32.astype(np.float64)
    err = np.abs(acc.astype(np.float64) - exact)
    bound = 2.0 ** -24 * (np.abs(np.float64(np.float32(eta)) * g32) + np.abs(acc.astype(np.float64))) + 1e-300
    assert np.all(err <= bound)
    # message: k pairs, ascending unique indices, values = acc at those indices
    idx, val = res["idx"], res["val"]
    assert idx.dtype == np.int32 and idx.size == k
    assert np.all(np.diff(idx.astype(np.int64)) > 0)
    assert np.array_equal(bits(val), bits(acc[idx]))
    # memory invariant, bitwise, with disjoint supports
    m_new, g = res["mem"], res["g"]
    assert np.array_equal(bits((m_new + g)), bits(acc))
    assert np.all(m_new[idx] == 0) and np.all(bits(m_new[idx]) == 0)  # +0.0
    rest = np.ones(d, bool)
    rest[idx] = False
    assert np.array_equal(bits(m_new[rest]), bits(acc[rest]))
    assert np.count_nonzero(g) == min(k, np.count_nonzero(acc))
    # k-contraction of top-k: ||acc - g||^2 <= (1 - k/d) ||acc||^2
    a64 = acc.astype(np.float64)
    assert np.sum((a64 - g.astype(np.float64)) ** 2) <= (1 - k / d) * np.sum(a64 ** 2) * (1 + 1e-12)
    # decode round trip: decode(message) + m_{t+1} == acc bitwise
    dec = oracle.topk_decode(idx, val, d)
    assert np.array_equal(bits(dec + m_new), bits(acc))


def test_hand_worked_example():
    ex = json.load(open(os.path.join(GOLD, "topk_hand_example.json")))
    mem = np.array(ex["mem"], np.float32)
    grad = np.array(ex["grad"], np.float32)
    for case in ex["cases"]:
        r = oracle.topk_ef_step(mem, grad, ex["eta"], case["k"])
        assert np.array_equal(r["acc"], np.array(ex["acc"], np.float32))
        assert r["idx"].tolist() == case["idx"]
        assert r["val"].tolist() == case["val"]
        assert np.array_equal(bits(r["mem"]), bits(np.array(case["mem"], np.float32)))
        check_step(r, mem, grad, ex["eta"], case["k"])
    r3 = oracle.topk_ef_step(mem, grad, ex["eta"], 3)
    assert oracle.topk_decode(r3["idx"], r3["val"], 8).tolist() == ex["decode_k3"]


def test_accumulate_wide_exponents_fp32_and_bf16():
    r = gen.rng(0, gen.KIND_MISC, 7)
    n = 200_000
    # wide exponent range, random signs: exercises subnormal-free rounding paths
    m = (r.standard_normal(n) * np.exp2(r.integers(-60, 60, n))).astype(np.float32)
    g = (r.standard_normal(n) * np.exp2(r.integers(-60, 60, n))).astype(np.float32)
    for eta in (1.0, 0.1, 3.7e-3, 1e-7):
        acc = oracle.ef_accumulate(m, g, eta)
        ref = m + np.float32(eta) * g
        assert np.array_equal(bits(acc), bits(ref))
        gb = gen.f32_to_bf16_bits(g)
        acc_b = oracle.ef_accumulate(m, gb, eta)
        ref_b = m + np.float32(eta) * gen.bf16_bits_as_f32(gb)
        assert np.array_equal(bits(acc_b), bits(ref_b))


def test_c1_ten_steps_brute_force():
    mem = np.zeros(gen.C1_D, np.float32)
    for t in range(gen.C1_STEPS):
        grad = gen.c1_grad(t)
        r = oracle.topk_ef_step(mem, grad, gen.C1_ETA, gen.C1_K)
        check_step(r, mem, grad, gen.C1_ETA, gen.C1_K)
        sel = brute_force_selected(r["acc"], gen.C1_K)
        assert np.array_equal(np.flatnonzero(sel), r["idx"])
        mem = r["mem"]


@pytest.mark.parametrize("k", [1, 7, 50, 333, 1000, 1999, 2000])
def test_tie_heavy_brute_force(k):
    d = 2000
    acc_in = gen.tie_heavy(d, seed_layer=k)
    mem = np.zeros(d, np.float32)
    r = oracle.topk_ef_step(mem, acc_in, 1.0, k)
    check_step(r, mem, acc_in, 1.0, k)
    sel = brute_force_selected(r["acc"], k)
    assert np.array_equal(np.flatnonzero(sel), r["idx"])


def test_signed_ties_lower_index_wins():
    acc = np.array([-2.0, 2.0, 1.0, -2.0, 2.0], np.float32)
    r = oracle.topk_ef_step(np.zeros(5, np.float32), acc, 1.0, 2)
    assert r["idx"].tolist() == [0, 1]
    r = oracle.topk_ef_step(np.zeros(5, np.float32), acc, 1.0, 3)
    assert r["idx"].tolist() == [0, 1, 3]


def test_special_cases():
    g = gen.gaussian_vector(1001, 3)
    mem = gen.gaussian_vector(1001, 4, 0.5)
    # k = d: everything sent, memory all +0.0
    r = oracle.topk_ef_step(mem, g, 0.25, 1001)
    assert np.array_equal(r["idx"], np.arange(1001))
    assert np.all(bits(r["mem"]) == 0)
    # k = 1: argmax of |acc| (numpy returns the first maximum = lowest index)
    r = oracle.topk_ef_step(mem, g, 0.25, 1)
    assert r["idx"].tolist() == [int(np.argmax(np.abs(r["acc"])))]
    acc = np.array([3.0, -3.0, 1.0], np.float32)
    assert oracle.topk_ef_step(np.zeros(3, np.float32), acc, 1.0, 1)["idx"].tolist() == [0]
    # d = 1
    r = oracle.topk_ef_step(np.array([0.5], np.float32), np.array([-2.0], np.float32), 0.5, 1)
    assert r["idx"].tolist() == [0] and r["val"].tolist() == [-0.5] and bits(r["mem"])[0] == 0
    # all-zero accumulator: k pairs of value 0, lowest indices
    r = oracle.topk_ef_step(np.zeros(10, np.float32), np.zeros(10, np.float32), 1.0, 3)
    assert r["idx"].tolist() == [0, 1, 2]
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros(4, np.float32), 0)
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros(4, np.float32), 5)


def test_decode_accumulate():
    idx = np.array([1, 4, 6], np.int32)
    val = np.array([0.5, -1.0, 2.0], np.float32)
    base = np.arange(8, dtype=np.float32)
    out = oracle.topk_decode(idx, val, 8, out=base, accumulate=True)
    assert out.tolist() == [0, 1.5, 2, 3, 3, 5, 8, 7]
    assert oracle.topk_decode(idx, val, 8).tolist() == [0, 0.5, 0, 0, -1, 0, 2, 0]


# ---------------------------------------------------------------- mutations

def _mutant_step(mem, grad, eta, k, mutation):
    acc = oracle.ef_accumulate(mem, grad, eta)
    if mutation == "single_rounding":   # fused multiply-add
        acc = (mem.astype(np.float64) + np.float64(np.float32(eta)) * grad.astype(np.float64)).astype(np.float32)
    if mutation == "minus":
        acc = (mem.astype(np.float64) - np.float64(np.float32(eta)) * grad.astype(np.float64)).astype(np.float32)
    key = np.abs(acc.astype(np.float64))
    if mutation == "higher_index_ties":
        order = np.lexsort((-np.arange(acc.size), -key))
    elif mutation == "signed_order":
        order = np.argsort(-acc.astype(np.float64), kind="stable")
    elif mutation == "off_by_one":
        order = np.argsort(-key, kind="stable")[1:]
    else:
        order = np.argsort(-key, kind="stable")
    idx = np.sort(order[:k]).astype(np.int32)
    g = np.zeros_like(acc)
    g[idx] = acc[idx]
    m_new = acc.copy() if mutation == "keep_memory" else acc - g
    return {"acc": acc, "idx": idx, "val": acc[idx], "g": g, "mem": m_new}


@pytest.mark.parametrize("mutation", ["single_rounding", "minus", "higher_index_ties",
                                      "signed_order", "off_by_one", "keep_memory"])
def test_pins_reject_mutations(mutation):
    caught = False
    cases = [(gen.tie_heavy(600, 99), np.zeros(600, np.float32), 1.0, 100)]
    r = gen.rng(0, gen.KIND_MISC, 8)
    m = (r.standard_normal(5000) * np.exp2(r.integers(-20, 20, 5000))).astype(np.float32)
    g = (r.standard_normal(5000) * np.exp2(r.integers(-20, 20, 5000))).astype(np.float32)
    cases.append((g, m, 0.3, 77))
    for grad, mem, eta, k in cases:
        res = _mutant_step(mem, grad, eta, k, mutation)
        try:
            check_step(res, mem, grad, eta, k)
            sel = brute_force_selected(res["acc"], k)
            assert np.array_equal(np.flatnonzero(sel), res["idx"])
        except AssertionError:
            caught = True
    assert caught, f"pins did not catch mutation {mutation}"
