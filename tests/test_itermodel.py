"""Pins of the iteration-time model (host code, no GPU).

The utility-of-compression page (method section) describes an analytic model
of compute, communication and encode-decode time but prints no formula, so the
model as a whole is "parity unpinned" against the pages.  What is pinned here:

* the ring collective costs, against a step-by-step simulation of the ring
  schedule that also checks that the schedule really reduces / gathers;
* the break-even interval, against a direct scan of the two step times;
* limits that hold for any such model, and the gradient-set shapes, against
  the workload generators.
"""
import math

import numpy as np
import pytest

import gen
from gradient_compression_error_amd import itermodel as im


def simulate_ring_allreduce(data, bandwidth, latency):
    """Ring reduce-scatter then all-gather over W workers, one chunk per message.

    Each of the 2 (W-1) steps sends one chunk from every worker to its right
    neighbour at the same time; a step lasts latency + (largest chunk sent) /
    bandwidth.  Returns (per-worker results, seconds, bytes sent per worker).
    """
    w = len(data)
    bufs = [np.array(x, dtype=np.float64) for x in data]
    chunks = np.array_split(np.arange(bufs[0].size), w)
    seconds, sent = 0.0, [0] * w
    for phase in ("reduce", "gather"):
        for step in range(w - 1):
            msgs = []
            for r in range(w):
                c = (r - step) % w if phase == "reduce" else (r + 1 - step) % w
                msgs.append((r, (r + 1) % w, c, bufs[r][chunks[c]].copy()))
            biggest = 0
            for src, dst, c, payload in msgs:
                if phase == "reduce":
                    bufs[dst][chunks[c]] += payload
                else:
                    bufs[dst][chunks[c]] = payload
                nbytes = payload.size * 4
                sent[src] += nbytes
                biggest = max(biggest, nbytes)
            seconds += latency + biggest / bandwidth
    return bufs, seconds, sent


def simulate_ring_allgather(data, bandwidth, latency):
    """Ring all-gather: in W-1 steps every worker forwards the block it got last."""
    w = len(data)
    have = [{r: np.array(data[r])} for r in range(w)]
    seconds = 0.0
    for step in range(w - 1):
        biggest = 0
        moves = []
        for r in range(w):
            blk = (r - step) % w
            moves.append(((r + 1) % w, blk, have[r][blk]))
        for dst, blk, payload in moves:
            have[dst][blk] = payload
            biggest = max(biggest, payload.size * 4)
        seconds += latency + biggest / bandwidth
    return have, seconds


@pytest.mark.parametrize("w", [2, 3, 5, 8])
def test_ring_allreduce_cost_matches_simulation(w):
    rng = np.random.default_rng(w)
    n = 64 * w                       # float32 entries, divisible into W equal chunks
    data = [rng.standard_normal(n) for _ in range(w)]
    bw, lat = 3.0e9, 7e-6
    out, seconds, sent = simulate_ring_allreduce(data, bw, lat)
    total = np.sum(data, axis=0)
    for x in out:
        np.testing.assert_allclose(x, total, rtol=1e-12, atol=1e-12)
    assert all(s == 2 * (w - 1) * (n // w) * 4 for s in sent)
    net = im.Network(w, bw, lat)
    assert seconds == pytest.approx(im.ring_allreduce_seconds(n * 4, net), rel=1e-12)


@pytest.mark.parametrize("w", [2, 4, 7])
def test_ring_allgather_cost_matches_simulation(w):
    rng = np.random.default_rng(100 + w)
    n = 50
    data = [rng.standard_normal(n) for _ in range(w)]
    have, seconds = simulate_ring_allgather(data, 2.0e9, 3e-6)
    for r in range(w):
        assert sorted(have[r]) == list(range(w))
        for blk in range(w):
            np.testing.assert_array_equal(have[r][blk], data[blk])
    assert seconds == pytest.approx(im.ring_allgather_seconds(n * 4, im.Network(w, 2.0e9, 3e-6)), rel=1e-12)


def test_single_worker_sends_nothing():
    net = im.Network(1, 1e9, 1e-5)
    assert im.ring_allreduce_seconds(1e9, net) == 0.0
    assert im.ring_allgather_seconds(1e9, net) == 0.0


def test_comm_cost_is_the_alpha_beta_form():
    rng = np.random.default_rng(5)
    for _ in range(50):
        pay = im.Payload(tuple(int(x) for x in rng.integers(0, 10**8, size=rng.integers(0, 4))),
                         int(rng.integers(0, 10**7)) * int(rng.integers(0, 2)))
        net = im.Network(int(rng.integers(1, 65)), float(10 ** rng.uniform(8, 12)), float(10 ** rng.uniform(-7, -4)))
        a, b = im.comm_cost(pay, net.workers)
        assert im.comm_seconds(pay, net) == pytest.approx(a * net.latency + b / net.bandwidth, rel=1e-12, abs=1e-18)


def _draw_case(rng):
    dense = im.Payload((int(10 ** rng.uniform(6, 9)),))
    kind = rng.integers(0, 3)
    if kind == 0:      # PowerSGD-like: two small all-reduces
        comp = im.Payload((int(10 ** rng.uniform(4, 8)), int(10 ** rng.uniform(4, 8))))
    elif kind == 1:    # top-k-like: one all-gather
        comp = im.Payload((), int(10 ** rng.uniform(4, 8)))
    else:              # a larger payload in one message
        comp = im.Payload((), int(dense.allreduce_bytes[0] * rng.uniform(0.5, 3.0)))
    compute = im.Compute(float(rng.uniform(0, 0.05)), float(rng.choice([0.0, rng.uniform(0, 0.2)])))
    t_ed = float(10 ** rng.uniform(-5, -1))
    w = int(rng.integers(2, 129))
    lat = float(rng.choice([0.0, 10 ** rng.uniform(-6, -3)]))
    return compute, dense, comp, t_ed, w, lat


def test_pays_interval_matches_a_scan_of_step_times():
    rng = np.random.default_rng(11)
    bws = np.logspace(3, 16, 1500)
    seen = {"never": 0, "below": 0, "above": 0}
    for _ in range(300):
        compute, dense, comp, t_ed, w, lat = _draw_case(rng)
        lo, hi = im.pays_interval(compute, dense, comp, t_ed, w, lat)
        seen["never" if hi == 0 else ("above" if lo > 0 else "below")] += 1
        for b in bws:
            net = im.Network(w, float(b), lat)
            t_sync = im.step_seconds(compute, dense, net)
            t_comp = im.step_seconds(compute, comp, net, t_ed)
            inside = lo < b < hi
            near = any(math.isfinite(e) and e > 0 and abs(b / e - 1) < 1e-6 for e in (lo, hi))
            if not near:
                assert (t_comp < t_sync) == inside, (compute, dense, comp, t_ed, w, lat, b, lo, hi)
    assert all(v > 0 for v in seen.values()), seen


def test_break_even_closed_form_without_window_or_latency():
    # no backward window, no latency: the dense all-reduce must outlast t_ed,
    # so B* = 2 (W-1)/W * S / t_ed
    dense, comp = im.Payload((10**9,)), im.Payload((10**6, 10**6))
    b = im.break_even_bandwidth(im.Compute(0.0, 0.0), dense, comp, 1e-3, 8, 0.0)
    assert b == pytest.approx(2 * 7 / 8 * 1e9 / 1e-3, rel=1e-12)


def test_break_even_raises_when_compression_wins_only_at_high_bandwidth():
    # a bigger payload in one all-gather against a dense all-reduce with many
    # latency terms: the compressed step wins only above some bandwidth
    dense, comp = im.Payload((10**6,)), im.Payload((), 10**6)
    with pytest.raises(ValueError):
        im.break_even_bandwidth(im.Compute(0.0, 0.0), dense, comp, 1e-6, 64, 1e-3)


def test_limits():
    compute = im.Compute(0.01, 0.03)
    dense = im.Payload((4 * 10**8,))
    net = im.Network(16, 1e10, 5e-6)
    # nothing compressed and no encode cost: identical steps
    assert im.speedup(compute, dense, dense, net, 0.0) == 1.0
    # unlimited bandwidth: both exchanges hide in the backward window and the
    # compressed step is longer by exactly t_ed
    fast = im.Network(16, 1e30, 0.0)
    comp = im.Payload((10**6,))
    assert im.step_seconds(compute, comp, fast, 2e-3) - im.step_seconds(compute, dense, fast) == pytest.approx(2e-3)
    # a cheaper encode never lowers the speed-up
    s = [im.speedup(compute, dense, comp, net, t) for t in (1e-1, 1e-2, 1e-3, 1e-4, 0.0)]
    assert all(b >= a for a, b in zip(s, s[1:]))


def test_gradient_sets_match_the_workload_shapes():
    sets = im.GRADIENT_SETS
    assert list(sets["bert-large"].matrices) == list(gen.BERT_MATS)
    assert sets["bert-large"].topk == ((gen.BERT_EMB[0] * gen.BERT_EMB[1], gen.C5_EMB_K),)
    assert list(sets["resnet18"].matrices) == list(gen.RESNET18_MATS)
    assert sets["resnet18"].dense_elems == gen.RESNET18_VECTOR_ELEMS
    assert list(sets["vgg19"].matrices) == list(gen.VGG19_MATS)
    assert sets["flat-25.6m"].topk == ((gen.C3_D, gen.C3_KS[1]),)
    # PowerSGD rank r sends r (n + m) floats per matrix
    b = sets["bert-large"].compressed()
    assert sum(b.allreduce_bytes) == 4 * 4 * sum(n + m for n, m in gen.BERT_MATS)
    assert b.allgather_bytes == 8 * gen.C5_EMB_K


def test_cli_prints_one_row_per_case(capsys):
    assert im.main(["--set", "bert-large", "--encdec-us", "1400", "--workers", "8",
                    "--bwd-ms", "0,50", "--compute-x", "1,4"]) == 0
    lines = capsys.readouterr().out.strip().splitlines()
    assert len(lines) == 4
