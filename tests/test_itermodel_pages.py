"""The iteration-time model against the results the utility page reports.

"On the Utility of Gradient Compression in Distributed Training Systems"
prints no formula and no worked example with its inputs, so the model cannot
be pinned to a number of the pages.  Its results section does state five
findings that any model of its kind has to reproduce; each test below checks
one of them as a property of the model, over seeded random draws of compute
times, payloads, worker counts and bandwidths (and, where the finding is about
a direction, one concrete case that shows it strictly):

1. above some link bandwidth a compressor with a fixed encode-decode cost is
   slower than synchronous SGD (the page finds this for PowerSGD);
2. an encode-decode time longer than the window in which the dense exchange
   would hide removes any speed-up, whatever the compression ratio;
3. a compressor whose payload is all-reduced (PowerSGD) scales with the worker
   count, one whose payload is all-gathered (sign SGD, top-k) does not;
4. faster computation (the page simulates up to 4x) raises what compression
   gains (the page reports up to 1.75x for PowerSGD rank 4 at 4x);
5. a shorter encode-decode time helps more than a higher compression ratio.

A model that drops the overlap of communication with the backward pass, adds
the encode-decode time on the network side, prices an all-gather like an
all-reduce, or scales t_ed with compute fails at least one of them.
Host code only.
"""
import math

import numpy as np
import pytest

from gradient_compression_error_amd import itermodel as im

GBIT = 1e9 / 8          # bytes/s in one Gbit/s


def draws(seed, count=300):
    """Random cases: compute times, a dense gradient of 4-400 MB, a payload
    compressed 10x-1000x, W in 2..96, t_ed from 0.1 ms to 200 ms."""
    rng = np.random.default_rng(seed)
    for _ in range(count):
        t_fwd = float(rng.uniform(0.0, 0.1))
        t_bwd = float(rng.uniform(0.0, 0.3))
        dense_bytes = int(10 ** rng.uniform(6.6, 8.6))
        ratio = float(10 ** rng.uniform(1, 3))
        w = int(rng.integers(2, 97))
        t_ed = float(10 ** rng.uniform(-4, math.log10(0.2)))
        comp_bytes = max(1, int(dense_bytes / ratio))
        # PowerSGD-like payload: two all-reduces (P then Q')
        comp = im.Payload((comp_bytes // 2, comp_bytes - comp_bytes // 2))
        yield im.Compute(t_fwd, t_bwd), im.Payload((dense_bytes,)), comp, t_ed, w


def test_fixed_encode_cost_loses_above_a_bandwidth():
    """Finding 1: with t_ed > 0 the break-even bandwidth is finite; below it
    the compressed step is faster, above it slower; at unlimited bandwidth the
    speed-up is (t_fwd + t_bwd) / (t_fwd + t_bwd + t_ed) < 1."""
    for compute, dense, comp, t_ed, w in draws(1):
        b_star = im.break_even_bandwidth(compute, dense, comp, t_ed, w)
        assert math.isfinite(b_star)
        if b_star > 0:
            assert im.speedup(compute, dense, comp, im.Network(w, b_star / 10), t_ed) > 1
        assert im.speedup(compute, dense, comp, im.Network(w, max(b_star, 1.0) * 10), t_ed) < 1
        limit = (compute.t_fwd + compute.t_bwd) / (compute.t_fwd + compute.t_bwd + t_ed)
        assert im.speedup(compute, dense, comp, im.Network(w, 1e30), t_ed) == pytest.approx(limit, rel=1e-12)
    # without an encode-decode cost (and no latency) a smaller payload never loses
    for compute, dense, comp, _, w in draws(2, 50):
        for b in 10 ** np.linspace(7, 12, 21):
            assert im.speedup(compute, dense, comp, im.Network(w, float(b)), 0.0) >= 1.0


def test_encode_longer_than_the_hiding_window_gives_no_speedup():
    """Finding 2: once t_ed reaches the part of the dense exchange that the
    backward pass does not hide, no payload, not even an empty one, helps."""
    rng = np.random.default_rng(3)
    for compute, dense, comp, _, w in draws(4):
        net = im.Network(w, float(10 ** rng.uniform(8, 10.5)))
        exposed = max(0.0, im.comm_seconds(dense, net) - compute.t_bwd)
        t_ed = exposed * float(rng.uniform(1.0, 3.0))
        for pay in (comp, im.Payload()):
            assert im.speedup(compute, dense, pay, net, t_ed) <= 1.0 + 1e-12
        # just inside the window an empty payload does pay, if anything is exposed
        if exposed > 1e-6:
            assert im.speedup(compute, dense, im.Payload(), net, 0.5 * exposed) > 1.0


def test_allgather_payload_stops_paying_as_workers_grow():
    """Finding 3: an all-gathered payload of S_c bytes per worker costs
    (W-1) S_c / B, growing with W, while an all-reduced one stays under
    2 S_c / B.  With no latency the all-gather compressor pays at no bandwidth
    once W S_c >= 2 S_dense; the all-reduce one keeps a positive B*."""
    compute = im.Compute(0.02, 0.06)
    dense = im.Payload((100_000_000,))
    s_c = 1_000_000                      # 1% of the dense bytes per worker
    gather, reduce_ = im.Payload((), s_c), im.Payload((s_c,))
    t_ed = 2e-3
    net_b = 10 * GBIT
    prev_r = None
    for w in (2, 4, 8, 16, 32, 64, 96, 128, 200, 256):
        net = im.Network(w, net_b)
        tg, tr = im.comm_seconds(gather, net), im.comm_seconds(reduce_, net)
        assert tg == pytest.approx((w - 1) * s_c / net_b, rel=1e-12)
        assert tr < 2 * s_c / net_b
        assert tg / tr == pytest.approx(w / 2, rel=1e-12)
        lo, hi = im.pays_interval(compute, dense, gather, t_ed, w)
        if w * s_c >= 2 * dense.allreduce_bytes[0]:
            assert (lo, hi) == (0.0, 0.0), w
        else:
            assert hi > 0, w
        b_r = im.break_even_bandwidth(compute, dense, reduce_, t_ed, w)
        assert b_r > 0
        # same bytes, same t_ed: the all-gather compressor is never the faster one
        s_g = im.speedup(compute, dense, gather, net, t_ed)
        s_r = im.speedup(compute, dense, reduce_, net, t_ed)
        assert s_g <= s_r * (1 + 1e-12), w
        if prev_r is not None:
            # the all-reduce compressor's speed-up and break-even move only through (W-1)/W
            assert s_r >= prev_r[0] * (1 - 1e-12) and b_r >= prev_r[1] * (1 - 1e-12)
        prev_r = (s_r, b_r)
    # at 2 workers both pay at 10 Gbit/s; at 256 the all-gather one loses
    assert im.speedup(compute, dense, gather, im.Network(2, net_b), t_ed) > 1
    assert im.speedup(compute, dense, gather, im.Network(256, net_b), t_ed) < 1
    assert im.speedup(compute, dense, reduce_, im.Network(256, net_b), t_ed) > 1


def test_faster_compute_raises_the_gain():
    """Finding 4: with t_ed fixed, wherever compression pays at 1x compute it
    pays at least as much at f x (1 < f <= 4), and the break-even bandwidth
    does not fall."""
    rng = np.random.default_rng(5)
    for compute, dense, comp, t_ed, w in draws(6):
        f = float(rng.uniform(1.0, 4.0))
        net = im.Network(w, float(10 ** rng.uniform(8, 10.5)))
        s1 = im.speedup(compute, dense, comp, net, t_ed)
        sf = im.speedup(compute.faster(f), dense, comp, net, t_ed)
        if s1 >= 1.0:
            assert sf >= s1 * (1 - 1e-12), (compute, dense, comp, t_ed, w, f, s1, sf)
        b1 = im.break_even_bandwidth(compute, dense, comp, t_ed, w)
        bf = im.break_even_bandwidth(compute.faster(f), dense, comp, t_ed, w)
        assert bf >= b1 * (1 - 1e-12)
    # a case that gains nothing at 1x and 1.75x at 4x: a 100 MB gradient, 32
    # workers on 20 Gbit/s links, 40 + 120 ms of compute, t_ed = 10 ms
    compute = im.Compute(0.04, 0.12)
    dense, comp = im.Payload((100_000_000,)), im.Payload((500_000, 500_000))
    net = im.Network(32, 20 * GBIT)
    assert im.speedup(compute, dense, comp, net, 0.01) == pytest.approx(0.16 / 0.17, rel=1e-9)
    assert im.speedup(compute.faster(4), dense, comp, net, 0.01) == pytest.approx(1.75, rel=1e-9)


def test_encode_time_matters_more_than_compression_ratio():
    """Finding 5: when the compressed step is bound by GPU work (t_bwd + t_ed
    covers the compressed exchange), its time does not depend on the payload,
    and every second cut from t_ed comes off the step; halving t_ed at half
    the compression ratio beats the original around its break-even point."""
    rng = np.random.default_rng(7)
    seen = 0
    for compute, dense, comp, t_ed, w in draws(8):
        net = im.Network(w, float(10 ** rng.uniform(9, 10.5)))
        if compute.t_bwd + t_ed < im.comm_seconds(comp, net):
            continue
        seen += 1
        t = im.step_seconds(compute, comp, net, t_ed)
        smaller = im.Payload(tuple(s // 2 for s in comp.allreduce_bytes))
        assert im.step_seconds(compute, smaller, net, t_ed) == t
        assert im.step_seconds(compute, comp, net, 0.9 * t_ed) == pytest.approx(t - 0.1 * t_ed, rel=1e-12)
    assert seen > 50
    # rank 4 with t_ed against rank 8 (half the ratio) with t_ed / 2
    compute = im.Compute(0.03, 0.09)
    dense = im.Payload((170_000_000,))
    r4, r8 = im.Payload((400_000, 400_000)), im.Payload((800_000, 800_000))
    t_ed = 0.05
    for w in (8, 32, 64):
        b4 = im.break_even_bandwidth(compute, dense, r4, t_ed, w)
        b8 = im.break_even_bandwidth(compute, dense, r8, t_ed / 2, w)
        assert b8 > b4
        for b in (b4 / 2, b4, 2 * b4):
            net = im.Network(w, b)
            assert im.step_seconds(compute, r8, net, t_ed / 2) < im.step_seconds(compute, r4, net, t_ed)
