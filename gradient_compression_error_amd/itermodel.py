"""Iteration-time model of one data-parallel step with gradient compression.

"On the Utility of Gradient Compression in Distributed Training Systems"
(method section) predicts whether a compressor speeds up training with an
analytic model of three measured parts of a step: computation, communication
and encode-decode time.  In that model communication is overlapped with the
backward pass (DDP communication hooks), and collectives are NCCL ring
collectives.  The results section reads a break-even network bandwidth off the
model, and simulates faster computation and faster encode-decode.  The pages do
not print the formula.  This module takes the plainest one that fits that
description:

* The GPU runs forward, backward and encode-decode one after the other.
* The network runs at the same time as the backward pass and the encode-decode
  work.  The step ends when both are done::

      T_sync = t_fwd + max(t_bwd,        t_comm(dense gradient))
      T_comp = t_fwd + max(t_bwd + t_ed, t_comm(compressed payload))

* Collectives are ring collectives with the alpha-beta cost.  W is the number
  of workers, B the bandwidth of each worker's link (bytes/s, one direction)
  and alpha the latency of one message step:

      all-reduce of S bytes:              2 (W-1) alpha + 2 (W-1)/W * S / B
      all-gather of S bytes per worker:     (W-1) alpha +   (W-1)   * S / B

PowerSGD is all-reduce compatible (utility page, results section).  It
all-reduces P and then Q' (two calls per step).  Top-k index sets differ per
worker, so the (index, value) pairs are all-gathered.  Uncompressed tensors
(biases, norms) stay in a dense all-reduce.

The pages print neither the formula nor a worked example with its inputs, so
no number of theirs can be reproduced.  The tests pin the collective costs
against a step-by-step ring simulation and the break-even bandwidth against a
scan of the step times; they also check, as properties over random draws, the
five findings of the results section: a fixed encode-decode cost loses above
some bandwidth; an encode-decode time beyond the hiding window removes any
speed-up; all-gathered payloads stop paying as workers grow while all-reduced
ones do not; faster compute raises the gain (a 1.75x case at 4x compute); and
a shorter encode-decode time beats a higher compression ratio.

Host code only: it makes no GPU call.
"""
from __future__ import annotations

import argparse
import json
import math
from dataclasses import dataclass, field
from typing import Iterable, Optional, Sequence, Tuple


@dataclass(frozen=True)
class Network:
    workers: int
    bandwidth: float          # bytes/s of each worker's link, one direction
    latency: float = 0.0      # seconds per message step


@dataclass(frozen=True)
class Compute:
    t_fwd: float              # seconds
    t_bwd: float              # seconds; the window communication can hide in

    def faster(self, factor: float) -> "Compute":
        """Computation `factor` times faster (the pages' compute speed-up study)."""
        return Compute(self.t_fwd / factor, self.t_bwd / factor)


@dataclass(frozen=True)
class Payload:
    """What one worker sends in one step."""
    allreduce_bytes: Tuple[int, ...] = ()   # one entry per all-reduce call
    allgather_bytes: int = 0                 # bytes each worker contributes to one all-gather

    def __add__(self, other: "Payload") -> "Payload":
        ag = self.allgather_bytes + other.allgather_bytes
        return Payload(self.allreduce_bytes + other.allreduce_bytes, ag)


def ring_allreduce_seconds(nbytes: float, net: Network) -> float:
    w = net.workers
    if w <= 1 or nbytes <= 0:
        return 0.0
    return 2 * (w - 1) * net.latency + 2.0 * (w - 1) / w * nbytes / net.bandwidth


def ring_allgather_seconds(nbytes_per_worker: float, net: Network) -> float:
    w = net.workers
    if w <= 1 or nbytes_per_worker <= 0:
        return 0.0
    return (w - 1) * net.latency + (w - 1) * nbytes_per_worker / net.bandwidth


def comm_cost(payload: Payload, workers: int) -> Tuple[float, float]:
    """(a, b) with communication seconds = a * alpha + b / B for W = workers."""
    w = workers
    if w <= 1:
        return 0.0, 0.0
    ar = [s for s in payload.allreduce_bytes if s > 0]
    a = 2.0 * (w - 1) * len(ar) + ((w - 1) if payload.allgather_bytes > 0 else 0)
    b = 2.0 * (w - 1) / w * sum(ar) + (w - 1) * payload.allgather_bytes
    return float(a), float(b)


def comm_seconds(payload: Payload, net: Network) -> float:
    t = sum(ring_allreduce_seconds(s, net) for s in payload.allreduce_bytes)
    return t + ring_allgather_seconds(payload.allgather_bytes, net)


def step_seconds(compute: Compute, payload: Payload, net: Network, t_encdec: float = 0.0) -> float:
    return compute.t_fwd + max(compute.t_bwd + t_encdec, comm_seconds(payload, net))


def speedup(compute: Compute, dense: Payload, compressed: Payload, net: Network, t_encdec: float) -> float:
    """Synchronous-SGD step time over the compressed step time (> 1: compression pays)."""
    return step_seconds(compute, dense, net) / step_seconds(compute, compressed, net, t_encdec)


def _above(coef: float, rhs: float) -> Tuple[float, float]:
    """The bandwidths B > 0 with coef / B > rhs, as an open interval (lo, hi)."""
    if coef > 0:
        return (0.0, coef / rhs) if rhs > 0 else (0.0, math.inf)
    if coef == 0:
        return (0.0, math.inf) if rhs < 0 else (0.0, 0.0)
    return (coef / rhs, math.inf) if rhs < 0 else (0.0, 0.0)


def pays_interval(compute: Compute, dense: Payload, compressed: Payload, t_encdec: float,
                  workers: int, latency: float = 0.0) -> Tuple[float, float]:
    """Open interval (lo, hi) of link bandwidths B (bytes/s) at which the
    compressed step is faster than the synchronous one; (0, 0) if none.

    With t_comm = a_s alpha + b_s / B (dense) and a_c alpha + b_c / B
    (compressed), the compressed step is faster exactly when both
      (1) a_s alpha + b_s / B > t_bwd + t_ed   (the dense exchange outlasts the
          GPU work of the compressed step), and
      (2) a_c alpha + b_c / B < a_s alpha + b_s / B.
    """
    a_s, b_s = comm_cost(dense, workers)
    a_c, b_c = comm_cost(compressed, workers)
    lat_s, lat_c = a_s * latency, a_c * latency
    lo1, hi1 = _above(b_s, compute.t_bwd + t_encdec - lat_s)
    lo2, hi2 = _above(b_s - b_c, lat_c - lat_s)
    lo, hi = max(lo1, lo2), min(hi1, hi2)
    return (lo, hi) if lo < hi else (0.0, 0.0)


def break_even_bandwidth(compute: Compute, dense: Payload, compressed: Payload, t_encdec: float,
                         workers: int, latency: float = 0.0) -> float:
    """B* (bytes/s) with: compressed step faster  <=>  B < B*.  0.0 when
    compression never pays, math.inf when it always does.  Raises ValueError
    when the compressed step wins only above some bandwidth (a larger payload
    sent in fewer messages), which has no single break-even point of this form.
    """
    lo, hi = pays_interval(compute, dense, compressed, t_encdec, workers, latency)
    if lo > 0:
        raise ValueError(f"compression pays only for {lo:.4g} < B < {hi:.4g} bytes/s")
    return hi


# ----------------------------------------------------------------------------- payloads

def dense_payload(nelem: int, bytes_per_elem: int) -> Payload:
    return Payload((int(nelem) * bytes_per_elem,))


def powersgd_payload(shapes: Sequence[Tuple[int, int]], ranks: Sequence[int] | int,
                     bytes_per_elem: int = 4) -> Payload:
    """P (n x r) in one all-reduce, then Q' (m x r) in a second one."""
    if isinstance(ranks, int):
        ranks = [ranks] * len(shapes)
    p = sum(n * r for (n, _), r in zip(shapes, ranks)) * bytes_per_elem
    q = sum(m * r for (_, m), r in zip(shapes, ranks)) * bytes_per_elem
    return Payload((int(p), int(q)))


def topk_payload(k: int, bytes_per_pair: int = 8) -> Payload:
    """k (int32 index, float32 value) pairs, all-gathered."""
    return Payload((), int(k) * bytes_per_pair)


# ----------------------------------------------------------------------------- gradient sets

def _expand(spec):
    out = []
    for count, n, m in spec:
        out += [(n, m)] * count
    return out


@dataclass(frozen=True)
class GradientSet:
    """A model's gradient as the compressor sees it (architecture shapes only)."""
    name: str
    matrices: Tuple[Tuple[int, int], ...]          # compressed with PowerSGD
    topk: Tuple[Tuple[int, int], ...] = ()          # (elements, k) compressed with top-k
    dense_elems: int = 0                            # sent uncompressed
    grad_bytes: int = 4                             # bytes per gradient entry in the dense exchange
    ranks: Tuple[int, ...] = field(default=())

    def nelem(self) -> int:
        return sum(n * m for n, m in self.matrices) + sum(d for d, _ in self.topk) + self.dense_elems

    def dense(self) -> Payload:
        return dense_payload(self.nelem(), self.grad_bytes)

    def compressed(self, rank: Optional[int] = None) -> Payload:
        ranks = [rank] * len(self.matrices) if rank is not None else list(self.ranks)
        pay = powersgd_payload(self.matrices, ranks) if self.matrices else Payload()
        for _, k in self.topk:
            pay = pay + topk_payload(k)
        if self.dense_elems:
            pay = pay + dense_payload(self.dense_elems, self.grad_bytes)
        return pay


_BERT_LAYER = [(1024, 1024)] * 4 + [(1024, 4096), (4096, 1024)]
GRADIENT_SETS = {
    # BERT-large: 24 encoder layers of PowerSGD matrices; the 30522 x 1024
    # embedding by top-k 1%; bf16 gradients
    "bert-large": GradientSet("bert-large", tuple(_BERT_LAYER * 24), topk=((30522 * 1024, 312_545),),
                              grad_bytes=2, ranks=(4,) * 144),
    # ResNet-18 (CIFAR-100) conv/fc weights as out x (in kh kw); BN and fc bias dense
    "resnet18": GradientSet("resnet18", tuple(_expand([
        (1, 64, 27), (4, 64, 576), (1, 128, 576), (3, 128, 1152), (1, 128, 64),
        (1, 256, 1152), (3, 256, 2304), (1, 256, 128), (1, 512, 2304),
        (3, 512, 4608), (1, 512, 256), (1, 100, 512)])), dense_elems=9700, ranks=(2,) * 21),
    # VGG-19 (CIFAR-100)
    "vgg19": GradientSet("vgg19", tuple(_expand([
        (1, 64, 27), (1, 64, 576), (1, 128, 576), (1, 128, 1152), (1, 256, 1152),
        (3, 256, 2304), (1, 512, 2304), (7, 512, 4608), (2, 512, 512), (1, 100, 512)])),
        ranks=(4,) * 19),
    # a flat 25.6M-entry gradient, top-k 1%
    "flat-25.6m": GradientSet("flat-25.6m", (), topk=((25_600_000, 256_000),)),
}


# ----------------------------------------------------------------------------- report

def break_even_table(gset: GradientSet, t_encdec: float, workers: Iterable[int], bwd_windows: Iterable[float],
                     latency: float, compute_speedups: Iterable[float] = (1.0,)) -> list:
    """Rows of break-even bandwidths (Gbit/s) for each (workers, backward window, compute speed-up)."""
    rows = []
    dense, comp = gset.dense(), gset.compressed()
    for w in workers:
        for tb in bwd_windows:
            for f in compute_speedups:
                c = Compute(0.0, tb).faster(f)
                b = break_even_bandwidth(c, dense, comp, t_encdec, w, latency)
                rows.append({"set": gset.name, "workers": w, "t_bwd_ms": tb * 1e3, "compute_x": f,
                             "t_encdec_ms": t_encdec * 1e3,
                             "break_even_gbit_s": (b * 8 / 1e9) if math.isfinite(b) else b})
    return rows


def main(argv: Optional[Sequence[str]] = None) -> int:
    ap = argparse.ArgumentParser(description="break-even link bandwidth of gradient compression "
                                             "(iteration-time model; host only)")
    ap.add_argument("--set", choices=sorted(GRADIENT_SETS), default="bert-large")
    ap.add_argument("--encdec-us", type=float, required=True,
                    help="measured encode+decode time of one step, microseconds")
    ap.add_argument("--workers", default="8,64")
    ap.add_argument("--bwd-ms", default="0,10,50,200", help="backward windows, milliseconds")
    ap.add_argument("--compute-x", default="1", help="compute speed-up factors")
    ap.add_argument("--latency-us", type=float, default=5.0, help="latency of one ring message step")
    a = ap.parse_args(argv)
    rows = break_even_table(GRADIENT_SETS[a.set], a.encdec_us * 1e-6,
                            [int(x) for x in a.workers.split(",")],
                            [float(x) * 1e-3 for x in a.bwd_ms.split(",")], a.latency_us * 1e-6,
                            [float(x) for x in a.compute_x.split(",")])
    for r in rows:
        print(json.dumps(r))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
