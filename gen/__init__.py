"""Seeded synthetic inputs for the gradient-compressor hot path.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds shapes, seeds and random draws only -- none of the
compression arithmetic -- so the oracle (``oracle/``) and the HIP path
(``gradient_compression_error_amd``) never share code through it.

Every stream is ``numpy.random.Generator(PCG64(SeedSequence([SEED, config,
kind, step, layer])))``.  Floating-point draws are made in float32 directly
(``standard_normal(dtype=float32)``) except Student-t, which numpy draws in
float64 and which is then rounded to float32 (round-to-nearest-even).  bf16
gradients are produced from those float32 values by round-to-nearest-even on
the bit pattern and are carried as ``uint16`` arrays.

The workloads stand in for the gradient sets of the pages' experiments:
ResNet-18 / VGG-19 on CIFAR-100 (Accordion paper, results section), ResNet-50
and BERT (utility-of-compression paper, method section) and a plain Gaussian
vector for the Mem-SGD analysis (Sparsified SGD with Memory, method section).
No dataset or trained weight is involved: only the tensor shapes and a value
distribution per tensor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SEED = 0

# kinds of random stream
KIND_GRAD = 0
KIND_SCALE = 1
KIND_QINIT = 2
KIND_MISC = 3

# config ids (stable integers used in the seed)
CFG_C1 = 1
CFG_C2 = 2
CFG_C3 = 3
CFG_C4 = 4
CFG_C5 = 5
CFG_ACC_TOPK = 6    # Accordion on top-k (the C3 vector with a norm trajectory)


def rng(config: int, kind: int, step: int = 0, layer: int = 0) -> np.random.Generator:
    """Independent, reproducible stream for (config, kind, step, layer)."""
    ss = np.random.SeedSequence([SEED, int(config), int(kind), int(step), int(layer)])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Inputs here are finite, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_as_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening); used to upload/inspect inputs."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------

def _expand(spec):
    out = []
    for count, n, m in spec:
        out += [(n, m)] * count
    return out


# ResNet-18 (CIFAR, 100 classes): conv weights as out x (in*kh*kw), fc 100x512.
RESNET18_MATS = _expand([
    (1, 64, 27), (4, 64, 576), (1, 128, 576), (3, 128, 1152), (1, 128, 64),
    (1, 256, 1152), (3, 256, 2304), (1, 256, 128), (1, 512, 2304),
    (3, 512, 4608), (1, 512, 256), (1, 100, 512),
])
# BN weight+bias for every BN layer (4800 channels x 2) plus the fc bias (100):
# passed uncompressed.  BN layers of the CIFAR ResNet-18: the stem (64), four in
# stage 1 (64), five in each later stage (two per block plus the shortcut's):
# 128, 256, 512 channels.  Each BN layer has a scale and a shift vector.
RESNET18_BN_CHANNELS = [64] * 5 + [128] * 5 + [256] * 5 + [512] * 5
RESNET18_VECTORS = [c for c in RESNET18_BN_CHANNELS for _ in range(2)] + [100]
RESNET18_VECTOR_ELEMS = 9700
assert sum(RESNET18_VECTORS) == RESNET18_VECTOR_ELEMS

# VGG-19 (CIFAR-100): 16 conv 3x3 layers, fc 512x512, 512x512, 100x512.
VGG19_MATS = _expand([
    (1, 64, 27), (1, 64, 576), (1, 128, 576), (1, 128, 1152), (1, 256, 1152),
    (3, 256, 2304), (1, 512, 2304), (7, 512, 4608), (2, 512, 512), (1, 100, 512),
])

# BERT-large: 24 layers x (4 x 1024x1024 attention, 1024x4096, 4096x1024).
BERT_LAYER_MATS = [(1024, 1024)] * 4 + [(1024, 4096), (4096, 1024)]
BERT_MATS = BERT_LAYER_MATS * 24
BERT_EMB = (30522, 1024)

C1_D, C1_K, C1_ETA, C1_STEPS = 10_000, 100, 0.1, 10
C3_D = 25_600_000
C3_KS = (25_600, 256_000)          # floor(0.001*d), floor(0.01*d)
C5_EMB_K = 312_545                 # floor(0.01 * 30522*1024)
C4_CHECK_EVERY = 10
C4_THRESHOLD = 0.5
C4_STEPS = 300
C4_RANK_LOW_COMPRESSION = 4        # level l_low (critical regime)
C4_RANK_HIGH_COMPRESSION = 2       # level l_high


def numel(shapes) -> int:
    return int(sum(n * m for n, m in shapes))


# --------------------------------------------------------------------------
# C1: Mem-SGD top-k tiny
# --------------------------------------------------------------------------

def c1_grad(step: int) -> np.ndarray:
    return rng(CFG_C1, KIND_GRAD, step).standard_normal(C1_D, dtype=np.float32)


# --------------------------------------------------------------------------
# C2: ResNet-18 gradient set
# --------------------------------------------------------------------------

def layer_sigmas(config: int, nlayers: int) -> np.ndarray:
    """Per-layer scale 10**U(-4,-2), fixed for the whole run (float64)."""
    u = rng(config, KIND_SCALE).uniform(-4.0, -2.0, size=nlayers)
    return np.power(10.0, u)


def gaussian_matrix(config: int, step: int, layer: int, n: int, m: int, sigma: float) -> np.ndarray:
    z = rng(config, KIND_GRAD, step, layer).standard_normal((n, m), dtype=np.float32)
    return (z * np.float32(sigma)).astype(np.float32)


def c2_grads(step: int) -> list[np.ndarray]:
    sig = layer_sigmas(CFG_C2, len(RESNET18_MATS))
    return [gaussian_matrix(CFG_C2, step, l, n, m, sig[l]) for l, (n, m) in enumerate(RESNET18_MATS)]


def c2_vectors(step: int) -> list[np.ndarray]:
    """The ResNet-18 BN/bias gradients of one step: N(0, s_v^2) per vector,
    s_v = 10**U(-4,-2) fixed per vector (a stream of its own, so the matrix
    draws above are unchanged)."""
    sig = rng(CFG_C2, KIND_SCALE, 1).uniform(-4.0, -2.0, size=len(RESNET18_VECTORS))
    out = []
    for v, n in enumerate(RESNET18_VECTORS):
        z = rng(CFG_C2, KIND_GRAD, step, 1000 + v).standard_normal(n, dtype=np.float32)
        out.append((z * np.float32(10.0 ** sig[v])).astype(np.float32))
    return out


def q_init(config: int, layer: int, m: int, cols: int = 4) -> np.ndarray:
    """Initial Q ~ N(0,1), m x cols stored column-major (array shape (cols, m))."""
    return rng(config, KIND_QINIT, 0, layer).standard_normal((cols, m), dtype=np.float32)


def q_refill(config: int, layer: int, step: int, m: int, cols: int) -> np.ndarray:
    """Fresh N(0,1) columns used when a rank switch grows Q (shape (cols, m))."""
    return rng(config, KIND_QINIT, step + 1, layer).standard_normal((cols, m), dtype=np.float32)


# --------------------------------------------------------------------------
# C3: ResNet-50-sized flat heavy-tailed gradient
# --------------------------------------------------------------------------

def c3_grad(step: int, d: int = C3_D) -> np.ndarray:
    t = rng(CFG_C3, KIND_GRAD, step).standard_t(3.0, size=d)
    return (t * 1e-3).astype(np.float32)


# --------------------------------------------------------------------------
# C4: VGG-19 with a synthetic norm trajectory
# --------------------------------------------------------------------------

def c4_scale(t: int) -> float:
    """Trajectory factor exp(-t/200) * J(t); J = 4 on [105, 205), else 1."""
    j = 4.0 if 105 <= t < 205 else 1.0
    return math.exp(-t / 200.0) * j


def c4_grads(step: int) -> list[np.ndarray]:
    sig0 = layer_sigmas(CFG_C4, len(VGG19_MATS))
    f = c4_scale(step)
    return [gaussian_matrix(CFG_C4, step, l, n, m, sig0[l] * f) for l, (n, m) in enumerate(VGG19_MATS)]


# --------------------------------------------------------------------------
# Accordion on top-k: the C3 vector shape with a norm trajectory
# --------------------------------------------------------------------------

ACC_TOPK_JUMP = (15, 25)           # scale x4 on [15, 25): one up jump, one down jump
ACC_TOPK_FRACTIONS = (0.01, 0.001)  # k / d at l_low (critical: low compression) and l_high


def acc_topk_scale(t: int) -> float:
    """Trajectory factor exp(-t/200) * J(t); J = 4 on [15, 25), else 1."""
    j = 4.0 if ACC_TOPK_JUMP[0] <= t < ACC_TOPK_JUMP[1] else 1.0
    return math.exp(-t / 200.0) * j


def acc_topk_ks(d: int) -> tuple[int, int]:
    """(k at l_low, k at l_high) = floor(fraction * d), at least 1."""
    return tuple(max(1, int(math.floor(f * d))) for f in ACC_TOPK_FRACTIONS)


def acc_topk_base(step: int, d: int) -> np.ndarray:
    """Unscaled draw of step `step`: 1e-3 * Student-t(3), float32."""
    t = rng(CFG_ACC_TOPK, KIND_GRAD, step).standard_t(3.0, size=d)
    return (t * 1e-3).astype(np.float32)


def acc_topk_grad(step: int, d: int) -> np.ndarray:
    return (acc_topk_base(step, d) * np.float32(acc_topk_scale(step))).astype(np.float32)


# --------------------------------------------------------------------------
# C5: BERT-large bf16 gradient set
# --------------------------------------------------------------------------

def c5_matrix_bf16(set_id: int, layer: int) -> np.ndarray:
    n, m = BERT_MATS[layer]
    z = rng(CFG_C5, KIND_GRAD, set_id, layer).standard_normal((n, m), dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(1e-3))


def c5_embedding_bf16(set_id: int) -> np.ndarray:
    n, m = BERT_EMB
    z = rng(CFG_C5, KIND_GRAD, set_id, 10_000).standard_normal(n * m, dtype=np.float32)
    return f32_to_bf16_bits(z * np.float32(1e-3))


# --------------------------------------------------------------------------
# Small structured inputs for edge cases
# --------------------------------------------------------------------------

def randk_indices(config: int, step: int, d: int, k: int) -> np.ndarray:
    """The rand-k draw of one step: k distinct coordinates of [0, d), uniform,
    sorted ascending (int32)."""
    r = rng(config, KIND_MISC, step, 777)
    return np.sort(r.choice(d, size=k, replace=False)).astype(np.int32)


def tie_heavy(d: int, seed_layer: int, levels: int = 6) -> np.ndarray:
    """Values in {+-0.25*j : j = 0..levels-1}: many exact magnitude ties."""
    r = rng(0, KIND_MISC, 0, seed_layer)
    j = r.integers(0, levels, size=d)
    s = r.choice(np.array([-1.0, 1.0]), size=d)
    return (s * 0.25 * j).astype(np.float32)


def gaussian_vector(d: int, seed_layer: int, scale: float = 1.0) -> np.ndarray:
    return (rng(0, KIND_MISC, 1, seed_layer).standard_normal(d, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def gaussian_mat(n: int, m: int, seed_layer: int, scale: float = 1.0) -> np.ndarray:
    return (rng(0, KIND_MISC, 2, seed_layer).standard_normal((n, m), dtype=np.float32) * np.float32(scale)).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    description: str


WORKLOADS = {
    "c1": Workload("c1", "Mem-SGD top-k tiny: fp32 d=10,000, k=100, eta=0.1, 10 steps"),
    "c2": Workload("c2", "ResNet-18 (CIFAR-100) gradient set, 21 matrices PowerSGD EF rank 1/2 + 41 BN/bias vectors (9,700 entries) uncompressed"),
    "c3": Workload("c3", "ResNet-50-sized flat fp32 gradient d=25.6M, Student-t(3)*1e-3, top-k EF k=0.1%/1%"),
    "c3randk": Workload("c3randk", "ResNet-50-sized flat fp32 gradient d=25.6M, Student-t(3)*1e-3, rand-k EF k=1% (seeded subsets)"),
    "c4": Workload("c4", "VGG-19 (CIFAR-100) gradient set, Accordion PowerSGD rank 4/2, checks every 10 steps"),
    "c3acc": Workload("c3acc", "ResNet-50-sized flat fp32 gradient d=25.6M with a norm trajectory, Accordion top-k EF: k=1% (l_low) / 0.1% (l_high), checks every 10 steps"),
    "c5": Workload("c5", "BERT-large gradient set: 144 matrices PowerSGD EF rank 4 + 30522x1024 embedding top-k 1% EF, bf16 grads, fp32 memory"),
}
