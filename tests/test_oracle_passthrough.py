"""Pins for the oracle of the uncompressed vectors (CPU only).

out = fl32(eta * grad), the memory untouched.  Facts fixed independently of
the oracle's float64 route:
  * eta = 1 leaves every value as it is, bit for bit (float32 and bf16 inputs);
  * a power-of-two eta scales exactly: the result is numpy.ldexp of the input
    while it stays in the normal range;
  * numpy's float32 multiply is IEEE-754 correctly rounded, so it must give
    the same bits for any eta (a second route to the same rounding);
  * an eta taken in float64 instead of float32, or a product rounded twice
    through bf16, is caught by the pins.
The sizes are those of the ResNet-18 BN/bias set (41 vectors, 9,700 entries).
"""
import numpy as np

import gen
import oracle


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_resnet18_vector_shapes():
    # every BN layer of the CIFAR ResNet-18 has a scale and a shift vector, plus the fc bias
    assert len(gen.RESNET18_VECTORS) == 41
    assert sum(gen.RESNET18_VECTORS) == gen.RESNET18_VECTOR_ELEMS == 9700
    # the channel counts match the matrices: one BN per convolution (stem, 16 block convs, 3 shortcuts)
    convs = [n for n, m in gen.RESNET18_MATS if m != 512 or n != 100]
    assert sorted(gen.RESNET18_BN_CHANNELS) == sorted(convs)
    vecs = gen.c2_vectors(0)
    assert [v.size for v in vecs] == gen.RESNET18_VECTORS
    assert all(v.dtype == np.float32 for v in vecs)


def test_eta_one_is_identity():
    for v in gen.c2_vectors(1):
        assert np.array_equal(bits(oracle.passthrough_step(v, 1.0)), bits(v))
    b = gen.f32_to_bf16_bits(gen.gaussian_vector(5000, 3, 1e-3))
    assert np.array_equal(bits(oracle.passthrough_step(b, 1.0)), bits(gen.bf16_bits_as_f32(b)))


def test_power_of_two_is_exact():
    v = gen.gaussian_vector(10_000, 4, 1e-2)
    for e in (-3, -1, 1, 2):
        assert np.array_equal(bits(oracle.passthrough_step(v, 2.0 ** e)), bits(np.ldexp(v, e)))


def test_matches_float32_multiply():
    vecs = gen.c2_vectors(2) + [gen.gaussian_vector(70_001, 5, 3.0)]
    for eta in (0.1, 0.8, 1.0 / 3.0, 7.25):
        e32 = np.float32(eta)
        for v in vecs:
            want = (e32 * v).astype(np.float32)
            assert np.array_equal(bits(oracle.passthrough_step(v, eta)), bits(want))


def test_planted_mistakes_fail():
    v = gen.gaussian_vector(100_000, 6, 1.0)
    want = (np.float32(0.1) * v).astype(np.float32)
    # eta used as float64 0.1 rather than its float32 value
    wrong_eta = (0.1 * v.astype(np.float64)).astype(np.float32)
    assert not np.array_equal(bits(wrong_eta), bits(want))
    # product rounded through bf16 first
    wrong_round = gen.bf16_bits_as_f32(gen.f32_to_bf16_bits(want))
    assert not np.array_equal(bits(wrong_round), bits(want))
    assert np.array_equal(bits(oracle.passthrough_step(v, 0.1)), bits(want))
