"""Pins for the PowerSGD error-feedback oracle (CPU only).

Independent facts the oracle must reproduce:
  * full rank (r = min(n, m)) reconstructs M exactly and leaves no residual;
  * Eckart-Young: the rank-r error is never below the truncated-SVD error
    (numpy.linalg.svd);
  * the subspace-iteration limit: warm-started steps on a fixed M with a known
    spectrum converge to the truncated-SVD error;
  * out is the orthogonal projection of M onto range(M Q_in), computed here
    with numpy.linalg.pinv, and P^ is numpy.linalg.qr's Q factor of M Q_in
    (signs fixed to a positive R diagonal);
  * P^ has orthonormal columns and the residual is orthogonal to them; the
    memory invariant m' + out = M.
"""
import numpy as np
import pytest

import gen
import oracle


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def qr_positive(A):
    Qf, R = np.linalg.qr(A)
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Qf * s


@pytest.mark.parametrize("n,m,r", [(1000, 3, 3), (4, 4608, 4), (7, 2, 2), (64, 1, 1), (2, 9, 2)])
def test_full_rank_is_exact(n, m, r):
    g = gen.gaussian_mat(n, m, 11)
    mem = gen.gaussian_mat(n, m, 12, 0.3)
    q = gen.gaussian_mat(m, 4, 13)
    res = oracle.powersgd_ef_step(g, mem, q, 0.7, r)
    assert rel(res["out"], res["M"]) < 1e-12
    assert np.linalg.norm(res["mem"]) <= 1e-12 * np.linalg.norm(res["M"])


@pytest.mark.parametrize("n,m,r", [(64, 27, 1), (64, 27, 4), (128, 576, 2), (100, 512, 4), (300, 40, 3)])
def test_eckart_young_and_projection(n, m, r):
    g = gen.gaussian_mat(n, m, 21 + r)
    mem = gen.gaussian_mat(n, m, 22 + r, 0.5)
    q = gen.gaussian_mat(m, 4, 23 + r)
    res = oracle.powersgd_ef_step(g, mem, q, 1.0, r)
    M = res["M"]
    s = np.linalg.svd(M, compute_uv=False)
    ey = np.sqrt(np.sum(s[r:] ** 2))
    assert np.linalg.norm(M - res["out"]) >= ey * (1 - 1e-12)
    # out = projection of M onto range(M Q_in)
    B = M @ q[:, :r].astype(np.float64)
    proj = B @ np.linalg.pinv(B) @ M
    assert rel(res["out"], proj) < 1e-10
    # P^ = Q factor of M Q_in, Q = M^T P^
    Ph = qr_positive(B)
    assert rel(res["P"], Ph) < 1e-10
    assert rel(res["Q"], M.T @ Ph) < 1e-10
    # orthonormal columns, residual orthogonal to them, memory invariant
    assert np.abs(res["P"].T @ res["P"] - np.eye(r)).max() < 1e-12
    assert np.abs(res["P"].T @ res["mem"]).max() < 1e-10 * np.linalg.norm(M)
    assert rel(res["mem"] + res["out"], M) < 1e-15


def test_rank1_closed_form():
    g = gen.gaussian_mat(50, 30, 31)
    mem = np.zeros((50, 30), np.float32)
    q = gen.gaussian_mat(30, 4, 32)
    res = oracle.powersgd_ef_step(g, mem, q, 2.0, 1)
    M = 2.0 * g.astype(np.float64)
    p = M @ q[:, 0].astype(np.float64)
    p /= np.linalg.norm(p)
    assert rel(res["out"], np.outer(p, p) @ M) < 1e-13


def test_subspace_iteration_limit():
    n, m, r = 512, 256, 2
    R = gen.rng(0, gen.KIND_MISC, 40)
    U = qr_positive(R.standard_normal((n, m)))
    V = qr_positive(R.standard_normal((m, m)))
    sig = np.geomspace(10.0, 0.01, m)
    sig[:4] = [10.0, 6.0, 2.0, 1.5]
    M = (U * sig) @ V.T
    Mf = M.astype(np.float32)
    q = R.standard_normal((m, r)).astype(np.float32)
    zero = np.zeros((n, m), np.float32)
    for _ in range(30):
        res = oracle.powersgd_ef_step(Mf, zero, q, 1.0, r)
        q = res["Q"].astype(np.float32)
    s = np.linalg.svd(Mf.astype(np.float64), compute_uv=False)
    ey = np.sqrt(np.sum(s[r:] ** 2))
    err = np.linalg.norm(Mf.astype(np.float64) - res["out"])
    assert ey <= err <= ey * 1.001


def test_zero_column_and_bf16():
    g = gen.gaussian_mat(20, 10, 51)
    q = gen.gaussian_mat(10, 4, 52)
    q[:, 1] = 0.0
    res = oracle.powersgd_ef_step(g, np.zeros_like(g), q, 1.0, 3)
    assert np.all(res["P"][:, 1] == 0.0)
    assert np.abs(res["P"][:, [0, 2]].T @ res["P"][:, [0, 2]] - np.eye(2)).max() < 1e-12
    # bf16 bit patterns give the same result as the float32 values they encode
    gb = gen.f32_to_bf16_bits(g)
    r1 = oracle.powersgd_ef_step(gb, np.zeros_like(g), q, 1.0, 2)
    r2 = oracle.powersgd_ef_step(gen.bf16_bits_as_f32(gb), np.zeros_like(g), q, 1.0, 2)
    assert np.array_equal(r1["out"], r2["out"])


def test_mgs_matches_qr():
    A = gen.gaussian_mat(200, 4, 61).astype(np.float64)
    assert rel(oracle.orthonormalize_mgs(A), qr_positive(A)) < 1e-12


@pytest.mark.parametrize("mutation", ["transpose_q", "no_orthonormalise", "residual_sign", "classical_no_norm"])
def test_pins_reject_mutations(mutation):
    n, m, r = 64, 27, 3
    g = gen.gaussian_mat(n, m, 71)
    mem = gen.gaussian_mat(n, m, 72, 0.5)
    q = gen.gaussian_mat(m, 4, 73)
    M = mem.astype(np.float64) + g.astype(np.float64)
    P = M @ q[:, :r].astype(np.float64)
    if mutation == "no_orthonormalise":
        Ph = P
    elif mutation == "classical_no_norm":
        Ph = P / np.linalg.norm(P, axis=0)
    else:
        Ph = oracle.orthonormalize_mgs(P)
    Q = (M.T @ Ph) if mutation != "transpose_q" else (M.T @ Ph)[::-1]
    out = Ph @ Q.T
    m_new = M - out if mutation != "residual_sign" else M + out
    B = M @ q[:, :r].astype(np.float64)
    proj = B @ np.linalg.pinv(B) @ M
    ok = (rel(out, proj) < 1e-10 and np.abs(Ph.T @ Ph - np.eye(r)).max() < 1e-12
          and rel(m_new + out, M) < 1e-15)
    assert not ok
