"""Pins of the oracle's basis calibration against facts that do not come from it.

* An exactly constructed SVD ``A = U diag(sigma) V^T`` (AQUA page, appendix on
  the SVD: the columns of ``V`` are the principal directions) -- catches left
  instead of right singular vectors, a transposed ``V``, ascending order,
  centring, squared vs plain singular values;
* the eigen-equation of ``A^T A`` on unstructured keys, orthonormality and
  decreasing order (the same appendix: ``V`` also comes from ``A^T A``);
* a rank-one key matrix along a coordinate axis, and identical key rows (the
  uncentred reading: centring would give nothing);
* scaling the keys scales the eigenvalues by the square and leaves ``P``;
* per-head independence and the batch elements' rows taken together;
* the sign convention (largest-magnitude entry positive);
* keys drawn from a known spectrum in a known basis give back that basis and
  the closed-form energy share of the leading directions (statistically).
"""

import numpy as np
import pytest

import oracle
from loki_inputs import make_basis


def _orthonormal_columns(n, d, seed):
    a = np.random.default_rng(seed).standard_normal((n, d))
    qm, _ = np.linalg.qr(a)
    return qm


def _as_cache(A, B=1):
    """Rows of A split evenly over B batch elements of one key/value head."""
    n, d = A.shape
    return A.reshape(B, n // B, d)[:, None]


@pytest.mark.parametrize("d,B", [(8, 1), (16, 2), (64, 4)])
def test_exact_svd_construction(d, B):
    n = 32 * d
    U = _orthonormal_columns(n, d, 1)
    V = make_basis(d, 5, 0)
    sigma = 3.0 * 0.8 ** np.arange(d)  # distinct, decreasing
    A = (U * sigma) @ V.T
    P, lam = oracle.calibrate(_as_cache(A, B))
    Vs = V * np.sign(V[np.argmax(np.abs(V), axis=0), np.arange(d)])
    assert np.max(np.abs(P[0] - Vs)) < 1e-10
    assert np.max(np.abs(lam[0] / sigma ** 2 - 1.0)) < 1e-10


def test_eigen_equation_on_unstructured_keys():
    rng = np.random.default_rng(3)
    K = rng.standard_normal((2, 3, 200, 16)) * np.exp(-np.arange(16) / 5.0)
    P, lam = oracle.calibrate(K)
    for kv in range(3):
        A = np.concatenate([K[0, kv], K[1, kv]])
        C = A.T @ A
        assert np.max(np.abs(C @ P[kv] - P[kv] * lam[kv])) < 1e-9 * lam[kv, 0]
        assert np.max(np.abs(P[kv].T @ P[kv] - np.eye(16))) < 1e-12
        assert np.all(np.diff(lam[kv]) <= 0) and lam[kv, -1] >= 0


def test_rank_one_along_an_axis():
    d, j = 12, 7
    x = np.random.default_rng(4).standard_normal(50)
    A = np.zeros((50, d))
    A[:, j] = x
    P, lam = oracle.calibrate(_as_cache(A))
    e = np.zeros(d)
    e[j] = 1.0
    assert np.array_equal(P[0][:, 0], e)
    assert abs(lam[0, 0] - np.sum(x * x)) < 1e-12 * np.sum(x * x)
    assert np.all(np.abs(lam[0, 1:]) < 1e-20)


def test_identical_rows_are_not_centred():
    # every key equal to c: the uncentred decomposition finds c / |c| with
    # eigenvalue n |c|^2 (centring would leave a zero matrix)
    c = np.array([3.0, -4.0, 0.0, 12.0])
    A = np.tile(c, (10, 1))
    P, lam = oracle.calibrate(_as_cache(A))
    assert np.max(np.abs(P[0][:, 0] - c / 13.0)) < 1e-14
    assert abs(lam[0, 0] - 10 * 169.0) < 1e-9
    assert np.all(np.abs(lam[0, 1:]) < 1e-9)


def test_scaling_keys():
    K = np.random.default_rng(5).standard_normal((1, 1, 64, 8)) * np.exp(-np.arange(8) / 3.0)
    P1, l1 = oracle.calibrate(K)
    P3, l3 = oracle.calibrate(3.0 * K)
    assert np.max(np.abs(P1 - P3)) < 1e-12
    assert np.max(np.abs(l3 / l1 - 9.0)) < 1e-12


def test_heads_independent_and_batch_rows_pooled():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((3, 2, 40, 8)) * np.exp(-np.arange(8) / 2.0)
    P, lam = oracle.calibrate(K)
    for kv in range(2):
        pooled = np.concatenate([K[b, kv] for b in range(3)])[None, None]
        Pk, lk = oracle.calibrate(pooled)
        assert np.max(np.abs(P[kv] - Pk[0])) < 1e-12
        assert np.max(np.abs(lam[kv] - lk[0])) < 1e-9 * lk[0, 0]
    # swapping the heads swaps the results
    Ps, _ = oracle.calibrate(K[:, ::-1])
    assert np.max(np.abs(Ps[0] - P[1])) < 1e-12


def test_sign_convention():
    K = np.random.default_rng(7).standard_normal((1, 2, 100, 16))
    P, _ = oracle.calibrate(K)
    for kv in range(2):
        j = np.argmax(np.abs(P[kv]), axis=0)
        assert np.all(P[kv][j, np.arange(16)] > 0)


def test_fewer_rows_than_dims_still_gives_an_orthonormal_basis():
    K = np.random.default_rng(8).standard_normal((1, 1, 5, 16))
    P, lam = oracle.calibrate(K)
    assert np.max(np.abs(P[0].T @ P[0] - np.eye(16))) < 1e-12
    assert np.all(lam[0, 5:] == 0.0)
    A = K[0, 0]
    assert np.max(np.abs(A.T @ A @ P[0][:, :5] - P[0][:, :5] * lam[0, :5])) < 1e-9 * lam[0, 0]


def test_recovers_the_generating_basis_and_energy_share():
    # keys drawn as z * exp(-j/tau) in a known basis P0: the sample basis
    # converges to P0 (up to sign) and the energy share of the leading r
    # directions to (1 - e^{-2r/tau}) / (1 - e^{-2d/tau})
    d, tau, n, r = 32, 4.0, 32768, 8
    P0 = make_basis(d, 11, 0)
    Z = np.random.default_rng(9).standard_normal((n, d)) * np.exp(-np.arange(d) / tau)
    P, lam = oracle.calibrate(_as_cache(Z @ P0.T, 2))
    cos = np.abs(np.sum(P[0][:, :r] * P0[:, :r], axis=0))
    assert np.all(cos > 0.99), cos
    want = (1 - np.exp(-2 * r / tau)) / (1 - np.exp(-2 * d / tau))
    got = oracle.energy_fraction(lam, r)[0]
    assert abs(got - want) < 0.01 * want
