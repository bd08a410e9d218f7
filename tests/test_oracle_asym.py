"""Pins of the oracle's asymmetric scoring index (SAKI page, abstract: the
score error weighted by the query and key second moments is minimised by
different query-side and key-side rank-r factors from one SVD) against facts
that do not come from it:

* Eckart-Young: the distortion of the factors equals the sum of the squared
  trailing singular values of Cq^{1/2} Ck^{1/2}, and no other rank-r product
  (PCA projector, random projections) does better;
* isotropic queries reduce it to the projector on the keys' leading
  principal directions (Loki's index);
* full rank gives exact scores;
* with A = B = P orthonormal and the index K P, the scores are Loki's;
* Monte Carlo: the mean squared score error of sampled q, k matches the
  distortion formula;
* keeping every token gives dense attention over the keys themselves.
"""

import numpy as np
import pytest

import oracle
from oracle import asym
from loki_inputs import make_basis


def _cov(d, seed, decay):
    U = make_basis(d, 80 + seed, 0)
    return (U * np.exp(-np.arange(d) / decay)) @ U.T


def test_eckart_young_optimum():
    d, r = 16, 5
    Cq, Ck = _cov(d, 1, 4.0), _cov(d, 2, 3.0)
    A, B = asym.saki_factors(Cq, Ck, r)
    W = asym._psd_pow(Cq, 0.5, 0.0) @ asym._psd_pow(Ck, 0.5, 0.0)
    s = np.linalg.svd(W, compute_uv=False)
    got = asym.distortion(Cq, Ck, A @ B.T)
    assert abs(got - np.sum(s[r:] ** 2)) < 1e-10 * np.sum(s ** 2)
    # no rank-r alternative does better: the keys' PCA projector, random ones
    w, V = np.linalg.eigh(Ck)
    Vr = V[:, np.argsort(-w)[:r]]
    assert got <= asym.distortion(Cq, Ck, Vr @ Vr.T) + 1e-12
    rng = np.random.default_rng(3)
    for _ in range(20):
        X, Y = rng.standard_normal((d, r)), rng.standard_normal((d, r))
        assert got <= asym.distortion(Cq, Ck, X @ Y.T) + 1e-12


def test_isotropic_queries_give_the_key_pca_projector():
    d, r = 12, 4
    Ck = _cov(d, 4, 2.5)
    A, B = asym.saki_factors(np.eye(d), Ck, r)
    w, V = np.linalg.eigh(Ck)
    Vr = V[:, np.argsort(-w)[:r]]
    assert np.max(np.abs(A @ B.T - Vr @ Vr.T)) < 1e-10
    # the same projector as the oracle's basis calibration on keys with that second moment
    Z = np.random.default_rng(5).standard_normal((4000, d))
    K = (Z * np.exp(-np.arange(d) / 5.0)) @ make_basis(d, 90, 0).T
    P, _ = oracle.calibrate(K[None, None])
    A2, B2 = asym.saki_factors(np.eye(d), K.T @ K / len(K), r)
    assert np.max(np.abs(A2 @ B2.T - P[0][:, :r] @ P[0][:, :r].T)) < 1e-9


def test_full_rank_scores_are_exact():
    d = 8
    Cq, Ck = _cov(d, 6, 2.0), _cov(d, 7, 3.0)
    A, B = asym.saki_factors(Cq, Ck, d)
    assert np.max(np.abs(A @ B.T - np.eye(d))) < 1e-8
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 2, d))
    K = rng.standard_normal((1, 1, 30, d))
    K_idx = np.einsum("bhsd,dr->bhsr", K, B)
    s = asym.scores(q, A[None], K_idx, d)
    assert np.max(np.abs(s[0] - q[0] @ K[0, 0].T)) < 1e-8


def test_orthonormal_symmetric_case_is_loki():
    d, r = 16, 6
    P = np.stack([make_basis(d, 91, kv) for kv in range(2)])
    rng = np.random.default_rng(9)
    q = rng.standard_normal((2, 4, d))
    K_rot = rng.standard_normal((2, 2, 40, d))
    s = asym.scores(q, P, K_rot, r)
    assert np.max(np.abs(s - oracle.approx_scores(q, P, K_rot, r))) < 1e-12


def test_monte_carlo_distortion():
    d, r, n = 8, 3, 200000
    Cq, Ck = _cov(d, 10, 2.0), _cov(d, 11, 4.0)
    A, B = asym.saki_factors(Cq, Ck, r)
    rng = np.random.default_rng(12)
    q = rng.standard_normal((n, d)) @ asym._psd_pow(Cq, 0.5, 0.0)
    k = rng.standard_normal((n, d)) @ asym._psd_pow(Ck, 0.5, 0.0)
    err = np.sum((q @ A) * (k @ B), axis=1) - np.sum(q * k, axis=1)
    want = asym.distortion(Cq, Ck, A @ B.T)
    assert abs(np.mean(err ** 2) / want - 1.0) < 0.05


def test_keep_everything_is_dense_attention():
    d = 16
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 4, d))
    K = rng.standard_normal((1, 2, 25, d))
    V = rng.standard_normal((1, 2, 25, d))
    A = rng.standard_normal((2, d, 4))
    K_idx = rng.standard_normal((1, 2, 25, 4))
    out, idx = asym.decode(q, A, K_idx, K, V, 4, 25)
    assert np.max(np.abs(out - oracle.dense(q, K, V))) < 1e-12


def test_calibrate_pools_the_group_queries():
    d, r = 8, 3
    rng = np.random.default_rng(14)
    qs = rng.standard_normal((50, 4, d))
    K = rng.standard_normal((2, 2, 40, d))
    A, B = asym.calibrate(qs, K, r)
    Qk = qs[:, 2:4].reshape(-1, d)
    Kk = np.concatenate([K[0, 1], K[1, 1]])
    A1, B1 = asym.saki_factors(Qk.T @ Qk / len(Qk), Kk.T @ Kk / len(Kk), r)
    assert np.max(np.abs(A[1] @ B[1].T - A1 @ B1.T)) < 1e-12
