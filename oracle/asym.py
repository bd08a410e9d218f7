"""Float64 oracle: an asymmetric low-rank scoring index (query side A, key side B).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* SAKI (page "SAKI: Score-Aware Low-Rank Key Indexing with Random-Matrix
  Noise Correction for KV Retrieval", abstract): the mean squared error
  of the scores under a rank-r key index, weighted by the query and key
  second moments, is minimised by two different (query-side, key-side)
  rank-r factors, both taken from one SVD: that of ``Cq^1/2 Ck^1/2``.  Written out: approximate scores are ``(q A_r) . (k B_r)``; with
  query and key second moments ``Cq = E[q^T q]``, ``Ck = E[k^T k]`` and
  independent q, k, the mean squared score error of ``M = A_r B_r^T`` is
  ``|| Cq^{1/2} (I - M) Ck^{1/2} ||_F^2``; by the Eckart-Young theorem the
  best rank-r M comes from the SVD ``Cq^{1/2} Ck^{1/2} = U S V^T``:
  ``A_r = Cq^{-1/2} U_r S_r^{1/2}``, ``B_r = Ck^{-1/2} V_r S_r^{1/2}``.
  :func:`saki_factors`, :func:`calibrate`, :func:`distortion`.
* The index is used like Loki's leading dims: the approximate scores rank the
  cached tokens, the ``k`` best are kept for this step, and exact attention
  runs over them with the query and keys themselves (AQUA page, eqs. 3-5 on
  the kept set).  :func:`scores`, :func:`select`, :func:`decode`.

Readings taken where the pages leave a step open:

1. Uncentred second moments (as for the basis calibration); the random-matrix
   noise correction of the pages is not part of this step.
2. One pair (A_r, B_r) per key/value head; the query statistics pool the
   queries of that head's group.
3. ``Cq^{-1/2}`` and ``Ck^{-1/2}`` are pseudo-inverse square roots:
   eigenvalues below ``floor * lambda_max`` count as zero.
4. The stored index ``K_idx = K B`` (rounded to the cache dtype) is an input of
   the decode, like Loki's rotated cache; exact attention uses ``q`` and ``K``.
"""

from __future__ import annotations

import numpy as np

from .loki import _f64, attend, topk_indices


def _psd_pow(C, p, floor):
    w, U = np.linalg.eigh(C)
    w = np.maximum(w, 0.0)
    keep = w > floor * max(w.max(), 0.0)
    wp = np.zeros_like(w)
    wp[keep] = w[keep] ** p
    return (U * wp) @ U.T


def saki_factors(Cq, Ck, r: int, floor: float = 1e-12):
    """``(A_r, B_r)``, each ``[d, r]``, minimising ``|| Cq^{1/2}(I - A_r B_r^T) Ck^{1/2} ||_F``."""
    Cq, Ck = np.asarray(Cq, np.float64), np.asarray(Ck, np.float64)
    W = _psd_pow(Cq, 0.5, floor) @ _psd_pow(Ck, 0.5, floor)
    U, s, Vt = np.linalg.svd(W)
    sr = np.sqrt(s[:r])
    A = _psd_pow(Cq, -0.5, floor) @ (U[:, :r] * sr)
    B = _psd_pow(Ck, -0.5, floor) @ (Vt[:r].T * sr)
    return A, B


def distortion(Cq, Ck, M) -> float:
    """``|| Cq^{1/2} (I - M) Ck^{1/2} ||_F^2``: the mean squared score error of
    ``q M k^T`` against ``q k^T`` for independent q, k with these second moments."""
    d = M.shape[0]
    E = _psd_pow(np.asarray(Cq, np.float64), 0.5, 0.0) @ (np.eye(d) - M) @ _psd_pow(np.asarray(Ck, np.float64), 0.5, 0.0)
    return float(np.sum(E * E))


def calibrate(q_samples, K, r: int, floor: float = 1e-12):
    """Per key/value head, the SAKI factors from query samples
    ``[N, Hq, d]`` (the queries of the head's group pooled) and the keys
    ``[B, Hkv, S, d]``: ``A [Hkv, d, r]``, ``B [Hkv, d, r]``."""
    Qs = _f64(q_samples)
    N, Hq, d = Qs.shape
    Bk, Hkv, S, _ = K.shape
    G = Hq // Hkv
    A = np.empty((Hkv, d, r))
    Bm = np.empty((Hkv, d, r))
    for kv in range(Hkv):
        Qk = Qs[:, kv * G:(kv + 1) * G].reshape(-1, d)
        Kk = np.concatenate([_f64(K[b, kv]) for b in range(Bk)])
        A[kv], Bm[kv] = saki_factors(Qk.T @ Qk / len(Qk), Kk.T @ Kk / len(Kk), r, floor)
    return A, Bm


def scores(q, A, K_idx, r: int) -> np.ndarray:
    """``s[b,h,j] = sum_{c<r} (q[b,h] A[kv])[c] K_idx[b,kv,j,c]``."""
    qq = _f64(q)
    B, Hq, d = qq.shape
    Hkv = K_idx.shape[1]
    G = Hq // Hkv
    S = K_idx.shape[2]
    out = np.empty((B, Hq, S))
    for b in range(B):
        for kv in range(Hkv):
            ki = _f64(K_idx[b, kv])[:, :r]
            Ak = _f64(A[kv])[:, :r]
            for g in range(G):
                h = kv * G + g
                out[b, h] = ki @ (qq[b, h] @ Ak)
    return out


def select(q, A, K_idx, r: int, k: int, return_scores: bool = False):
    s = scores(q, A, K_idx, r)
    B, Hq, _ = s.shape
    idx = np.empty((B, Hq, k), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            idx[b, h] = topk_indices(s[b, h], k)
    return (idx, s) if return_scores else idx


def decode(q, A, K_idx, K, V, r: int, k: int):
    """Token selection by the index scores, exact attention with ``q`` and
    ``K`` over the kept tokens: ``(out, idx)``."""
    idx = select(q, A, K_idx, r, k)
    d = q.shape[-1]
    Hkv = K.shape[1]
    eye = np.broadcast_to(np.eye(d), (Hkv, d, d))
    return attend(q, eye, K, V, idx), idx
