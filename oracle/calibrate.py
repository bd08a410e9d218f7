"""Float64 oracle: offline calibration of the projection basis ``P``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* The basis is the set of principal directions of the keys: write the sampled
  keys as a matrix ``A`` (a row per key, ``d_head`` columns) and take its SVD
  ``A = U Sigma V^T``; the right singular vectors (columns of ``V``) are the
  key matrix's principal directions, and keeping the leading ones keeps the
  largest share of the rows' energy (AQUA page, appendix on the SVD, which
  also relates ``V`` to the eigenvectors of ``A^T A``).  Loki uses an
  offline-computed matrix of this kind and keeps the leading dimensions (AQUA
  page, related work "LoKi Attention"); AQUA calibrates it once on another
  dataset (AQUA page, information-retention paragraph and Figure 2).
* :func:`calibrate` is that definition written out with a library SVD: the
  key rows of every batch element of one key/value head form ``A``; ``P`` is
  ``V`` with its columns in decreasing singular-value order, and the reported
  eigenvalues are the squared singular values (the eigenvalues of ``A^T A``).

Readings taken where the pages leave a step open:

1. No centring: the pages decompose the key matrix itself, and the method only
   ever uses ``P`` in dot products with uncentred queries and keys.
2. One basis per key/value head, from the rows of all batch elements of that
   head (the decode's ``P`` is per key/value head and shared over the batch).
3. The sign of an eigenvector is not fixed by the decomposition; the
   convention here makes each column's entry of largest magnitude positive
   (the first such entry when several tie).  When ``A`` has fewer than ``d``
   independent rows, the directions of its null space are any orthonormal
   completion (``numpy``'s full SVD); only the non-degenerate columns are
   unique.
"""

from __future__ import annotations

import numpy as np

from .loki import _f64


def fix_signs(P: np.ndarray) -> np.ndarray:
    """Each column scaled by +-1 so that its entry of largest magnitude (the
    first, on exact ties) is positive."""
    P = np.array(P, dtype=np.float64, copy=True)
    j = np.argmax(np.abs(P), axis=0)  # first maximum per column
    s = np.sign(P[j, np.arange(P.shape[1])])
    s[s == 0] = 1.0
    return P * s


def calibrate(K):
    """Principal basis of the keys, per key/value head.

    ``K``: keys in the cache layout ``[B, Hkv, S, d]`` (NumPy or torch CPU,
    any float dtype; upcast exactly to float64).  Returns ``P [Hkv, d, d]``
    (columns = principal directions, decreasing) and ``eigvals [Hkv, d]``
    (eigenvalues of ``A^T A`` = squared singular values of ``A``, decreasing).
    """
    B, Hkv, S, d = K.shape
    P = np.empty((Hkv, d, d), dtype=np.float64)
    lam = np.zeros((Hkv, d), dtype=np.float64)
    for kv in range(Hkv):
        A = np.concatenate([_f64(K[b, kv]) for b in range(B)], axis=0)  # [B*S, d]
        # the thin decomposition has all d right singular vectors once there
        # are at least d rows; with fewer, the full one completes the basis
        _, sv, Vt = np.linalg.svd(A, full_matrices=A.shape[0] < d)
        P[kv] = fix_signs(Vt.T)
        lam[kv, :sv.shape[0]] = sv ** 2
    return P, lam


def energy_fraction(eigvals, r: int) -> np.ndarray:
    """Share of the keys' energy on the leading ``r`` principal directions,
    per head (the complement of the retention loss of the truncated keys,
    summed over the calibration keys)."""
    lam = np.asarray(eigvals, dtype=np.float64)
    tot = lam.sum(axis=-1)
    return np.where(tot > 0, lam[..., :r].sum(axis=-1) / np.where(tot > 0, tot, 1.0), 1.0)
