"""Float64 oracle: query-magnitude dimension selection for the score stage.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* AQUA (AQUA page, online phase and Algorithm 1 prose): after projecting the
  query into the basis, the dimensions kept for the approximate scores are
  the ones where the projected query has the largest magnitude, and the
  approximate scores use only those dimensions of the query and of every
  cached key.  :func:`query_dims`, :func:`approx_scores`.
* Here those scores rank the cached tokens exactly as Loki's leading-dims
  scores do: the ``k`` best tokens are kept and exact attention runs over
  them with the full rotated query and keys (the same :func:`~oracle.loki.attend`).
  :func:`select`, :func:`decode`.
* The information retention loss of a vector ``v`` with projection
  ``v_hat = v P`` and kept indices ``I`` (AQUA page, information-retention
  paragraph): ``| ||v|| - ||v_hat[I]|| | / ||v||``.  :func:`info_loss`.

Readings taken where the pages leave a step open:

1. The number of kept dimensions is ``r`` (AQUA's ``k`` counts dimensions;
   here ``k`` counts tokens).
2. Ties in magnitude go to the lower dimension index; the kept dimensions are
   reported in ascending order.
3. Each query head chooses its own dimensions; the keys of a group are read
   at every head's own dimensions (grouped-query attention as in Loki).
"""

from __future__ import annotations

import numpy as np

from .loki import _f64, _shapes, attend, rotate_queries, topk_indices


def query_dims(q, P, r: int):
    """Per query head, the ``r`` dimensions of ``q_rot = q P[kv]`` with the
    largest magnitude (ties -> lower index), ascending: ``[B, Hq, r]`` int64."""
    qr = rotate_queries(q, P)
    B, Hq, d = qr.shape
    out = np.empty((B, Hq, r), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            order = np.argsort(-np.abs(qr[b, h]), kind="stable")  # stable: lower index first on ties
            out[b, h] = np.sort(order[:r])
    return out


def approx_scores(q, P, K_rot, r: int) -> np.ndarray:
    """``s[b,h,j] = sum_{c in I_h} q_rot[b,h,c] K_rot[b,kv,j,c]``, I_h the
    head's magnitude-selected dimensions."""
    return scores_on_dims(q, P, K_rot, query_dims(q, P, r))


def scores_on_dims(q, P, K_rot, dims) -> np.ndarray:
    """The approximate scores of each query head on a given set of rotated
    dimensions ``dims [B, Hq, r]``: ``s[b,h,j] = sum_{c in dims[b,h]}
    q_rot[b,h,c] K_rot[b,kv,j,c]``."""
    B, Hq, Hkv, S, d, G = _shapes(q, K_rot)
    qr = rotate_queries(q, P)
    dims = np.asarray(dims)
    s = np.empty((B, Hq, S), dtype=np.float64)
    for b in range(B):
        for kv in range(Hkv):
            kr = _f64(K_rot[b, kv])
            for g in range(G):
                h = kv * G + g
                I = dims[b, h]
                s[b, h] = kr[:, I] @ qr[b, h, I]
    return s


def select(q, P, K_rot, r: int, k: int, return_scores: bool = False):
    """The ``k`` tokens with the largest magnitude-selected approximate
    scores per query head (ties -> lower index), ascending."""
    s = approx_scores(q, P, K_rot, r)
    B, Hq, _ = s.shape
    idx = np.empty((B, Hq, k), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            idx[b, h] = topk_indices(s[b, h], k)
    return (idx, s) if return_scores else idx


def decode(q, P, K_rot, V, r: int, k: int):
    """Token selection by the magnitude-selected scores, then exact attention
    over the kept tokens: ``(out [B,Hq,d], idx [B,Hq,k])``."""
    idx = select(q, P, K_rot, r, k)
    return attend(q, P, K_rot, V, idx), idx


def info_loss(q, P, dims) -> np.ndarray:
    """Information retention loss of each query head's kept dimensions:
    ``| ||q|| - ||q_rot[I]|| | / ||q||`` (0 for a zero query)."""
    qq = _f64(q)
    qr = rotate_queries(q, P)
    B, Hq, _ = qq.shape
    out = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            n = np.linalg.norm(qq[b, h])
            if n > 0:
                out[b, h] = abs(n - np.linalg.norm(qr[b, h, dims[b, h]])) / n
    return out
