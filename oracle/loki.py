"""Float64 oracle: the decode step of Loki-style low-rank-key sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* Decode attention for one new token (AQUA page, preliminaries, eqs. 3-5):
  scores ``S = q K^T`` (eq. 3), weights ``A = softmax(S / sqrt(d_head))``
  (eq. 4), context ``c = A V`` (eq. 5), over the cache after the new key and
  value were appended (eqs. 1-2).  :func:`dense` is exactly that.
* Projection into an offline basis with the row-vector convention
  ``v_hat = v P`` (AQUA page, information-retention-loss paragraph), applied
  to queries and keys; with an orthogonal ``P`` it preserves every ``q . k``
  (AQUA page, appendix proof that the projection is a lossless rotation).
  :func:`project`, :func:`rotate_queries`.
* Loki (Loki page, abstract; AQUA page, related work "LoKi Attention"): the
  rotated query and keys are truncated to their leading dimensions, the
  resulting approximate scores rank the cached tokens, the best ones are kept
  for this step only (nothing is evicted), and attention runs over the kept
  tokens.  :func:`approx_scores`, :func:`select`, :func:`attend`,
  :func:`decode`; :func:`decode_varlen` for a batch of sequences of
  different lengths (each one a decode over its own prefix).

Readings taken where the pages leave a step open:

1. "Slicing off the trailing dimensions" keeps the LEADING ``r`` rotated
   dimensions (the first columns of ``P`` carry the most key variance).
2. Approximate scores are unscaled (a positive scale never changes a ranking).
3. The kept set is the ``k`` largest approximate scores per QUERY head; ties
   go to the lower token index; indices are returned in ascending order.
4. The exact stage uses the full-``d`` rotated keys ``K_rot[idx]`` with the
   full rotated query and the ``1/sqrt(d)`` scale of eq. 4; the softmax is
   normalised over the kept tokens only; ``V`` is not rotated.
5. Grouped-query attention: query head ``h`` reads key/value head
   ``h // (Hq/Hkv)`` (contiguous groups), and ``P`` belongs to the key head.
6. No causal mask: every cached token is eligible.

Inputs may be NumPy arrays or torch CPU tensors of any float dtype; each
``(b, kv)`` slice is upcast exactly to float64 on its own so that large
caches never exist whole in float64.
"""

from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a NumPy array or torch tensor (fp32/bf16/fp64) to float64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    import torch  # torch only as a container of the stored values
    return x.detach().to("cpu").to(torch.float64).numpy()


def _shapes(q, K_rot):
    B, Hq, d = q.shape
    Bk, Hkv, S, dk = K_rot.shape
    if Bk != B or dk != d or Hq % Hkv:
        raise ValueError("inconsistent shapes")
    return B, Hq, Hkv, S, d, Hq // Hkv


def project(K, P) -> np.ndarray:
    """Cached keys in the rotated basis, ``K_rot[b, kv] = K[b, kv] P[kv]``.

    Row-vector convention ``v_hat = v P`` (AQUA page, information-retention
    paragraph); one matrix product per (batch, key head).
    """
    B, Hkv, S, d = K.shape
    out = np.empty((B, Hkv, S, d), dtype=np.float64)
    for kv in range(Hkv):
        Pk = _f64(P[kv])
        for b in range(B):
            out[b, kv] = _f64(K[b, kv]) @ Pk
    return out


def rotate_queries(q, P) -> np.ndarray:
    """``q_rot[b, h] = q[b, h] P[h // G]`` in float64 (full head dimension)."""
    B, Hq, d = q.shape
    Hkv = P.shape[0]
    G = Hq // Hkv
    qq = _f64(q)
    out = np.empty((B, Hq, d), dtype=np.float64)
    for h in range(Hq):
        out[:, h] = qq[:, h] @ _f64(P[h // G])
    return out


def approx_scores(q, P, K_rot, r: int) -> np.ndarray:
    """Low-dimensional scores ``s[b, h, j] = sum_{c<r} q_rot[b,h,c] K_rot[b,kv,j,c]``.

    The rotated query and keys keep their leading ``r`` dimensions (Loki page,
    abstract: scores computed in a low-dimensional space; AQUA page, related
    work: Loki slices after an offline projection).  Unscaled.
    """
    B, Hq, Hkv, S, d, G = _shapes(q, K_rot)
    if not 1 <= r <= d:
        raise ValueError("r out of range")
    qr = rotate_queries(q, P)
    s = np.empty((B, Hq, S), dtype=np.float64)
    for b in range(B):
        for kv in range(Hkv):
            kslice = _f64(K_rot[b, kv, :, :r])
            for g in range(G):
                h = kv * G + g
                s[b, h] = kslice @ qr[b, h, :r]
    return s


def topk_indices(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the ``k`` largest entries of a 1-D score vector.

    Ties are broken towards the lower index (a stable sort of ``-s``); the
    result is returned in ascending index order.
    """
    S = s.shape[0]
    if not 1 <= k <= S:
        raise ValueError("k out of range")
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:k])


def select(q, P, K_rot, r: int, k: int, return_scores: bool = False):
    """Per query head, the ``k`` cached tokens with the largest approximate scores.

    Returns ``idx [B, Hq, k]`` (int64, ascending), and the float64 approximate
    scores ``[B, Hq, S]`` when ``return_scores``.
    """
    s = approx_scores(q, P, K_rot, r)
    B, Hq, S = s.shape
    idx = np.empty((B, Hq, k), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            idx[b, h] = topk_indices(s[b, h], k)
    return (idx, s) if return_scores else idx


def attend(q, P, K_rot, V, idx, return_weights: bool = False):
    """Exact softmax attention of each query head over its kept tokens only.

    For kept tokens ``j in idx[b, h]``: ``e_j = q_rot . K_rot[b,kv,j,:] /
    sqrt(d)`` (eqs. 3-4 with the full head dimension; the rotation preserves
    ``q . k``), ``w = softmax(e)`` over the kept set, ``out = sum_j w_j
    V[b,kv,j,:]`` (eq. 5).  Tokens outside ``idx`` take no part in this step.
    """
    B, Hq, Hkv, S, d, G = _shapes(q, K_rot)
    idx = np.asarray(idx)
    qr = rotate_queries(q, P)
    out = np.empty((B, Hq, d), dtype=np.float64)
    weights = np.empty(idx.shape, dtype=np.float64) if return_weights else None
    scale = 1.0 / math.sqrt(d)
    for b in range(B):
        for kv in range(Hkv):
            kk = _f64(K_rot[b, kv])
            vv = _f64(V[b, kv])
            for g in range(G):
                h = kv * G + g
                sel = idx[b, h]
                e = (kk[sel] @ qr[b, h]) * scale
                w = np.exp(e - e.max())
                w /= w.sum()
                out[b, h] = w @ vv[sel]
                if return_weights:
                    weights[b, h] = w
    return (out, weights) if return_weights else out


def decode(q, P, K_rot, V, r: int, k: int):
    """One Loki decode step: select by leading-``r`` scores, then attend exactly.

    Returns ``(out [B,Hq,d] float64, idx [B,Hq,k] int64 ascending)``.
    """
    idx = select(q, P, K_rot, r, k)
    return attend(q, P, K_rot, V, idx), idx


def decode_varlen(q, P, K_rot, V, lens, r: int, k: int, return_scores: bool = False):
    """One Loki decode step over a ragged batch.

    Sequence ``b`` holds only its first ``len_b`` cached tokens (``lens[b]``
    clamped into ``[1, S]``); the rest of its cache rows are unused capacity
    and take no part.  Each sequence is an ordinary decode over its own prefix
    (the AQUA page's eqs. 1-5 on a cache of ``len_b`` tokens, Loki's selection
    on it): the kept set is its ``min(k, len_b)`` best tokens, and ``idx``
    rows of sequences shorter than ``k`` end with ``-1``.

    Returns ``(out [B,Hq,d], idx [B,Hq,k])`` and, with ``return_scores``, the
    approximate scores ``[B,Hq,S]`` with ``-inf`` past each sequence's end.
    """
    B, Hq, Hkv, S, d, G = _shapes(q, K_rot)
    out = np.empty((B, Hq, d), dtype=np.float64)
    idx = np.full((B, Hq, k), -1, dtype=np.int64)
    scores = np.full((B, Hq, S), -np.inf) if return_scores else None
    for b in range(B):
        L = min(max(int(lens[b]), 1), S)
        kb = min(k, L)
        sel, s = select(q[b:b + 1], P, K_rot[b:b + 1, :, :L], r, kb, return_scores=True)
        out[b] = attend(q[b:b + 1], P, K_rot[b:b + 1, :, :L], V[b:b + 1, :, :L], sel)[0]
        idx[b, :, :kb] = sel[0]
        if return_scores:
            scores[b, :, :L] = s[0]
    return (out, idx, scores) if return_scores else (out, idx)


def dense(q, K, V) -> np.ndarray:
    """Full decode attention over the unrotated cache (AQUA page, eqs. 3-5).

    ``A = softmax(q K^T / sqrt(d))`` over all cached tokens, ``c = A V``;
    query head ``h`` reads key/value head ``h // G``.
    """
    B, Hq, Hkv, S, d, G = _shapes(q, K)
    qq = _f64(q)
    out = np.empty((B, Hq, d), dtype=np.float64)
    for b in range(B):
        for kv in range(Hkv):
            kk = _f64(K[b, kv])
            vv = _f64(V[b, kv])
            for g in range(G):
                h = kv * G + g
                e = (kk @ qq[b, h]) / math.sqrt(d)
                w = np.exp(e - e.max())
                w /= w.sum()
                out[b, h] = w @ vv
    return out
