"""Seeded generators for the decode workloads.

Recipe (all in float64, then one rounding to the storage dtype):

* ``P[kv]`` -- the Q factor of the QR decomposition of a seeded N(0,1)
  ``d x d`` matrix, with column signs fixed so that ``diag(R) > 0``.  One
  basis per key/value head, shared over the batch.  Columns are the rotated
  coordinate axes; the row-vector convention ``v_hat = v P`` of the AQUA page
  (information-retention-loss paragraph) maps a vector into them.
* Keys are generated in the rotated coordinates and mapped back:
  ``K_rot_true = Z * s`` with ``Z ~ N(0,1)`` of shape ``[S, d]`` and
  ``s_j = exp(-j/tau)``; the cached keys in the original basis are
  ``K = K_rot_true P^T``.  For a noisy workload ``noise * N(0,1)`` is added
  to every rotated coordinate; since ``P`` is orthogonal this is the same
  distribution as isotropic noise added in the original basis.
* Queries are drawn the same way per query head, in the basis of the key
  head they read: ``q = (z * s) P[kv]^T``.
* Values are ``V ~ N(0,1)`` of shape ``[S, d]``, never rotated.
* Heavy tokens (long-context workload): for each query head, in head order,
  ``heavy`` distinct positions are drawn; at each, the key's component along
  the head's unit query direction ``u`` is set to ``+4 sigma`` where
  ``sigma^2 = sum_j u_j^2 (s_j^2 + noise^2)`` is the variance of ``k . u``
  over the key distribution.

The tensor handed to the decode call is ``K_rot = round(K_rot_true)``; the
tensor handed to the key projection is ``K = round(K_rot_true P^T)``.  The
two are consistent up to rounding only, which is irrelevant to parity since
both the oracle and the GPU path consume the same stored values.

Every random stream is ``numpy.random.default_rng(SeedSequence([0x4C4F4B49,
cfg_no, role, b, h, seed]))`` so each slice can be regenerated alone.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import Config

_MAGIC = 0x4C4F4B49
ROLE_P, ROLE_K, ROLE_Q, ROLE_V, ROLE_HEAVY, ROLE_NOISE, ROLE_INT, ROLE_QSAMPLE = range(8)

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def rng(cfg_no: int, role: int, b: int = 0, h: int = 0, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([_MAGIC, cfg_no, role, b, h, seed]))


def make_basis(d: int, cfg_no: int, kv: int, seed: int = 0) -> np.ndarray:
    """Orthonormal ``d x d`` basis from the QR of a seeded Gaussian matrix."""
    a = rng(cfg_no, ROLE_P, 0, kv, seed).standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    signs = np.sign(np.diag(rm))
    signs[signs == 0] = 1.0
    return qm * signs[None, :]


def spectrum(cfg: Config) -> np.ndarray:
    return np.exp(-np.arange(cfg.d, dtype=np.float64) / cfg.tau)


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dtype])


def make_inputs(cfg: Config, need_K: bool = False, seed: int = 0) -> dict:
    """All decode inputs of one workload as CPU torch tensors in ``cfg.dtype``.

    Returns a dict with ``q [B,Hq,d]``, ``P [Hkv,d,d]``, ``K_rot [B,Hkv,S,d]``,
    ``V [B,Hkv,S,d]``, ``K [B,Hkv,S,d]`` (only if ``need_K``), ``heavy_idx
    [B,Hq,heavy]`` int64 (or None) and ``cfg``.
    """
    B, Hq, Hkv, d, S, G = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.S, cfg.G
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    tdt = TORCH_DTYPE[cfg.dtype]
    s = spectrum(cfg)
    P64 = np.stack([make_basis(d, cfg.cfg_no, kv, seed) for kv in range(Hkv)])
    q = torch.empty((B, Hq, d), dtype=tdt)
    K_rot = torch.empty((B, Hkv, S, d), dtype=tdt)
    V = torch.empty((B, Hkv, S, d), dtype=tdt)
    K = torch.empty((B, Hkv, S, d), dtype=tdt) if need_K else None
    heavy_idx = torch.empty((B, Hq, cfg.heavy), dtype=torch.int64) if cfg.heavy else None
    for b in range(B):
        for kv in range(Hkv):
            kr = rng(cfg.cfg_no, ROLE_K, b, kv, seed).standard_normal((S, d)) * s
            if cfg.noise:
                kr += cfg.noise * rng(cfg.cfg_no, ROLE_NOISE, b, kv, seed).standard_normal((S, d))
            for g in range(G):
                h = kv * G + g
                qr = rng(cfg.cfg_no, ROLE_Q, b, h, seed).standard_normal(d) * s
                q[b, h] = _to(qr @ P64[kv].T, cfg.dtype)
                if cfg.heavy:
                    pos = rng(cfg.cfg_no, ROLE_HEAVY, b, h, seed).choice(S, cfg.heavy, replace=False)
                    u = qr / np.linalg.norm(qr)
                    sigma = np.sqrt(np.sum(u * u * (s * s + cfg.noise ** 2)))
                    along = kr[pos] @ u
                    kr[pos] += (4.0 * sigma - along)[:, None] * u[None, :]
                    heavy_idx[b, h] = torch.from_numpy(np.sort(pos))
            K_rot[b, kv] = _to(kr, cfg.dtype)
            if need_K:
                K[b, kv] = _to(kr @ P64[kv].T, cfg.dtype)
            V[b, kv] = _to(rng(cfg.cfg_no, ROLE_V, b, kv, seed).standard_normal((S, d)), cfg.dtype)
    return {"q": q, "P": _to(P64, cfg.dtype), "K_rot": K_rot, "V": V, "K": K,
            "heavy_idx": heavy_idx, "cfg": cfg, "P64": P64}


def make_query_samples(cfg: Config, n: int, seed: int = 0) -> torch.Tensor:
    """``n`` further queries per query head drawn like the workload's queries
    (the spectrum in ``make_basis(d, cfg_no, kv, seed)``: the basis of the key
    head they read for the workload's own seed, another basis for another
    seed), as calibration data: ``[n, Hq, d]`` in ``cfg.dtype``."""
    s = spectrum(cfg)
    out = np.empty((n, cfg.Hq, cfg.d))
    for kv in range(cfg.Hkv):
        P = make_basis(cfg.d, cfg.cfg_no, kv, seed)
        for g in range(cfg.G):
            h = kv * cfg.G + g
            z = rng(cfg.cfg_no, ROLE_QSAMPLE, 0, h, seed).standard_normal((n, cfg.d)) * s
            out[:, h] = z @ P.T
    return _to(out, cfg.dtype)


def make_integer_inputs(B: int, Hq: int, Hkv: int, d: int, S: int, dtype: str,
                        seed: int = 0, lo: int = -3, hi: int = 3, P_kind: str = "identity") -> dict:
    """Inputs whose scores are exact small integers in any precision.

    ``P`` is the identity (or a signed permutation when ``P_kind='signed_perm'``),
    ``q`` and ``K_rot`` hold integers in ``[lo, hi]``, so every dot product is an
    exact integer in fp32 and float64 alike and planted ties stay ties on both
    sides.  ``V`` is integer-valued too.
    """
    g = rng(900, ROLE_INT, 0, 0, seed)
    q = g.integers(lo, hi + 1, size=(B, Hq, d)).astype(np.float64)
    Kr = g.integers(lo, hi + 1, size=(B, Hkv, S, d)).astype(np.float64)
    Vv = g.integers(-4, 5, size=(B, Hkv, S, d)).astype(np.float64)
    if P_kind == "identity":
        P = np.broadcast_to(np.eye(d), (Hkv, d, d)).copy()
    elif P_kind == "signed_perm":
        P = np.zeros((Hkv, d, d))
        for kv in range(Hkv):
            perm = g.permutation(d)
            sg = g.choice([-1.0, 1.0], size=d)
            P[kv, np.arange(d), perm] = sg
    else:
        raise ValueError(P_kind)
    return {"q": _to(q, dtype), "P": _to(P, dtype), "K_rot": _to(Kr, dtype), "V": _to(Vv, dtype)}


def ordered_scores_fixture(S: int, seed: int = 0) -> np.ndarray:
    """Integer-valued score vector with planted exact ties (for selection tests)."""
    g = rng(901, ROLE_INT, 0, 0, seed)
    return g.integers(-5, 6, size=S).astype(np.float64)
