"""Comparison rules between the HIP path and the float64 oracle.

Selected index sets: bit-exact, except tokens whose oracle approximate score
lies within 1e-4 (relative) of the oracle's k-th largest score; those may be
exchanged for one another (several answers are then correct).
Outputs: max-abs 1e-5 for fp32 storage, 2e-2 for bf16 storage.
"""

from __future__ import annotations

import numpy as np
import torch

BAND_REL = 1e-4
OUT_TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def check_index_sets(idx_gpu: np.ndarray, idx_oracle: np.ndarray, s_oracle: np.ndarray, k: int):
    """Returns the list of (b, h) rows whose GPU set differs from the oracle's
    (inside the band only); raises AssertionError on any real mismatch."""
    B, Hq, kk = idx_gpu.shape
    assert kk == k
    differ = []
    for b in range(B):
        for h in range(Hq):
            g = idx_gpu[b, h]
            assert np.all(np.diff(g) > 0), f"row {(b, h)}: not strictly ascending"
            assert g[0] >= 0 and g[-1] < s_oracle.shape[-1], f"row {(b, h)}: index out of range"
            o = idx_oracle[b, h]
            if np.array_equal(g, o):
                continue
            s = s_oracle[b, h]
            sstar = np.sort(s)[::-1][k - 1]
            if sstar == 0.0:
                band = set(np.nonzero(s == 0.0)[0].tolist())
            else:
                band = set(np.nonzero(np.abs(s - sstar) <= BAND_REL * abs(sstar))[0].tolist())
            gs, os_ = set(g.tolist()) - band, set(o.tolist()) - band
            assert gs == os_, (f"row {(b, h)}: {len(gs ^ os_)} tokens differ outside the tie band "
                               f"(band size {len(band)})")
            differ.append((b, h))
    return differ


def max_abs(a, b) -> float:
    a = a.double().cpu().numpy() if isinstance(a, torch.Tensor) else np.asarray(a, dtype=np.float64)
    b = b.double().cpu().numpy() if isinstance(b, torch.Tensor) else np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def oracle_attend_rows(q, P, K_rot, V, idx, rows, lens=None) -> dict:
    """The oracle's exact attention of each listed (b, h) row over the kept set
    that ``idx[b, h]`` gives (entries < 0 dropped), on that row's own prefix
    when ``lens`` is given: ``{(b, h): out [d] float64}``.  Each row is one
    oracle call on its own (query head, key head) slice, so the other rows'
    sets take no part."""
    import oracle
    Hq, Hkv, S = q.shape[1], K_rot.shape[1], K_rot.shape[2]
    G = Hq // Hkv
    res = {}
    for b, h in rows:
        kv = h // G
        L = S if lens is None else min(max(int(lens[b]), 1), S)
        sel = np.asarray(idx[b, h]).astype(np.int64)
        sel = sel[sel >= 0]
        o = oracle.attend(q[b:b + 1, h:h + 1], P[kv:kv + 1], K_rot[b:b + 1, kv:kv + 1, :L],
                          V[b:b + 1, kv:kv + 1, :L], sel[None, None, :])
        res[(b, h)] = o[0, 0]
    return res


def check_band_rows(out_gpu: np.ndarray, idx_gpu: np.ndarray, rows, q, P, K_rot, V, tol: float, lens=None):
    """Rows whose kept set legitimately differs from the oracle's (inside the
    tie band): the GPU output must be the oracle's attention over the GPU's
    own kept set, to the output tolerance."""
    want = oracle_attend_rows(q, P, K_rot, V, idx_gpu, rows, lens)
    for (b, h), o in want.items():
        err = float(np.max(np.abs(out_gpu[b, h] - o)))
        assert err <= tol, f"band row {(b, h)}: output max-abs {err} > {tol} against the oracle on its own set"
