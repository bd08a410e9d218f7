"""Pins of the oracle's query-magnitude dimension selection (AQUA page,
online phase and information-retention paragraph) against facts that do not
come from it:

* with all d dimensions kept it is Loki's full-rank selection;
* a query whose rotated form lives on the leading r dimensions chooses
  exactly those, so it equals Loki's leading-dims selection;
* permuting the basis columns (and the cached keys' columns with them)
  changes nothing -- the choice follows the query, not the column order --
  while Loki's leading-dims scores do change;
* brute force on tiny d: the kept set maximises the retained query energy
  over all subsets of size r (ties -> the lower-index set);
* closed forms of the information retention loss;
* exact attention over the kept tokens is the same stage as Loki's.
"""

import itertools

import numpy as np
import pytest

import oracle
from oracle import aqua
from loki_inputs import make_basis


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(B=2, Hq=4, Hkv=2, S=60, d=16, seed=0):
    P = np.stack([make_basis(d, 40 + seed, kv) for kv in range(Hkv)])
    q = _rand((B, Hq, d), seed + 1)
    K = _rand((B, Hkv, S, d), seed + 2)
    V = _rand((B, Hkv, S, d), seed + 3)
    return q, P, K, V


def test_all_dims_is_full_rank_loki():
    q, P, K, V = _case()
    d = q.shape[-1]
    s_a = aqua.approx_scores(q, P, K, d)
    s_l = oracle.approx_scores(q, P, K, d)
    assert np.max(np.abs(s_a - s_l)) < 1e-12 * np.max(np.abs(s_l))
    out_a, idx_a = aqua.decode(q, P, K, V, d, 7)
    out_l, idx_l = oracle.decode(q, P, K, V, d, 7)
    assert np.array_equal(idx_a, idx_l)
    assert np.max(np.abs(out_a - out_l)) < 1e-12


def test_query_on_leading_dims_equals_loki():
    B, Hq, Hkv, S, d, r = 1, 2, 1, 80, 16, 5
    P = make_basis(d, 50, 0)[None]
    qr = np.zeros((B, Hq, d))
    qr[..., :r] = _rand((B, Hq, r), 1) + 3.0 * np.sign(_rand((B, Hq, r), 2))  # |.| well above 0
    q = qr @ P[0].T
    K = _rand((B, Hkv, S, d), 3)
    dims = aqua.query_dims(q, P, r)
    assert np.array_equal(dims, np.broadcast_to(np.arange(r), (B, Hq, r)))
    assert np.array_equal(aqua.select(q, P, K, r, 9), oracle.select(q, P, K, r, 9))


def test_invariant_to_basis_column_order():
    q, P, K, V = _case(d=16)
    perm = np.random.default_rng(7).permutation(16)
    Pp, Kp = P[:, :, perm], K[..., perm]
    # the same dimensions (relabelled) are chosen, so the scores are the same
    assert np.max(np.abs(aqua.approx_scores(q, P, K, 5) - aqua.approx_scores(q, Pp, Kp, 5))) < 1e-12
    assert np.array_equal(aqua.select(q, P, K, 5, 8), aqua.select(q, Pp, Kp, 5, 8))
    # Loki's leading-dims scores depend on the column order
    assert np.max(np.abs(oracle.approx_scores(q, P, K, 5) - oracle.approx_scores(q, Pp, Kp, 5))) > 1e-3


@pytest.mark.parametrize("seed", range(6))
def test_dims_maximise_retained_energy_brute_force(seed):
    # a signed-permutation basis keeps the integer query exact after the
    # rotation, so equal magnitudes are exact ties
    d, r = 8, 3
    rng = np.random.default_rng(seed)
    P = np.zeros((1, d, d))
    P[0, np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], size=d)
    q = rng.integers(-3, 4, size=(1, 1, d)).astype(np.float64)
    got = aqua.query_dims(q, P, r)[0, 0]
    qrr = oracle.rotate_queries(q, P)[0, 0]
    best, best_set = -1.0, None
    for I in itertools.combinations(range(d), r):  # lexicographic: lower-index sets first
        e = float(np.sum(qrr[list(I)] ** 2))
        if e > best:
            best, best_set = e, I
    assert tuple(got) == best_set


def test_info_loss_closed_forms():
    d = 4
    P = np.eye(d)[None]
    q = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    assert abs(aqua.info_loss(q, P, np.array([[[0]]]))[0, 0] - 0.4) < 1e-15   # |5 - 3| / 5
    assert aqua.info_loss(q, P, np.array([[[0, 1]]]))[0, 0] == 0.0
    # any orthogonal basis with all dims kept loses nothing
    P2 = make_basis(8, 70, 0)[None]
    q2 = _rand((1, 3, 8), 4)
    assert np.max(aqua.info_loss(q2, P2, np.broadcast_to(np.arange(8), (1, 3, 8)))) < 1e-14
    # magnitude selection loses no more than the leading-dims slice of the same size
    q3 = _rand((2, 4, 16), 5)
    P3 = np.stack([make_basis(16, 71, kv) for kv in range(2)])
    lead = np.broadcast_to(np.arange(6), (2, 4, 6))
    assert np.all(aqua.info_loss(q3, P3, aqua.query_dims(q3, P3, 6)) <= aqua.info_loss(q3, P3, lead) + 1e-15)


def test_per_head_dims_and_group_keys():
    # GQA: each query head of a group uses its own dimensions of the shared keys
    q, P, K, V = _case(B=1, Hq=4, Hkv=1, S=30, d=8)
    s = aqua.approx_scores(q, P, K, 3)
    qr = oracle.rotate_queries(q, P)
    dims = aqua.query_dims(q, P, 3)
    for h in range(4):
        want = np.array([sum(qr[0, h, c] * K[0, 0, j, c] for c in dims[0, h]) for j in range(30)])
        assert np.max(np.abs(s[0, h] - want)) < 1e-12
    assert len({tuple(dims[0, h]) for h in range(4)}) > 1
