"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test names the fact it relies on and the plausible oracle mistakes it
would catch:

* rotation invariance of q.k under an orthogonal basis (AQUA page, appendix
  proof of the lossless rotation) -- catches ``q P^T`` vs ``q P``, a wrong
  projection side, a transposed basis;
* full rank and full k equal dense attention (AQUA page, eqs. 3-5) -- catches
  a wrong softmax scale (sqrt(r) instead of sqrt(d)), softmax over the wrong
  set, values rotated by mistake;
* closed forms for two-token softmax attention -- catches a wrong scale in
  the dense definition itself (which the equivalence tests share);
* brute-force top-k over all subsets on tiny inputs -- catches reversed
  order, wrong tie rule, off-by-one k;
* planted leading/trailing-dimension keys -- catches keeping the trailing
  instead of the leading r dimensions;
* k = 1, constant values, S = 1, softmax weights summing to one;
* GQA equals MHA on a head-repeated cache (the textbook repeat of key/value
  heads) -- catches ``h % G`` instead of ``h // G``;
* a signed permutation basis projects exactly.
"""

import itertools
import math

import numpy as np
import pytest

import oracle
from loki_inputs import make_basis


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- rotation


@pytest.mark.parametrize("d", [2, 16, 64, 128])
def test_rotation_preserves_dot_products(d):
    P = make_basis(d, 77, 0)[None]
    q = _rand((1, 1, d), 1)
    K = _rand((1, 1, 50, d), 2)
    qr = oracle.rotate_queries(q, P)
    Kr = oracle.project(K, P)
    got = Kr[0, 0] @ qr[0, 0]
    want = np.array([float(np.dot(K[0, 0, j], q[0, 0])) for j in range(50)])
    bound = 1e-12 * np.linalg.norm(q) * np.linalg.norm(K[0, 0], axis=1)
    assert np.all(np.abs(got - want) <= bound)


def test_projection_is_row_vector_convention():
    # v_hat = v P: with P the 90-degree rotation [[0,1],[-1,0]], (1,0) maps to (0,1).
    P = np.array([[[0.0, 1.0], [-1.0, 0.0]]])
    K = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    assert np.array_equal(oracle.project(K, P)[0, 0], np.array([[0.0, 1.0], [-1.0, 0.0]]))


def test_signed_permutation_projection_is_exact():
    d = 32
    g = np.random.default_rng(5)
    perm = g.permutation(d)
    sg = g.choice([-1.0, 1.0], size=d)
    P = np.zeros((1, d, d))
    P[0, np.arange(d), perm] = sg
    K = g.standard_normal((1, 1, 40, d))
    Kr = oracle.project(K, P)
    for i in range(d):
        assert np.array_equal(Kr[0, 0, :, perm[i]], sg[i] * K[0, 0, :, i])


# ---------------------------------------------------------------- dense closed forms


def test_dense_two_token_closed_form():
    # q = (a, 0), keys e0 and e1: scores a and 0, scaled by 1/sqrt(2);
    # softmax of two numbers is the logistic function.
    a = 1.7
    q = np.array([[[a, 0.0]]])
    K = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    V = np.array([[[[3.0, -1.0], [0.5, 2.0]]]])
    w0 = 1.0 / (1.0 + math.exp(-a / math.sqrt(2.0)))
    want = w0 * V[0, 0, 0] + (1 - w0) * V[0, 0, 1]
    assert np.allclose(oracle.dense(q, K, V)[0, 0], want, rtol=0, atol=1e-15)


def test_dense_equal_scores_average_values():
    q = np.zeros((1, 1, 4))
    K = _rand((1, 1, 7, 4), 3)
    V = _rand((1, 1, 7, 4), 4)
    assert np.allclose(oracle.dense(q, K, V)[0, 0], V[0, 0].mean(axis=0), atol=1e-15)


# ---------------------------------------------------------------- equivalence with dense


@pytest.mark.parametrize("G", [1, 4])
def test_full_rank_full_k_equals_dense(G):
    B, Hkv, S, d = 2, 2, 37, 16
    Hq = Hkv * G
    P = np.stack([make_basis(d, 11, kv) for kv in range(Hkv)])
    q = _rand((B, Hq, d), 6)
    K = _rand((B, Hkv, S, d), 7)
    V = _rand((B, Hkv, S, d), 8)
    out, idx = oracle.decode(q, P, oracle.project(K, P), V, r=d, k=S)
    assert np.array_equal(idx, np.broadcast_to(np.arange(S), (B, Hq, S)))
    assert np.max(np.abs(out - oracle.dense(q, K, V))) <= 1e-12


@pytest.mark.parametrize("r", [1, 5, 8])
def test_full_k_equals_dense_for_any_rank(r):
    B, Hkv, G, S, d = 1, 2, 2, 29, 16
    P = np.stack([make_basis(d, 12, kv) for kv in range(Hkv)])
    q = _rand((B, Hkv * G, d), 9)
    K = _rand((B, Hkv, S, d), 10)
    V = _rand((B, Hkv, S, d), 11)
    out, _ = oracle.decode(q, P, oracle.project(K, P), V, r=r, k=S)
    assert np.max(np.abs(out - oracle.dense(q, K, V))) <= 1e-12


def test_full_rank_selection_is_exact_top_k():
    # With r = d the approximate scores are the exact q.k (rotation invariance),
    # so the kept set is the top-k of scores computed on the UNROTATED cache.
    d, S, k = 16, 60, 9
    P = make_basis(d, 13, 0)[None]
    q = _rand((1, 1, d), 12)
    K = _rand((1, 1, S, d), 13)
    idx = oracle.select(q, P, oracle.project(K, P), r=d, k=k)
    exact = K[0, 0] @ q[0, 0]
    want = sorted(sorted(range(S), key=lambda j: -exact[j])[:k])
    assert list(idx[0, 0]) == want


# ---------------------------------------------------------------- selection


def _brute_topk(s, k):
    """Lexicographically smallest index set among the k-subsets of maximum sum."""
    best = None
    for c in itertools.combinations(range(len(s)), k):
        key = (-sum(int(s[j]) for j in c), c)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_brute_force_with_ties(seed):
    g = np.random.default_rng(100 + seed)
    S = int(g.integers(1, 11))
    k = int(g.integers(1, S + 1))
    s = g.integers(-2, 3, size=S).astype(np.float64)  # integers: many exact ties
    got = list(oracle.topk_indices(s, k))
    assert got == _brute_topk(s, k)
    # and against a full sort by (score desc, index asc)
    assert got == sorted(sorted(range(S), key=lambda j: (-s[j], j))[:k])


def test_topk_all_equal_takes_lowest_indices():
    s = np.full(10, 3.0)
    assert list(oracle.topk_indices(s, 4)) == [0, 1, 2, 3]


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([-0.0, 0.0, -0.0, -1.0])
    assert list(oracle.topk_indices(s, 2)) == [0, 1]


def test_selection_uses_leading_dimensions():
    # P = I and q = e0: the leading-r score of token j is K[j, 0].  The
    # trailing dimensions hold huge values ranking tokens in the opposite order,
    # so keeping the trailing (or all) dimensions picks a different set.
    d, S, r, k = 8, 20, 2, 5
    P = np.eye(d)[None]
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    q[0, 0, d - 1] = 1.0
    K = np.zeros((1, 1, S, d))
    K[0, 0, :, 0] = np.arange(S)               # leading: token S-1 best
    K[0, 0, :, d - 1] = -1000.0 * np.arange(S)  # trailing: token 0 best
    idx = oracle.select(q, P, K, r=r, k=k)
    assert list(idx[0, 0]) == list(range(S - k, S))


def test_select_returns_ascending_distinct():
    q = _rand((2, 4, 16), 20)
    P = np.stack([make_basis(16, 14, kv) for kv in range(2)])
    K = _rand((2, 2, 100, 16), 21)
    idx = oracle.select(q, P, K, r=4, k=17)
    assert idx.shape == (2, 4, 17)
    assert np.all(np.diff(idx, axis=-1) > 0)


# ---------------------------------------------------------------- attention


def test_weights_sum_to_one():
    q = _rand((1, 2, 16), 30)
    P = make_basis(16, 15, 0)[None]
    K = _rand((1, 1, 64, 16), 31) * 5.0
    V = _rand((1, 1, 64, 16), 32)
    idx = oracle.select(q, P, K, r=4, k=13)
    _, w = oracle.attend(q, P, K, V, idx, return_weights=True)
    assert np.all(w > 0)
    assert np.all(np.abs(w.sum(axis=-1) - 1.0) <= 1e-14)


def test_k_equals_one_returns_value_of_best_token():
    q = _rand((1, 1, 16), 33)
    P = make_basis(16, 16, 0)[None]
    K = _rand((1, 1, 64, 16), 34)
    V = _rand((1, 1, 64, 16), 35)
    out, idx = oracle.decode(q, P, K, V, r=3, k=1)
    s = oracle.approx_scores(q, P, K, 3)[0, 0]
    j = int(np.argmax(s))
    assert idx[0, 0, 0] == j
    assert np.array_equal(out[0, 0], V[0, 0, j])


def test_constant_values_give_that_value():
    q = _rand((1, 1, 16), 36)
    P = make_basis(16, 17, 0)[None]
    K = _rand((1, 1, 40, 16), 37)
    row = _rand(16, 38)
    V = np.broadcast_to(row, (1, 1, 40, 16)).copy()
    out, _ = oracle.decode(q, P, K, V, r=4, k=11)
    assert np.max(np.abs(out[0, 0] - row)) <= 1e-15


def test_single_token_cache():
    q = _rand((1, 1, 8), 39)
    P = make_basis(8, 18, 0)[None]
    K = _rand((1, 1, 1, 8), 40)
    V = _rand((1, 1, 1, 8), 41)
    out, idx = oracle.decode(q, P, K, V, r=2, k=1)
    assert idx.tolist() == [[[0]]]
    assert np.array_equal(out[0, 0], V[0, 0, 0])


def test_gqa_equals_mha_on_repeated_cache():
    B, Hkv, G, S, d = 2, 3, 4, 50, 16
    Hq = Hkv * G
    P = np.stack([make_basis(d, 19, kv) for kv in range(Hkv)])
    q = _rand((B, Hq, d), 42)
    K = _rand((B, Hkv, S, d), 43)
    V = _rand((B, Hkv, S, d), 44)
    # textbook repeat of key/value heads: head h of the repeated cache is kv head h // G
    Krep = np.repeat(K, G, axis=1)
    Vrep = np.repeat(V, G, axis=1)
    Prep = np.repeat(P, G, axis=0)
    o1, i1 = oracle.decode(q, P, K, V, r=5, k=9)
    o2, i2 = oracle.decode(q, Prep, Krep, Vrep, r=5, k=9)
    assert np.array_equal(i1, i2)
    assert np.array_equal(o1, o2)


def test_attend_closed_form_two_kept_tokens():
    # 45-degree basis, r = 1: the approximate score of key (x, y) is
    # (x + y)(q0 + q1)/2, so with q = (1, 1) the kept set is the two keys with
    # the largest x + y; exact scores are q.k / sqrt(2).
    c = 1.0 / math.sqrt(2.0)
    P = np.array([[[c, -c], [c, c]]])
    q = np.array([[[1.0, 1.0]]])
    K = np.array([[[[2.0, 0.0], [0.0, -1.0], [1.0, 2.0], [-3.0, 0.5]]]])
    V = np.array([[[[1.0, 0.0], [5.0, 5.0], [0.0, 1.0], [7.0, 7.0]]]])
    out, idx = oracle.decode(q, P, oracle.project(K, P), V, r=1, k=2)
    assert idx.tolist() == [[[0, 2]]]
    e0, e2 = 2.0 / math.sqrt(2.0), 3.0 / math.sqrt(2.0)
    w0 = 1.0 / (1.0 + math.exp(e2 - e0))
    want = np.array([w0, 1.0 - w0])
    assert np.max(np.abs(out[0, 0] - want)) <= 1e-15


# ---------------------------------------------------------------- ragged batches
# decode_varlen: each sequence of a batch is a decode over its own prefix of
# the cache (the AQUA page's eqs. 1-5 on a cache of that many tokens).


def test_varlen_keeping_everything_is_dense_on_each_prefix():
    # k >= len_b: sequence b is dense attention over its first len_b tokens of
    # the UNROTATED cache (eqs. 3-5 on the prefix); idx lists them, then -1.
    # Catches attending over the whole capacity and wrong padding.
    B, Hkv, G, S, d = 3, 2, 2, 20, 16
    P = np.stack([make_basis(d, 31, kv) for kv in range(Hkv)])
    q = _rand((B, Hkv * G, d), 40)
    K = _rand((B, Hkv, S, d), 41)
    V = _rand((B, Hkv, S, d), 42)
    lens = [5, 20, 1]
    k = 20
    out, idx = oracle.decode_varlen(q, P, oracle.project(K, P), V, lens, r=4, k=k)
    for b, L in enumerate(lens):
        want = oracle.dense(q[b:b + 1], K[b:b + 1, :, :L], V[b:b + 1, :, :L])[0]
        assert np.max(np.abs(out[b] - want)) <= 1e-12
        assert np.array_equal(idx[b, :, :L], np.broadcast_to(np.arange(L), (Hkv * G, L)))
        assert np.all(idx[b, :, L:] == -1)


def test_varlen_ignores_rows_past_each_end():
    # rows past a sequence's length are unused capacity: filling them with
    # huge values changes nothing.  Catches scoring or attending past the end.
    B, Hkv, G, S, d = 2, 1, 3, 40, 16
    P = np.stack([make_basis(d, 32, kv) for kv in range(Hkv)])
    q = _rand((B, Hkv * G, d), 43)
    Kr = oracle.project(_rand((B, Hkv, S, d), 44), P)
    V = _rand((B, Hkv, S, d), 45)
    lens = [17, 33]
    out1, idx1 = oracle.decode_varlen(q, P, Kr, V, lens, r=5, k=6)
    Kr2, V2 = Kr.copy(), V.copy()
    for b, L in enumerate(lens):
        Kr2[b, :, L:] = 1e6 * _rand(Kr2[b, :, L:].shape, 46 + b)
        V2[b, :, L:] = -1e6
    out2, idx2 = oracle.decode_varlen(q, P, Kr2, V2, lens, r=5, k=6)
    assert np.array_equal(idx1, idx2)
    assert np.array_equal(out1, out2)


def test_varlen_selection_is_brute_force_top_k_of_the_prefix():
    # tiny prefix: the kept set is the subset of the prefix with the largest
    # sum of leading-r scores (ties to lower indices), found by enumeration,
    # with scores computed here from the definition q_rot[:r] . K_rot[j, :r]
    d, r, S, L, k = 8, 3, 12, 7, 3
    P = make_basis(d, 33, 0)[None]
    q = _rand((1, 1, d), 47)
    Kr = oracle.project(_rand((1, 1, S, d), 48), P)
    Kr[0, 0, 2, :r] = Kr[0, 0, 5, :r]  # a planted exact tie inside the prefix
    qr = q[0, 0] @ P[0]
    s = [float(qr[:r] @ Kr[0, 0, j, :r]) for j in range(L)]
    best = max(itertools.combinations(range(L), k), key=lambda c: (sum(s[j] for j in c), [-j for j in c]))
    _, idx = oracle.decode_varlen(q, P, Kr, _rand((1, 1, S, d), 49), [L], r=r, k=k)
    assert list(idx[0, 0]) == sorted(best)


def test_varlen_full_lengths_equal_decode_and_lengths_are_clamped():
    B, Hkv, G, S, d = 2, 2, 2, 25, 16
    P = np.stack([make_basis(d, 34, kv) for kv in range(Hkv)])
    q = _rand((B, Hkv * G, d), 50)
    Kr = oracle.project(_rand((B, Hkv, S, d), 51), P)
    V = _rand((B, Hkv, S, d), 52)
    out, idx = oracle.decode(q, P, Kr, V, r=4, k=6)
    out2, idx2 = oracle.decode_varlen(q, P, Kr, V, [S, S + 100], r=4, k=6)
    assert np.array_equal(idx, idx2) and np.max(np.abs(out - out2)) <= 1e-12
    out3, idx3 = oracle.decode_varlen(q, P, Kr, V, [0, -5], r=4, k=6)  # clamped to one token
    assert np.all(idx3[:, :, 0] == 0) and np.all(idx3[:, :, 1:] == -1)
    assert np.max(np.abs(out3 - V[:, np.repeat(np.arange(Hkv), G), 0])) <= 1e-15
