"""The float64 oracle against the hand-worked examples in tests/golden/.

Each fixture cites the definition it works through and derives its expected
values by exact arithmetic (see the fixture's "derivation"); nothing in them
comes from the oracle or from the GPU library.  Integer results (index sets,
chosen dims) must match exactly, real ones to within float64 rounding.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import aqua, asym

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        fx = json.load(fh)
    assert fx["cite"] and fx["derivation"]
    return fx


def arr(x):
    return np.asarray(x, dtype=np.float64)


def test_every_fixture_is_checked():
    names = sorted(n for n in os.listdir(GOLDEN) if n.endswith(".json"))
    assert names == sorted(FIXTURES)


def check_leading_dims(fx):
    i, e = fx["inputs"], fx["expected"]
    q, P, Kr, V = (arr(i[n]) for n in ("q", "P", "K_rot", "V"))
    s = oracle.approx_scores(q, P, Kr, i["r"])
    assert np.array_equal(s, arr(e["approx_scores"]))
    out, idx = oracle.decode(q, P, Kr, V, i["r"], i["k"])
    assert np.array_equal(idx, np.asarray(e["idx"]))
    assert np.max(np.abs(out - arr(e["out"]))) <= 1e-14


def check_gqa(fx):
    i, e = fx["inputs"], fx["expected"]
    q, P, Kr, V = (arr(i[n]) for n in ("q", "P", "K_rot", "V"))
    out, idx = oracle.decode(q, P, Kr, V, i["r"], i["k"])
    assert np.array_equal(idx, np.asarray(e["idx"]))
    assert np.array_equal(out, arr(e["out"]))  # one kept token: weight exactly 1


def check_aqua(fx):
    i, e = fx["inputs"], fx["expected"]
    q, P, Kr = (arr(i[n]) for n in ("q", "P", "K_rot"))
    dims = aqua.query_dims(q, P, i["r"])
    assert np.array_equal(dims, np.asarray(e["dims"]))
    loss = aqua.info_loss(q, P, dims)
    want = 1.0 - math.sqrt(e["norm_sq_kept"] / e["norm_sq_all"])
    assert abs(float(loss[0, 0]) - want) <= 1e-15
    assert np.array_equal(aqua.approx_scores(q, P, Kr, i["r"]), arr(e["approx_scores"]))
    assert np.array_equal(aqua.select(q, P, Kr, i["r"], i["k"]), np.asarray(e["idx"]))
    assert np.array_equal(oracle.select(q, P, Kr, i["r"], i["k"]), np.asarray(e["idx_leading_dims"]))


def check_calibrate(fx):
    P, lam = oracle.calibrate(arr(fx["inputs"]["K"]))
    e = fx["expected"]
    assert np.max(np.abs(P - arr(e["P"]))) <= 1e-15
    assert np.max(np.abs(lam - arr(e["eigvals"]))) <= 1e-14


def check_saki(fx):
    i, e = fx["inputs"], fx["expected"]
    Cq, Ck = arr(i["Cq"]), arr(i["Ck"])
    A, B = asym.saki_factors(Cq, Ck, i["r"])
    assert np.max(np.abs(A @ B.T - arr(e["M"]))) <= 1e-14
    assert np.max(np.abs(A.T ** 4 - arr(e["A_columns_pow4"]))) <= 1e-13
    assert np.max(np.abs(B.T ** 4 - arr(e["B_columns_pow4"]))) <= 1e-13
    assert abs(asym.distortion(Cq, Ck, A @ B.T) - e["distortion"]) <= 1e-12


FIXTURES = {
    "loki_leading_dims_ties.json": check_leading_dims,
    "gqa_two_query_heads.json": check_gqa,
    "aqua_query_magnitude_dims.json": check_aqua,
    "calibrate_axis_keys.json": check_calibrate,
    "saki_diagonal_moments.json": check_saki,
}


@pytest.mark.parametrize("name", sorted(FIXTURES))
def test_oracle_matches_worked_example(name):
    FIXTURES[name](load(name))
