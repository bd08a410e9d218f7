"""GPU parity of the basis calibration (loki_calibrate_pca) through the C ABI.

The oracle is the SVD of each key head's rows in float64.  The GPU forms the
Gram matrix A^T A and diagonalises it by Jacobi in fp64, so the two differ by
the Gram matrix's accumulation error E and the eigensolver's rounding:

* bf16 keys: products are exact and at most 256 of them are summed in fp32
  before the fp64 sum, so |E_ij| <= 512 * 2^-24 * sum_n |a_ni a_nj|
  (conservative: at most 256 + 32 roundings, each at most 2^-24 of the
  partial sum's magnitude); fp32 keys: exact products, fp64 sums over B*S
  rows, |E_ij| <= 4 B S 2^-53 sum_n |a_ni a_nj|;
* the fp64 Jacobi sweeps add at most 1e-12 * lambda_max (a few hundred
  roundings of 2^-53 per entry).

Eigenvalues must agree within ||E||_F + 1e-12 lambda_max (Weyl).  An
eigenvector whose eigenvalue is separated from its neighbours by a gap g >
4 e (e that bound) is determined up to sign, with sin(angle) <= e / (g - e)
(Davis-Kahan); such columns must agree entry-wise within twice that plus the
output rounding.  The other columns are checked only as part of an
orthonormal basis.  Closed forms pin the GPU directly: axis-aligned keys give
an exact permutation basis, zero keys the identity, keys drawn in a known
basis give that basis back.
"""

import numpy as np
import pytest
import torch

import oracle
from loki_inputs import CONFIGS, make_basis, make_inputs

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
OUT_ROUND = {"f32": 2.0 ** -23, "bf16": 2.0 ** -8}


def dev(t):
    return t.to("cuda")


def _rows(K, kv):
    return np.concatenate([K[b, kv].double().numpy() for b in range(K.shape[0])])


def check_against_oracle(K, P_g, lam_g, dt, heads=None):
    """Compare the GPU result with the oracle on the given heads (all by default)."""
    P_g = P_g.double().cpu().numpy()
    lam_g = lam_g.cpu().numpy()
    B, Hkv, S, d = K.shape
    heads = range(Hkv) if heads is None else heads
    gamma = 512 * 2.0 ** -24 if dt == "bf16" else 4 * B * S * 2.0 ** -53
    determined = 0
    for kv in heads:
        P_o, lam_o = oracle.calibrate(K[:, kv:kv + 1])
        P_o, lam_o = P_o[0], lam_o[0]
        A = _rows(K, kv)
        absA = np.abs(A)
        e = gamma * np.linalg.norm(absA.T @ absA) + 1e-12 * lam_o[0]
        assert np.all(np.abs(lam_g[kv] - lam_o) <= e), np.max(np.abs(lam_g[kv] - lam_o))
        assert np.all(np.diff(lam_g[kv]) <= 0)
        # orthonormal basis, every column
        G = P_g[kv].T @ P_g[kv]
        assert np.max(np.abs(G - np.eye(d))) <= 4 * d * OUT_ROUND[dt] + 1e-12
        # sign convention on the GPU's own output
        assert np.all(P_g[kv].max(axis=0) >= -P_g[kv].min(axis=0))
        for j in range(d):
            gap = min(abs(lam_o[j] - lam_o[i]) for i in (j - 1, j + 1) if 0 <= i < d)
            if gap <= 4 * e:
                continue
            sin = e / (gap - e)
            pg, po = P_g[kv][:, j], P_o[:, j]
            s = 1.0 if pg @ po >= 0 else -1.0
            assert np.max(np.abs(s * pg - po)) <= 2 * sin + 2 * OUT_ROUND[dt], (kv, j)
            # both sides follow the same sign rule: they agree wherever the
            # oracle's largest entry stands clear of the runner-up
            top = np.sort(np.abs(po))[::-1]
            if top[0] - top[1] > 4 * sin + 4 * OUT_ROUND[dt]:
                assert s > 0, (kv, j)
            determined += 1
    return determined


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_calibrate_matches_oracle(gpu_lib, dt, d):
    # keys with a decaying spectrum in a random basis; B*S = 2000 rows per
    # head: eight Gram blocks with a ragged last one
    cfg = CONFIGS["C1"].replace(B=2, Hq=2, Hkv=2, d=d, S=1000, r=16, k=64, dtype=dt, tau=8.0)
    K = make_inputs(cfg, need_K=True)["K"]
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    assert P_g.dtype == TDT[dt] and lam_g.dtype == torch.float64
    n = check_against_oracle(K, P_g, lam_g, dt)
    assert n >= 2 * 16  # at least the leading r columns of both heads are pinned


def test_calibrate_axis_aligned_keys_give_a_permutation(gpu_lib):
    # every key row is a unit vector along one coordinate axis, axis j holding
    # w_j rows (w a permutation of 1..d, rows shuffled over both batch
    # elements): A^T A = diag(w) exactly, so the basis is the permutation that
    # orders the axes by decreasing w, exactly
    d, Hkv, B = 64, 2, 2
    S = d * (d + 1) // 2 // B
    rng = np.random.default_rng(21)
    K = np.zeros((B, Hkv, S, d))
    for kv in range(Hkv):
        w = rng.permutation(d) + 1
        axis = rng.permutation(np.repeat(np.arange(d), w))
        rows = np.zeros((B * S, d))
        rows[np.arange(B * S), axis] = 1.0
        K[:, kv] = rows.reshape(B, S, d)
    for dt in ("f32", "bf16"):
        Kt = torch.from_numpy(K).to(TDT[dt])
        P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(Kt))
        torch.cuda.synchronize()
        for kv in range(Hkv):
            diag = (K[:, kv] ** 2).sum(axis=(0, 1))
            assert len(set(diag.tolist())) == d  # distinct: the order is unique
            order = np.argsort(-diag, kind="stable")
            want = np.zeros((d, d))
            want[order, np.arange(d)] = 1.0
            assert np.array_equal(P_g[kv].double().cpu().numpy(), want)
            assert np.array_equal(lam_g[kv].cpu().numpy(), diag[order])
        P_o, lam_o = oracle.calibrate(Kt)
        assert np.max(np.abs(P_o - P_g.double().cpu().numpy())) < 1e-12


def test_calibrate_zero_keys_give_the_identity(gpu_lib):
    K = torch.zeros((1, 3, 100, 128), dtype=torch.bfloat16)
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    for kv in range(3):
        assert torch.equal(P_g[kv].cpu().float(), torch.eye(128))
    assert torch.all(lam_g == 0)


def test_calibrate_fewer_rows_than_dims(gpu_lib):
    # 20 key rows in 64 dims: 20 determined directions, the rest an
    # orthonormal completion
    cfg = CONFIGS["C1"].replace(B=1, Hq=1, Hkv=1, d=64, S=20, r=8, k=4, dtype="f32", tau=8.0)
    K = make_inputs(cfg, need_K=True)["K"]
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    check_against_oracle(K, P_g, lam_g, "f32")
    assert np.all(np.abs(lam_g[0, 20:].cpu().numpy()) <= 1e-9 * float(lam_g[0, 0]))


def test_calibrate_recovers_the_generating_basis(gpu_lib):
    # keys z * exp(-j/4) in a known basis P0: the leading directions come back
    # (a fact about the data, independent of the oracle)
    d, n, r = 128, 32768, 8
    P0 = make_basis(d, 31, 0)
    Z = np.random.default_rng(22).standard_normal((n, d)) * np.exp(-np.arange(d) / 4.0)
    K = torch.from_numpy((Z @ P0.T).reshape(4, 1, n // 4, d)).to(torch.bfloat16)
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    cos = np.abs(np.sum(P_g[0].double().cpu().numpy()[:, :r] * P0[:, :r], axis=0))
    assert np.all(cos > 0.99), cos
    want = (1 - np.exp(-2 * r / 4.0)) / (1 - np.exp(-2 * d / 4.0))
    got = float(lam_g[0, :r].sum() / lam_g[0].sum())
    assert abs(got - want) < 0.01 * want


def test_calibrate_is_deterministic_and_takes_a_workspace(gpu_lib):
    cfg = CONFIGS["C1"].replace(B=3, Hq=2, Hkv=2, d=128, S=777, r=16, k=64, dtype="bf16", tau=12.0)
    K = dev(make_inputs(cfg, need_K=True)["K"])
    P1, l1 = gpu_lib.loki_calibrate_pca(K)
    ws = torch.empty(gpu_lib.loki_calibrate_workspace_bytes(3, 2, 777, 128), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # stale contents must not matter
    P2, l2 = gpu_lib.loki_calibrate_pca(K, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(P1.view(torch.int16), P2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.slow
def test_calibrate_full_c5_cache(gpu_lib):
    # the prefill-plus-decode workload's whole key cache (4 x 8 heads x 32768
    # tokens, bf16): every head is an orthonormal, decreasing basis; two heads
    # are compared with the oracle
    cfg = CONFIGS["C5"]
    K = make_inputs(cfg, need_K=True)["K"]
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    Pd = P_g.double().cpu().numpy()
    for kv in range(cfg.Hkv):
        assert np.max(np.abs(Pd[kv].T @ Pd[kv] - np.eye(cfg.d))) <= 4 * cfg.d * OUT_ROUND["bf16"]
        assert np.all(np.diff(lam_g[kv].cpu().numpy()) <= 0)
    n = check_against_oracle(K, P_g, lam_g, "bf16", heads=[0, cfg.Hkv - 1])
    # the flat noisy spectrum (tau = 24, noise 0.05) leaves fewer columns
    # separated by more than the conservative bound: at least r of the two
    # heads' columns are still pinned
    assert n >= cfg.r
    # every head's leading r columns as a subspace (what the scores use: q
    # P_r P_r^T k), with no column matching: by Ky Fan, the energy of the
    # exact Gram C captured by an orthonormal r-frame is at most the sum of
    # its r largest eigenvalues, with equality on the top-r subspace only.
    # The GPU's frame solves C + E (||E||_2 <= e): it loses at most 2 r e,
    # and its bf16 rounding (2^-9 per entry) a second-order r 2^-18 lambda_0
    # (doubled below)
    gamma = 512 * 2.0 ** -24
    B, Hkv, S, d = K.shape
    for kv in range(cfg.Hkv):
        A = _rows(K, kv)
        C = A.T @ A
        lam = np.linalg.eigvalsh(C)[::-1]
        absA = np.abs(A)
        e = gamma * np.linalg.norm(absA.T @ absA) + 1e-12 * lam[0]
        Q, _ = np.linalg.qr(Pd[kv][:, :cfg.r])
        loss = lam[:cfg.r].sum() - np.trace(Q.T @ C @ Q)
        assert -1e-9 * lam[0] <= loss <= 2 * cfg.r * e + cfg.r * 2.0 ** -17 * lam[0], (kv, loss / lam[0])


def test_calibrate_full_c5_cache_f32(gpu_lib):
    # the same cache's values in fp32 (exact copies of the bf16 keys): the
    # fp64 Gram's bound is tight enough to pin every column of every head
    # against the oracle, which fixes the eigensolver over the whole basis
    cfg = CONFIGS["C5"]
    K = make_inputs(cfg, need_K=True)["K"].float()
    P_g, lam_g = gpu_lib.loki_calibrate_pca(dev(K))
    torch.cuda.synchronize()
    assert P_g.dtype == torch.float32
    n = check_against_oracle(K, P_g, lam_g, "f32")
    assert n == cfg.Hkv * cfg.d
