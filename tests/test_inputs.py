"""The seeded input generator: shapes, reproducibility, basis, spectra."""

import numpy as np
import pytest
import torch

from loki_inputs import CONFIGS, make_basis, make_inputs, make_integer_inputs, spectrum


def _small(name):
    cfg = CONFIGS[name]
    return cfg.scaled(S=min(cfg.S, 512), B=min(cfg.B, 2))


@pytest.mark.parametrize("name", list(CONFIGS))
def test_shapes_and_dtypes(name):
    cfg = _small(name)
    x = make_inputs(cfg, need_K=True)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    assert x["q"].shape == (cfg.B, cfg.Hq, cfg.d) and x["q"].dtype == dt
    assert x["P"].shape == (cfg.Hkv, cfg.d, cfg.d) and x["P"].dtype == dt
    for key in ("K_rot", "V", "K"):
        assert x[key].shape == (cfg.B, cfg.Hkv, cfg.S, cfg.d) and x[key].dtype == dt
    assert 1 <= cfg.k <= cfg.S and 1 <= cfg.r <= cfg.d


def test_reproducible_and_seed_sensitive():
    cfg = _small("C3")
    a, b = make_inputs(cfg), make_inputs(cfg)
    c = make_inputs(cfg, seed=1)
    for key in ("q", "P", "K_rot", "V"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])


@pytest.mark.parametrize("d", [64, 128])
def test_basis_orthonormal_with_positive_r_diagonal(d):
    P = make_basis(d, 3, 5)
    assert np.max(np.abs(P.T @ P - np.eye(d))) < 1e-12
    # Q R = A with diag(R) > 0 means R = Q^T A has a positive diagonal
    a = np.random.default_rng(np.random.SeedSequence([0x4C4F4B49, 3, 0, 0, 5, 0])).standard_normal((d, d))
    assert np.all(np.diag(P.T @ a) > 0)


@pytest.mark.parametrize("name", ["C1", "C3", "C4", "C5"])
def test_leading_energy_matches_closed_form(name):
    # E|K_rot[:, :r]|^2 / E|K_rot|^2 = (1 - e^{-2r/tau}) / (1 - e^{-2d/tau})
    # (geometric sums of the spectrum's variances), before any noise.
    cfg = CONFIGS[name].scaled(S=4096, B=1).replace(noise=0.0, heavy=0)
    x = make_inputs(cfg)
    kr = x["K_rot"][0, 0].double().numpy()
    share = np.sum(kr[:, :cfg.r] ** 2) / np.sum(kr ** 2)
    t = cfg.tau
    want = (1 - np.exp(-2 * cfg.r / t)) / (1 - np.exp(-2 * cfg.d / t))
    assert abs(share - want) < 0.03 * want


def test_keys_consistent_with_rotated_keys():
    cfg = _small("C5")
    x = make_inputs(cfg, need_K=True)
    K = x["K"][1, 3].double().numpy()
    Kr = x["K_rot"][1, 3].double().numpy()
    err = np.linalg.norm(K @ x["P64"][3] - Kr) / np.linalg.norm(Kr)
    assert err < 1e-2  # two bf16 roundings


def test_heavy_tokens_score_high():
    cfg = CONFIGS["C4"].scaled(S=16384, heavy=64)
    x = make_inputs(cfg)
    G = cfg.G
    hv = x["heavy_idx"]
    assert hv.shape == (1, cfg.Hq, 64)
    q = x["q"].double().numpy()
    for h in (0, 5, 31):
        kv = h // G
        K = x["K_rot"][0, kv].double().numpy() @ x["P64"][kv].T  # back to the original basis
        s = K @ q[0, h]
        top = set(np.argsort(-s)[: cfg.k].tolist())
        assert len(top & set(hv[0, h].tolist())) >= 60


def test_integer_inputs_are_exact():
    x = make_integer_inputs(1, 2, 1, 16, 33, "bf16")
    for key in ("q", "K_rot", "V", "P"):
        v = x[key].double()
        assert torch.equal(v, v.round())


def test_spectrum_values():
    cfg = CONFIGS["C1"]
    s = spectrum(cfg)
    assert s[0] == 1.0 and abs(s[8] - np.exp(-1.0)) < 1e-15
