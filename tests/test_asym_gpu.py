"""GPU parity of the decode step with an asymmetric scoring index
(loki_decode_asym) against the float64 oracle (oracle.asym), through the C ABI.

The query-side matrix A and key-side matrix B come from the oracle's
closed-form calibration on seeded query samples and the keys; both are
rounded once to the cache dtype, and the key index K_idx = (K B)[..., :R] is
formed by the oracle and rounded the same way, so both sides consume the same
stored values (as the rotated cache is shared by the leading-dims decode).
The scores are computed as for the leading-dims decode with A in place of
the basis, so the same rules apply: kept sets bit-exact outside the 1e-4 tie
band, outputs within 1e-5 (fp32) / 2e-2 (bf16).  The GPU's index projection
(loki_project_keys_lead with K_rot = NULL) is checked separately against the
oracle's projection.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import asym
from loki_inputs import CONFIGS, make_inputs, make_query_samples
from parity_helpers import OUT_TOL, check_band_rows, check_index_sets, max_abs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(t):
    return t.to("cuda")


def asym_inputs(cfg, n_q=256):
    x = make_inputs(cfg, need_K=True)
    qs = make_query_samples(cfg, n_q)
    A, Bm = asym.calibrate(qs, x["K"], cfg.r)
    d = cfg.d
    R = cfg.r
    Ap = np.zeros((cfg.Hkv, d, d))
    Bp = np.zeros((cfg.Hkv, d, d))
    Ap[:, :, :cfg.r] = A
    Bp[:, :, :cfg.r] = Bm
    tdt = TDT[cfg.dtype]
    A_t = torch.from_numpy(Ap).to(tdt)
    B_t = torch.from_numpy(Bp).to(tdt)
    K_idx = torch.from_numpy(oracle.project(x["K"], B_t)[..., :R].copy()).to(tdt)
    return x, A_t, B_t, K_idx


def run_asym(rks, x, A_t, K_idx, r, k, lens=None):
    q, K, V = dev(x["q"]), dev(x["K"]), dev(x["V"])
    lens_d = None if lens is None else dev(torch.tensor(lens, dtype=torch.int32))
    out_g, idx_g = rks.loki_decode_asym(q, dev(A_t), dev(K_idx), K, V, r, k, lens=lens_d)
    torch.cuda.synchronize()
    B, Hq, d = x["q"].shape
    S = x["K"].shape[2]
    ig = idx_g.cpu().numpy().astype(np.int64)
    og = out_g.double().cpu().numpy()
    tol = OUT_TOL[x["q"].dtype]
    eye = np.broadcast_to(np.eye(d), (x["K"].shape[1], d, d))
    for b in range(B):
        L = S if lens is None else min(max(int(lens[b]), 1), S)
        kb = min(k, L)
        idx_o, s_o = asym.select(x["q"][b:b + 1], A_t, K_idx[b:b + 1, :, :L], r, kb, return_scores=True)
        out_o = oracle.attend(x["q"][b:b + 1], eye, x["K"][b:b + 1, :, :L], x["V"][b:b + 1, :, :L], idx_o)
        assert np.all(ig[b, :, kb:] == -1)
        differ = check_index_sets(ig[b:b + 1, :, :kb], idx_o, s_o, kb)
        same = np.ones(Hq, dtype=bool)
        for _, h in differ:
            same[h] = False
        if same.any():
            assert np.max(np.abs(og[b] - out_o[0])[same]) <= tol, b
        # band rows: the oracle's exact attention (query and keys themselves)
        # over the GPU's own kept set
        check_band_rows(og[b:b + 1], ig[b:b + 1, :, :kb], differ, x["q"][b:b + 1], eye,
                        x["K"][b:b + 1, :, :L], x["V"][b:b + 1, :, :L], tol)
    return out_g, idx_g


CASES = {
    "pair_fused": CONFIGS["C3"].scaled(S=2048, B=16),      # rotation + scores + selection per pair of heads
    "two_kernel": CONFIGS["C3"].scaled(S=4096, B=2),
    "mha_fused": CONFIGS["C2"].scaled(S=2048, B=8),
    "r64": CONFIGS["C5"].scaled(S=4096, B=1),
    "f32": CONFIGS["C1"].replace(B=2, Hq=4, Hkv=2),
    # heads over 32768 tokens: two-stage selection over 16384-token chunks,
    # with the first stage in its own kernel (96 head x chunk blocks) and
    # fused with the scores (288 blocks)
    "long_chunked": CONFIGS["C4"].scaled(S=40000),
    "long_chunked_fused": CONFIGS["C4"].scaled(S=40000, B=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_asym_decode_matches_oracle(gpu_lib, name):
    cfg = CASES[name]
    x, A_t, _, K_idx = asym_inputs(cfg)
    run_asym(gpu_lib, x, A_t, K_idx, cfg.r, cfg.k)


def test_asym_ragged_batch(gpu_lib):
    cfg = CONFIGS["C3"].scaled(S=2048, B=5)
    x, A_t, _, K_idx = asym_inputs(cfg)
    lens = [2048, 600, 1, cfg.k - 5, 1777]
    run_asym(gpu_lib, x, A_t, K_idx, cfg.r, cfg.k, lens=lens)


def test_asym_keep_all_is_dense_attention(gpu_lib):
    cfg = CONFIGS["C3"].scaled(S=512, B=2).replace(k=512)
    x, A_t, _, K_idx = asym_inputs(cfg)
    out_g, _ = gpu_lib.loki_decode_asym(dev(x["q"]), dev(A_t), dev(K_idx), dev(x["K"]), dev(x["V"]), cfg.r, cfg.k)
    torch.cuda.synchronize()
    assert max_abs(out_g, oracle.dense(x["q"], x["K"], x["V"])) <= OUT_TOL[torch.bfloat16]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_index_projection_lead_only(gpu_lib, dt):
    # the key index written alone equals the lead dims of the full projection
    # bit for bit, and the oracle's projection within the rounding bound
    cfg = CONFIGS["C3"].scaled(S=1000, B=2).replace(dtype=dt)
    x, _, B_t, _ = asym_inputs(cfg)
    K, Bd = dev(x["K"]), dev(B_t)
    R = cfg.r
    idx_only = gpu_lib.loki_project_keys(K, Bd, R=R, lead_only=True)
    _, lead = gpu_lib.loki_project_keys(K, Bd, R=R)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t)
    assert torch.equal(bits(idx_only.cpu()), bits(lead.cpu()))
    exact = oracle.project(x["K"], B_t)[..., :R]
    acc = 2.0 * (cfg.d + 2) * U * oracle.project(x["K"].abs(), B_t.abs())[..., :R]
    tol = (2.0 ** -8 * (np.abs(exact) + acc) + acc) if dt == "bf16" else acc + 1e-30
    assert np.all(np.abs(idx_only.double().cpu().numpy() - exact) <= tol)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_calibrate_asym_matches_oracle(gpu_lib, dt, d):
    # the GPU's factors give the oracle's rank-r product M = A_r B_r^T (unique:
    # the columns themselves carry a sign per pair) and reach the optimal
    # distortion; the columns past r are zero
    cfg = CONFIGS["C1"].replace(B=2, Hq=4, Hkv=2, d=d, S=1000, r=16, dtype=dt, tau=6.0)
    x = make_inputs(cfg, need_K=True)
    qs = make_query_samples(cfg, 300)
    A_g, B_g = gpu_lib.loki_calibrate_asym(dev(qs), dev(x["K"]), cfg.r)
    torch.cuda.synchronize()
    A_o, B_o = asym.calibrate(qs, x["K"], cfg.r)
    Ag, Bg = A_g.double().cpu().numpy(), B_g.double().cpu().numpy()
    assert np.all(Ag[:, :, cfg.r:] == 0) and np.all(Bg[:, :, cfg.r:] == 0)
    for kv in range(cfg.Hkv):
        Qk = qs[:, 2 * kv:2 * kv + 2].double().numpy().reshape(-1, d)
        Kk = np.concatenate([x["K"][b, kv].double().numpy() for b in range(cfg.B)])
        Cq, Ck = Qk.T @ Qk / len(Qk), Kk.T @ Kk / len(Kk)
        Mg = Ag[kv, :, :cfg.r] @ Bg[kv, :, :cfg.r].T
        Mo = A_o[kv] @ B_o[kv].T
        rel = 1e-4 if dt == "f32" else 2e-2
        assert np.max(np.abs(Mg - Mo)) <= rel * np.max(np.abs(Mo)), (kv, np.max(np.abs(Mg - Mo)))
        dg, do = asym.distortion(Cq, Ck, Mg), asym.distortion(Cq, Ck, Mo)
        assert dg <= do * (1.0 + (1e-6 if dt == "f32" else 5e-2)) + 1e-12 * np.trace(Cq) * np.trace(Ck)


def test_calibrated_index_end_to_end(gpu_lib):
    # calibrate, write the index and decode, all on the GPU, against the
    # oracle's own pipeline from the same query samples and keys
    cfg = CONFIGS["C3"].scaled(S=2048, B=2)
    x = make_inputs(cfg, need_K=True)
    qs = make_query_samples(cfg, 256)
    K = dev(x["K"])
    A_g, B_g = gpu_lib.loki_calibrate_asym(dev(qs), K, cfg.r)
    K_idx = gpu_lib.loki_project_keys(K, B_g, R=cfg.r, lead_only=True)
    out_g, idx_g = gpu_lib.loki_decode_asym(dev(x["q"]), A_g, K_idx, K, dev(x["V"]), cfg.r, cfg.k)
    torch.cuda.synchronize()
    # the oracle's own pipeline from the same q samples and keys
    A_o, B_o = asym.calibrate(qs, x["K"], cfg.r)
    idx_o = asym.select(x["q"], A_o, np.einsum("bhsd,hdr->bhsr", x["K"].double().numpy(), B_o), cfg.r, cfg.k)
    # both pipelines keep nearly the same tokens (bf16 storage of A, B and the
    # index moves scores near the threshold; the recall of the oracle's set)
    ig = idx_g.cpu().numpy()
    recall = np.mean([len(set(ig[b, h]) & set(idx_o[b, h])) / cfg.k
                      for b in range(cfg.B) for h in range(cfg.Hq)])
    assert recall > 0.95, recall
    # the decode stage on the GPU's stored factors and index against the
    # oracle's decode on the same stored values: kept sets by the tie-band
    # rule, outputs to the tolerance (band rows on the GPU's own sets)
    x2 = {"q": x["q"], "K": x["K"], "V": x["V"]}
    run_asym_stored = run_asym(gpu_lib, x2, A_g.cpu(), K_idx.cpu(), cfg.r, cfg.k)
    assert torch.equal(run_asym_stored[1], idx_g)
    assert torch.equal(run_asym_stored[0].view(torch.int16), out_g.view(torch.int16))
