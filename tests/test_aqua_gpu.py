"""GPU parity of the decode step with query-magnitude dimensions
(loki_decode_aqua) against the float64 oracle (oracle.aqua), through the C ABI.

Each query head's dims are chosen on |q_rot| (fp32 on the GPU, float64 in
the oracle).  Dims whose oracle magnitude lies within 1e-5 ||q_rot|| of the
r-th largest are a tie band (the fp32 rotation's error is below that): the
chosen sets must agree outside it.  A head whose sets differ inside the band
legitimately scores different dims; the oracle then scores that head on the
GPU's dims.  Every head then follows the token tie-band rule of the
leading-dims decode on the oracle's scores (kept sets bit-exact outside the
1e-4 band, outputs within 1e-5 fp32 / 2e-2 bf16, a row whose set differs
inside the band against the oracle's attention over the GPU's own set), and
the retention loss is the oracle's for the GPU's dims.  Integer inputs with an identity basis make
every magnitude an exact small integer, so the tie rule (lower dim index)
is compared bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import aqua
from loki_inputs import CONFIGS, make_inputs, make_integer_inputs
from parity_helpers import OUT_TOL, check_band_rows, check_index_sets

pytestmark = pytest.mark.gpu

DIM_BAND = 1e-5


def dev(t):
    return t.to("cuda")


def dims_agree(qr, r, dims_g, dims_o):
    """True if the sets are equal; False if they differ only inside the tie
    band (then the GPU's set must still be a valid choice); raises otherwise."""
    if np.array_equal(dims_g, dims_o):
        return True
    a = np.abs(qr)
    mr = np.sort(a)[::-1][r - 1]
    band = set(np.nonzero(np.abs(a - mr) <= DIM_BAND * np.linalg.norm(qr))[0].tolist())
    g, o = set(dims_g.tolist()), set(dims_o.tolist())
    assert g - band == o - band, f"dims differ outside the tie band: {sorted(g ^ o)}"
    assert len(g) == r and np.all(np.diff(dims_g) > 0)
    return False


def run_aqua(rks, x, r, k, lens=None):
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    lens_d = None if lens is None else dev(torch.tensor(lens, dtype=torch.int32))
    out_g, idx_g, dims_g, info_g = rks.loki_decode_aqua(q, P, Kr, V, r, k, lens=lens_d)
    torch.cuda.synchronize()
    B, Hq, d = x["q"].shape
    S = x["K_rot"].shape[2]
    qr = oracle.rotate_queries(x["q"], x["P"])
    dims_o = aqua.query_dims(x["q"], x["P"], r)
    dg = dims_g.cpu().numpy()
    ig = idx_g.cpu().numpy().astype(np.int64)
    og = out_g.double().cpu().numpy()
    tol = OUT_TOL[x["q"].dtype]
    same_dims = np.ones((B, Hq), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            same_dims[b, h] = dims_agree(qr[b, h], r, dg[b, h], dims_o[b, h])
    # the retention loss of the dims the GPU chose (the oracle's own where
    # the two sets agree)
    info_o = aqua.info_loss(x["q"], x["P"], dg)
    assert np.all(np.abs(info_g.cpu().numpy() - info_o) <= 1e-5)
    for b in range(B):
        L = S if lens is None else min(max(int(lens[b]), 1), S)
        kb = min(k, L)
        sl = {n: x[n][b:b + 1] for n in ("q", "K_rot", "V")}
        # the oracle's scores on the dims each head scored with: its own dims,
        # or the GPU's where they differ inside the dim band; then the token
        # rule of the leading-dims decode on those scores
        dims_use = np.where(same_dims[b][:, None], dims_o[b], dg[b])
        s_o = aqua.scores_on_dims(sl["q"], x["P"], sl["K_rot"][:, :, :L], dims_use[None])
        idx_o = np.stack([oracle.topk_indices(s_o[0, h], kb) for h in range(Hq)])[None]
        out_o = oracle.attend(sl["q"], x["P"], sl["K_rot"][:, :, :L], sl["V"][:, :, :L], idx_o)
        assert np.all(ig[b, :, kb:] == -1)
        differ = check_index_sets(ig[b:b + 1, :, :kb], idx_o, s_o, kb)
        same = np.ones(Hq, dtype=bool)
        for _, h in differ:
            same[h] = False
        if same.any():
            assert np.max(np.abs(og[b] - out_o[0])[same]) <= tol, b
        # band rows: the oracle's attention over the GPU's own kept set
        check_band_rows(og[b:b + 1], ig[b:b + 1, :, :kb], differ, sl["q"], x["P"], sl["K_rot"][:, :, :L],
                        sl["V"][:, :, :L], tol)
    return int((~same_dims).sum())


CASES = {
    "C1_f32": (CONFIGS["C1"], {}),
    "C2_mha": (CONFIGS["C2"].scaled(S=2048), {}),
    "C3_gqa": (CONFIGS["C3"].scaled(S=4096, B=2), {}),
    "C5_r64": (CONFIGS["C5"].scaled(S=4096, B=1), {}),
    "gqa_f32_d128": (CONFIGS["C3"].replace(dtype="f32").scaled(S=3000, B=2), {}),
    "C4_long": (CONFIGS["C4"].scaled(S=40000), {}),
    "C3_b16": (CONFIGS["C3"].scaled(S=2048, B=16), {}),     # 512 query heads
}


@pytest.mark.parametrize("name", list(CASES))
def test_aqua_decode_matches_oracle(gpu_lib, name):
    cfg, _ = CASES[name]
    x = make_inputs(cfg)
    n_band = run_aqua(gpu_lib, x, cfg.r, cfg.k)
    assert n_band <= max(1, cfg.B * cfg.Hq // 8)


@pytest.mark.parametrize("r", [1, 7, 64])
def test_aqua_decode_edge_ranks(gpu_lib, r):
    cfg = CONFIGS["C1"].replace(B=2, Hq=4, Hkv=2, S=777, k=50)
    run_aqua(gpu_lib, make_inputs(cfg), r, cfg.k)


def test_aqua_full_rank_equals_full_rank_loki(gpu_lib):
    # r = d keeps every dim, so the masked query is the query itself and the
    # step is the leading-dims decode at r = d through the same kernels: bit
    # for bit the same result
    cfg = CONFIGS["C3"].scaled(S=2048, B=2)
    x = make_inputs(cfg)
    run_aqua(gpu_lib, x, cfg.d, cfg.k)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    out_a, idx_a, _, _ = gpu_lib.loki_decode_aqua(q, P, Kr, V, cfg.d, cfg.k)
    out_l, idx_l = gpu_lib.loki_decode(q, P, Kr, V, r=cfg.d, k=cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_l)
    assert torch.equal(out_a.view(torch.int16), out_l.view(torch.int16))


def test_aqua_ragged_batch(gpu_lib):
    cfg = CONFIGS["C3"].scaled(S=2048, B=5)
    x = make_inputs(cfg)
    g = torch.Generator().manual_seed(3)
    x["K_rot"][1, :, 700:] = torch.randn((cfg.Hkv, 2048 - 700, cfg.d), generator=g).to(torch.bfloat16) * 50
    lens = [2048, 700, 1, cfg.k - 3, 1500]
    run_aqua(gpu_lib, x, cfg.r, cfg.k, lens=lens)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_aqua_exact_integer_ties(gpu_lib, dt):
    # identity basis, integer queries and keys: every |q_rot| and every score
    # is an exact small integer, so dims and kept sets tie exactly and the
    # lower-index rules decide; both sides must agree bit for bit
    x = make_integer_inputs(B=2, Hq=4, Hkv=2, d=64, S=300, dtype=dt, seed=4)
    r, k = 9, 40
    out_g, idx_g, dims_g, info_g = gpu_lib.loki_decode_aqua(dev(x["q"]), dev(x["P"]), dev(x["K_rot"]),
                                                            dev(x["V"]), r, k)
    torch.cuda.synchronize()
    assert np.array_equal(dims_g.cpu().numpy(), aqua.query_dims(x["q"], x["P"], r))
    assert np.array_equal(idx_g.cpu().numpy(), aqua.select(x["q"], x["P"], x["K_rot"], r, k))
    out_o, _ = aqua.decode(x["q"], x["P"], x["K_rot"], x["V"], r, k)
    assert np.max(np.abs(out_g.double().cpu().numpy() - out_o)) <= OUT_TOL[x["q"].dtype]


def test_aqua_large_batch_ragged_and_full_rank(gpu_lib):
    # 512 query heads: ragged lengths, then r = d: the same kept sets as the
    # leading-dims decode at r = d (which runs the whole step of each pair of
    # heads in one kernel here; its scores equal the score kernel's bit for
    # bit, its attention sums in another order), both outputs against the
    # oracle
    cfg = CONFIGS["C3"].scaled(S=2048, B=16)
    x = make_inputs(cfg)
    lens = [2048 - 97 * b for b in range(cfg.B)]
    lens[3], lens[7] = 1, cfg.k - 1
    run_aqua(gpu_lib, x, cfg.r, cfg.k, lens=lens)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    out_a, idx_a, _, _ = gpu_lib.loki_decode_aqua(q, P, Kr, V, cfg.d, cfg.k)
    out_l, idx_l = gpu_lib.loki_decode(q, P, Kr, V, r=cfg.d, k=cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_l)
    # the kept sets against the oracle's full-rank selection (tie-band rule),
    # both outputs against the oracle's attention over those sets
    idx_o, s_o = oracle.select(x["q"], x["P"], x["K_rot"], cfg.d, cfg.k, return_scores=True)
    ig = idx_l.cpu().numpy().astype(np.int64)
    check_index_sets(ig, idx_o, s_o, cfg.k)
    want = oracle.attend(x["q"], x["P"], x["K_rot"], x["V"], ig)
    for o in (out_a, out_l):
        assert np.max(np.abs(o.double().cpu().numpy() - want)) <= OUT_TOL[torch.bfloat16]
