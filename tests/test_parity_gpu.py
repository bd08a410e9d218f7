"""GPU parity: every stage and the whole decode step against the float64 oracle.

All calls go through the C ABI (rank_key_sparse_amd's ctypes binding).  Inputs
come from the seeded generator; expected values come only from the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from loki_inputs import CONFIGS, make_inputs, make_integer_inputs
from parity_helpers import OUT_TOL, check_band_rows, check_index_sets, max_abs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def dev(x):
    return x.to("cuda") if isinstance(x, torch.Tensor) else x


def as_np(t):
    return t.detach().cpu().double().numpy()


# ---------------------------------------------------------------- helpers


def run_decode(rks, x, r, k, check_out=True, R=None):
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    K_lead = Kr[..., :R].contiguous() if R else None
    out_g, idx_g = rks.loki_decode(q, P, Kr, V, r=r, k=k, K_lead=K_lead)
    torch.cuda.synchronize()
    idx_o, s_o = oracle.select(x["q"], x["P"], x["K_rot"], r, k, return_scores=True)
    out_o = oracle.attend(x["q"], x["P"], x["K_rot"], x["V"], idx_o)
    ig = idx_g.cpu().numpy().astype(np.int64)
    differ = check_index_sets(ig, idx_o, s_o, k)
    tol = OUT_TOL[x["q"].dtype]
    og = as_np(out_g)
    same = np.ones(og.shape[:2], dtype=bool)
    for b, h in differ:
        same[b, h] = False
    if check_out:
        err = float(np.max(np.abs(og - out_o)[same])) if same.any() else 0.0
        assert err <= tol, f"output max-abs {err} > {tol}"
    # rows whose kept set legitimately differs (inside the tie band): the
    # output is the oracle's attention over the GPU's own set
    check_band_rows(og, ig, differ, x["q"], x["P"], x["K_rot"], x["V"], tol)
    return out_g, idx_g, differ


def cfg_case(name, **kw):
    cfg = CONFIGS[name]
    return cfg.scaled(**kw) if kw else cfg


DECODE_CASES = {
    "C1": cfg_case("C1"),
    "C2@S1024": cfg_case("C2", S=1024),
    "C3@B2S4096": cfg_case("C3", S=4096, B=2),
    "C4@S16384": cfg_case("C4", S=16384),
    "C5@B1S8192": cfg_case("C5", S=8192, B=1),
    "C3@B8S4096": cfg_case("C3", S=4096, B=8),
    "C2@B8S4096": cfg_case("C2", S=4096, B=8),      # MHA, >= 256 heads: fused score+select path
    "C2": cfg_case("C2"),
    "C3": cfg_case("C3"),
    "C4": cfg_case("C4"),
    "C5": cfg_case("C5"),
}



# ---------------------------------------------------------------- stages


SCORE_CASES = [
    ("C1", CONFIGS["C1"]),
    ("C3@B2S2048", CONFIGS["C3"].scaled(S=2048, B=2)),
    ("ragged_f32_r5", CONFIGS["C3"].replace(name="rf", cfg_no=51, B=1, Hq=6, Hkv=3, S=1001, dtype="f32", r=5)),
    ("d64_bf16_G2_r40", CONFIGS["C3"].replace(name="d64", cfg_no=52, B=2, Hq=4, Hkv=2, S=700, d=64, r=40)),
    ("f32_d128_r128", CONFIGS["C3"].replace(name="f128", cfg_no=53, B=1, Hq=2, Hkv=1, S=333, dtype="f32", r=128)),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_scores_within_fp32_bound(gpu_lib, case):
    _, cfg = case
    x = make_inputs(cfg)
    s_g = gpu_lib.loki_scores(dev(x["q"]), dev(x["P"]), dev(x["K_rot"]), cfg.r).cpu().double().numpy()
    s_o = oracle.approx_scores(x["q"], x["P"], x["K_rot"], cfg.r)
    # bound from the arithmetic: fp32 q_rot (d FMAs) then an r-term fp32 dot
    qabs = oracle.rotate_queries(x["q"].abs(), x["P"].abs())
    G = cfg.G
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            ka = as_np(x["K_rot"][b, h // G, :, :cfg.r]).__abs__()
            bound = 2.0 * (cfg.r + cfg.d + 2) * U * (ka @ qabs[b, h, :cfg.r]) + 1e-30
            assert np.all(np.abs(s_g[b, h] - s_o[b, h]) <= bound), (b, h)


def _score_rows():
    g = np.random.default_rng(7)
    rows = {}
    rows["normal"] = g.standard_normal((8, 3000)).astype(np.float32)
    rows["int_ties"] = g.integers(-5, 6, size=(6, 2500)).astype(np.float32)
    rows["all_equal"] = np.full((3, 1000), 2.5, dtype=np.float32)
    z = np.zeros((2, 500), dtype=np.float32)
    z[:, ::2] = -0.0
    z[:, 7] = 1.0
    rows["signed_zero"] = z
    h = g.standard_normal((4, 4000)).astype(np.float32)
    h[:, 0] = 1e30
    h[:, 1] = -1e30
    rows["huge_range"] = h
    t = g.standard_normal((4, 20000)).astype(np.float32)
    t[:, 5000:9000] = 0.75  # thousands of exact ties around the threshold
    rows["crowded_bin"] = t
    rows["ascending"] = np.tile(np.arange(4097, dtype=np.float32), (2, 1))
    rows["big_global"] = g.standard_normal((3, 70000)).astype(np.float32)
    c = g.standard_normal((2, 70000)).astype(np.float32)
    c[:, 1000:30000] = -0.25
    rows["big_crowded"] = c
    rows["S1"] = np.array([[3.0], [-1.0]], dtype=np.float32)
    # long rows selected per 16384-token chunk, then over the chunk winners:
    # a block of equal top values straddles a chunk boundary, and integer
    # ties spread over every chunk
    t = g.standard_normal((2, 50000)).astype(np.float32)
    t[:, 12000:22000] = 3.0
    rows["chunk_ties"] = t
    rows["chunk_int_ties"] = g.integers(-3, 4, size=(2, 50000)).astype(np.float32)
    return rows


SCORE_ROWS = _score_rows()


@pytest.mark.parametrize("name", list(SCORE_ROWS))
def test_select_topk_bit_exact(gpu_lib, name):
    s = SCORE_ROWS[name]
    S = s.shape[1]
    ks = sorted({1, max(1, S // 16), max(1, S // 2), S, min(S, 7)})
    sd = torch.from_numpy(s).to("cuda")
    for k in ks:
        idx_g = gpu_lib.loki_select_topk(sd, k).cpu().numpy()
        for i in range(s.shape[0]):
            want = oracle.topk_indices(s[i].astype(np.float64), k)
            assert np.array_equal(idx_g[i], want), (name, k, i)


@pytest.mark.parametrize("name", ["C1", "C3@B2S4096", "C4@S16384"])
def test_attend_on_oracle_sets(gpu_lib, name):
    cfg = DECODE_CASES[name]
    x = make_inputs(cfg)
    idx_o = oracle.select(x["q"], x["P"], x["K_rot"], cfg.r, cfg.k)
    out_o = oracle.attend(x["q"], x["P"], x["K_rot"], x["V"], idx_o)
    out_g = gpu_lib.loki_attend(dev(x["q"]), dev(x["P"]), dev(x["K_rot"]), dev(x["V"]),
                                torch.from_numpy(idx_o.astype(np.int32)).to("cuda"))
    assert max_abs(out_g, out_o) <= OUT_TOL[x["q"].dtype]


def test_attend_ignores_out_of_range_and_duplicates(gpu_lib):
    cfg = CONFIGS["C3"].replace(name="dup", cfg_no=54, B=1, Hq=4, Hkv=2, S=500, r=8, k=6)
    x = make_inputs(cfg)
    idx = np.array([[[3, 3, 10, -1, 499, 700]] * 4], dtype=np.int32)
    out_g = gpu_lib.loki_attend(dev(x["q"]), dev(x["P"]), dev(x["K_rot"]), dev(x["V"]),
                                torch.from_numpy(idx).to("cuda"))
    clean = np.array([[[3, 10, 499]] * 4])
    out_o = oracle.attend(x["q"], x["P"], x["K_rot"], x["V"], clean)
    assert max_abs(out_g, out_o) <= OUT_TOL[torch.bfloat16]


# ---------------------------------------------------------------- projection


def _proj_inputs(B, Hkv, S, d, dt, kind, seed=0):
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    K = torch.randn((B, Hkv, S, d), generator=g).to(tdt)
    if kind == "random":
        from loki_inputs import make_basis
        P = torch.from_numpy(np.stack([make_basis(d, 60, kv) for kv in range(Hkv)])).to(tdt)
    elif kind == "identity":
        P = torch.eye(d).expand(Hkv, d, d).contiguous().to(tdt)
    else:
        P = torch.zeros((Hkv, d, d))
        for kv in range(Hkv):
            perm = torch.randperm(d, generator=g)
            sg = torch.randint(0, 2, (d,), generator=g).float() * 2 - 1
            P[kv, torch.arange(d), perm] = sg
        P = P.to(tdt)
    return K, P


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["identity", "signed_perm", "random"])
def test_project_keys(gpu_lib, dt, d, kind):
    B, Hkv, S = 2, 3, 1000  # ragged: not a multiple of the 128-row tile
    K, P = _proj_inputs(B, Hkv, S, d, dt, kind)
    got = gpu_lib.loki_project_keys(dev(K), dev(P)).cpu()
    exact = oracle.project(K, P)
    if kind != "random":
        # products with +-1 and sums with exact zeros: exactly representable
        want = torch.from_numpy(exact).to(K.dtype)
        assert torch.equal(got.view(torch.int16) if dt == "bf16" else got, want.view(torch.int16) if dt == "bf16" else want)
        return
    absprod = oracle.project(K.abs(), P.abs())
    acc_err = 2.0 * (d + 2) * U * absprod
    g = got.double().numpy()
    if dt == "bf16":
        tol = 2.0 ** -8 * (np.abs(exact) + acc_err) + acc_err
    else:
        tol = acc_err + 1e-30
    assert np.all(np.abs(g - exact) <= tol)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lead", [False, True])
def test_append_kv(gpu_lib, dt, d, lead):
    # one decode step's new tokens written into the caches in place, at a
    # per-sequence position; the last sequence's position is outside the cache
    B, Hkv, S, R = 4, 3, 300, 32
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(11 + d)
    K_rot = torch.randn((B, Hkv, S, d), generator=g).to(tdt)
    V = torch.randn((B, Hkv, S, d), generator=g).to(tdt)
    k_new = torch.randn((B, Hkv, d), generator=g).to(tdt)
    v_new = torch.randn((B, Hkv, d), generator=g).to(tdt)
    from loki_inputs import make_basis
    P = torch.from_numpy(np.stack([make_basis(d, 61, kv) for kv in range(Hkv)])).to(tdt)
    pos = torch.tensor([0, 137, S - 1, S], dtype=torch.int32)
    Kd, Vd = dev(K_rot), dev(V)
    Ld = dev(K_rot[..., :R].contiguous()) if lead else None
    gpu_lib.loki_append_kv(dev(k_new), dev(v_new), dev(P), dev(pos), Kd, Vd, Ld)
    Kg, Vg = Kd.cpu(), Vd.cpu()
    written = torch.zeros((B, Hkv, S), dtype=torch.bool)
    for b in range(B):
        if 0 <= int(pos[b]) < S:
            written[b, :, int(pos[b])] = True
    bits = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t)
    # every other row is untouched, bit for bit
    assert torch.equal(bits(Kg)[~written], bits(K_rot)[~written])
    assert torch.equal(bits(Vg)[~written], bits(V)[~written])
    exact = oracle.project(k_new[:, :, None, :], P)[:, :, 0, :]
    acc_err = 2.0 * (d + 2) * U * oracle.project(k_new.abs()[:, :, None, :], P.abs())[:, :, 0, :]
    tol = 2.0 ** -8 * (np.abs(exact) + acc_err) + acc_err if dt == "bf16" else acc_err + 1e-30
    for b in range(B):
        p = int(pos[b])
        if not 0 <= p < S:
            continue
        got = Kg[b, :, p].double().numpy()
        assert np.all(np.abs(got - exact[b]) <= tol[b])
        assert torch.equal(bits(Vg[b, :, p]), bits(v_new[b]))
    if lead:
        assert torch.equal(bits(Ld.cpu()), bits(Kg[..., :R].contiguous()))


def test_append_then_decode(gpu_lib):
    # a short decode loop on a C3-shaped cache: the GPU appends the step's
    # token at the end of each sequence's filled prefix and decodes over its
    # cache; the oracle keeps its own cache, written from its own projection
    # of the same new keys (rounded to bf16 by torch), and decodes over that.
    # The new keys are drawn 4x wider than the cache's leading dims, so their
    # scores sit far from every head's selection threshold and a last-bit
    # difference between the two roundings of an appended row cannot change
    # a kept set (inputs and seeds fixed: the outcome is deterministic)
    cfg = cfg_case("C3", S=1024, B=2)
    x = make_inputs(cfg)
    q, P = dev(x["q"]), dev(x["P"])
    Kd, Vd = dev(x["K_rot"]), dev(x["V"])
    Ld = Kd[..., :cfg.r].contiguous()
    y = dict(x)
    y["K_rot"], y["V"] = x["K_rot"].clone(), x["V"].clone()
    g = torch.Generator().manual_seed(5)
    tol = OUT_TOL[torch.bfloat16]
    for step in range(3):
        k_new = (4.0 * torch.randn((cfg.B, cfg.Hkv, cfg.d), generator=g)).to(torch.bfloat16)
        v_new = torch.randn((cfg.B, cfg.Hkv, cfg.d), generator=g).to(torch.bfloat16)
        pos = [cfg.S - 3 + step, cfg.S - 5 + step]
        gpu_lib.loki_append_kv(dev(k_new), dev(v_new), P, dev(torch.tensor(pos, dtype=torch.int32)), Kd, Vd, Ld)
        rot = torch.from_numpy(oracle.project(k_new[:, :, None, :], x["P"])[:, :, 0, :]).to(torch.bfloat16)
        for b in range(cfg.B):
            y["K_rot"][b, :, pos[b]] = rot[b]
            y["V"][b, :, pos[b]] = v_new[b]
        out_g, idx_g = gpu_lib.loki_decode(q, P, Kd, Vd, r=cfg.r, k=cfg.k, K_lead=Ld)
        torch.cuda.synchronize()
        idx_o, s_o = oracle.select(y["q"], y["P"], y["K_rot"], cfg.r, cfg.k, return_scores=True)
        out_o = oracle.attend(y["q"], y["P"], y["K_rot"], y["V"], idx_o)
        ig = idx_g.cpu().numpy().astype(np.int64)
        differ = check_index_sets(ig, idx_o, s_o, cfg.k)
        assert not differ, differ
        assert max_abs(out_g, out_o) <= tol
        # the appended tokens are kept by some heads, so the step reads them
        assert sum(int(np.any(ig[b] == pos[b])) for b in range(cfg.B)) > 0


@pytest.mark.parametrize("shape", [
    ("pair", "C3", dict(S=2048, B=16)),        # rotation + scores + selection fused per pair of heads
    ("two_kernel", "C3", dict(S=4096, B=2)),   # rotation, scores, selection, attention kernels
    ("mha_fused", "C2", dict(S=2048, B=8)),    # one block per MHA head for scores + selection
], ids=lambda c: c[0])
def test_decode_graph_replay(gpu_lib, shape):
    # one decode step captured in a HIP graph: every replay equals the eager
    # call, also after a new query is written into the captured input and
    # with eager work on the outputs between replays
    _, name, kw = shape
    cfg = cfg_case(name, **kw)
    x = make_inputs(cfg)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    Kl = Kr[..., :cfg.r].contiguous()
    nbytes = gpu_lib.loki_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.d, cfg.r, cfg.k, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    idx = torch.empty((cfg.B, cfg.Hq, cfg.k), dtype=torch.int32, device="cuda")
    g = torch.Generator().manual_seed(21)
    q2 = dev(torch.randn(q.shape, generator=g).to(q.dtype))
    want = {}
    for tag, qq in (("q", q.clone()), ("q2", q2)):
        o, i = gpu_lib.loki_decode(qq, P, Kr, V, cfg.r, cfg.k, K_lead=Kl)
        want[tag] = (o.clone(), i.clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            gpu_lib.loki_decode(q, P, Kr, V, cfg.r, cfg.k, out=out, idx=idx, workspace=ws, K_lead=Kl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # the oracle's step for each query (selection with scores, attention)
    ref = {}
    for tag, qq in (("q", x["q"]), ("q2", q2.cpu())):
        idx_o, s_o = oracle.select(qq, x["P"], x["K_rot"], cfg.r, cfg.k, return_scores=True)
        ref[tag] = (qq, idx_o, s_o, oracle.attend(qq, x["P"], x["K_rot"], x["V"], idx_o))
    tol = OUT_TOL[x["q"].dtype]
    q_orig = q.clone()
    for rep, tag in enumerate(("q", "q", "q2", "q", "q2")):
        q.copy_(q_orig if tag == "q" else q2)
        out.zero_()
        idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o, i = want[tag]
        assert torch.equal(idx, i), (rep, tag)
        assert torch.equal(out.view(torch.int16), o.view(torch.int16)), (rep, tag)
        # and against the oracle: kept sets by the tie-band rule, outputs to
        # the tolerance (band rows on their own sets)
        qq, idx_o, s_o, out_o = ref[tag]
        ig = idx.cpu().numpy().astype(np.int64)
        og = as_np(out)
        differ = check_index_sets(ig, idx_o, s_o, cfg.k)
        same = np.ones(og.shape[:2], dtype=bool)
        for b, h in differ:
            same[b, h] = False
        assert float(np.max(np.abs(og - out_o)[same])) <= tol, (rep, tag)
        check_band_rows(og, ig, differ, qq, x["P"], x["K_rot"], x["V"], tol)


def run_decode_varlen(rks, x, lens, r, k, R=None):
    """GPU decode over a ragged batch against the oracle's (each sequence a
    decode over its own prefix), with the tie-band rule on each prefix."""
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    K_lead = Kr[..., :R].contiguous() if R else None
    out_g, idx_g = rks.loki_decode(q, P, Kr, V, r=r, k=k, K_lead=K_lead,
                                   lens=dev(torch.tensor(lens, dtype=torch.int32)))
    torch.cuda.synchronize()
    out_o, idx_o, s_o = oracle.decode_varlen(x["q"], x["P"], x["K_rot"], x["V"], lens, r, k, return_scores=True)
    ig = idx_g.cpu().numpy().astype(np.int64)
    S = Kr.shape[2]
    B, Hq, _ = ig.shape
    differ = []
    for b in range(B):
        L = min(max(int(lens[b]), 1), S)
        kb = min(k, L)
        assert np.all(ig[b, :, kb:] == -1), f"sequence {b}: entries past {kb} must be -1"
        rows = check_index_sets(ig[b:b + 1, :, :kb], idx_o[b:b + 1, :, :kb], s_o[b:b + 1, :, :L], kb)
        differ += [(b, h) for _, h in rows]
    tol = OUT_TOL[x["q"].dtype]
    og = as_np(out_g)
    same = np.ones(og.shape[:2], dtype=bool)
    for b, h in differ:
        same[b, h] = False
    err = float(np.max(np.abs(og - out_o)[same])) if same.any() else 0.0
    assert err <= tol, f"output max-abs {err} > {tol}"
    check_band_rows(og, ig, differ, x["q"], x["P"], x["K_rot"], x["V"], tol, lens=lens)
    return out_g, idx_g


VARLEN = [
    # (label, B, Hq, Hkv, S, d, dtype, r, k, R) -- the dispatch path each one takes
    ("pair_fused", 16, 32, 8, 2048, 128, "bf16", 32, 100, 32),
    ("mha_fused", 16, 16, 16, 1500, 128, "bf16", 24, 77, None),
    ("regs16_two_kernel", 9, 8, 2, 4000, 128, "bf16", 32, 300, 32),
    ("regs32_two_kernel", 9, 4, 2, 20000, 64, "bf16", 16, 700, None),
    ("chunked", 9, 4, 2, 40000, 128, "bf16", 16, 1500, 16),
    ("chunked_fused", 4, 32, 8, 40000, 128, "bf16", 16, 1500, 16),
    ("global", 9, 2, 1, 40000, 64, "bf16", 16, 20000, None),
    ("f32", 9, 6, 2, 1200, 64, "f32", 8, 50, None),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_decode_varlen(gpu_lib, case):
    label, B, Hq, Hkv, S, d, dt, r, k, R = case
    print(f"\n[varlen {label}] B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} {dt} r={r} k={k} R={R}", flush=True)
    cfg = CONFIGS["C3"].replace(name=label, cfg_no=51, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt, r=r, k=k)
    x = make_inputs(cfg)
    base = [S, 1, k - 1, k, k + 1, S - 1, S // 2 + 3, 2 * S, 0]
    lens = [base[b % len(base)] for b in range(B)]
    g = np.random.default_rng(7)
    for b in range(len(base), B):
        lens[b] = int(g.integers(1, S + 1))
    run_decode_varlen(gpu_lib, x, lens, r, k, R=R)


def test_decode_varlen_full_lengths_match_decode(gpu_lib):
    # every sequence full: bit-identical to the plain decode on the same path
    cfg = cfg_case("C3", S=2048, B=16)
    x = make_inputs(cfg)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    Kl = Kr[..., :cfg.r].contiguous()
    o1, i1 = gpu_lib.loki_decode(q, P, Kr, V, cfg.r, cfg.k, K_lead=Kl)
    o2, i2 = gpu_lib.loki_decode(q, P, Kr, V, cfg.r, cfg.k, K_lead=Kl,
                                 lens=dev(torch.full((cfg.B,), cfg.S, dtype=torch.int32)))
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_project_then_decode_c5_shape(gpu_lib):
    # the prefill-plus-decode workload: the GPU projection agrees with the
    # oracle's projection element-wise, and decode over the oracle's
    # (rounded) rotated keys matches the oracle
    cfg = CONFIGS["C5"].scaled(S=4096, B=2)
    x = make_inputs(cfg, need_K=True)
    K, P = x["K"], x["P"]
    got = gpu_lib.loki_project_keys(dev(K), dev(P)).cpu()
    exact = oracle.project(K, P)
    acc_err = 2.0 * (cfg.d + 2) * U * oracle.project(K.abs(), P.abs())
    assert np.all(np.abs(got.double().numpy() - exact) <= 2.0 ** -8 * (np.abs(exact) + acc_err) + acc_err)
    y = dict(x)
    y["K_rot"] = torch.from_numpy(exact).to(torch.bfloat16)
    run_decode(gpu_lib, y, cfg.r, cfg.k)


# ---------------------------------------------------------------- planted boundary ties


def _bits_step(row: torch.Tensor, c: int, step: int) -> torch.Tensor:
    """A copy of the 1-D stored row with element c moved `step` representable
    values in magnitude (sign-magnitude formats: +1 on the bit pattern is the
    next value away from zero)."""
    out = row.clone()
    iv = out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32)
    iv[c] += step
    return out


def plant_boundary_ties(x, cfg, max_groups=16):
    """For one query head per (b, kv) group (up to max_groups groups), copies
    the leading r dims of the head's k-th best token (by the oracle's
    approximate scores) onto two tokens ranked below it: the first copy is an
    exact tie with the k-th score; the second moves one to three of those dims
    by one or two storage ulps each, chosen so that its score differs by the
    smallest non-zero amount (far below 1e-5 relative).  Returns the new
    inputs and the planted (b, h, jk, ja, jb)."""
    import itertools
    Kr = x["K_rot"].clone()
    B, Hkv, S, _ = Kr.shape
    G, k, r = cfg.Hq // cfg.Hkv, cfg.k, cfg.r
    qr = oracle.rotate_queries(x["q"], x["P"])
    s = oracle.approx_scores(x["q"], x["P"], Kr, r)
    steps = (-2, -1, 1, 2)
    planted = []
    for gi in range(min(B * Hkv, max_groups)):
        b, kv = divmod(gi, Hkv)
        h = kv * G + gi % G
        if k + 100 >= S:
            continue
        order = np.argsort(-s[b, h], kind="stable")
        jk, ja, jb = (int(order[i]) for i in (k - 1, k + 40, k + 90))
        row = Kr[b, kv, jk, :r].clone()
        vals = row.double().numpy()
        # score change of each single move (dim c, step), exact in float64
        a = np.zeros((r, len(steps)))
        for c in range(r):
            if abs(vals[c]) < 1e-20:
                continue  # no steps at zero (they would leave the normal range)
            for si, st in enumerate(steps):
                a[c, si] = qr[b, h, c] * (float(_bits_step(row, c, st)[c]) - vals[c])
        best = (np.inf, ())
        dims = [c for c in range(r) if abs(vals[c]) >= 1e-20]
        for n in (1, 2, 3):
            if n == 3 and r > 16:
                break
            for cs in itertools.combinations(dims, n):
                for sis in itertools.product(range(len(steps)), repeat=n):
                    dlt = sum(a[c, si] for c, si in zip(cs, sis))
                    if dlt != 0.0 and abs(dlt) < best[0]:
                        best = (abs(dlt), tuple(zip(cs, (steps[si] for si in sis))))
        near = row
        for c, st in best[1]:
            near = _bits_step(near, c, st)
        Kr[b, kv, ja, :r] = row
        Kr[b, kv, jb, :r] = near
        planted.append((b, h, jk, ja, jb))
    y = dict(x)
    y["K_rot"] = Kr
    return y, planted


PLANT = [
    # (label, B, Hq, Hkv, S, d, dtype, r, k, R) -- one shape per dispatch path
    ("pair_fused", 16, 32, 8, 2048, 128, "bf16", 32, 100, 32),
    ("mha_fused", 16, 16, 16, 1500, 128, "bf16", 24, 77, None),
    ("regs16_two_kernel", 9, 8, 2, 4000, 128, "bf16", 32, 300, 32),
    ("regs32_two_kernel", 9, 4, 2, 20000, 64, "bf16", 16, 700, None),
    ("chunked", 9, 4, 2, 40000, 128, "bf16", 16, 1500, 16),
    ("chunked_fused", 4, 32, 8, 40000, 128, "bf16", 16, 1500, 16),
    ("global", 3, 2, 1, 60000, 64, "bf16", 16, 17000, None),
    ("f32", 9, 6, 2, 1200, 64, "f32", 8, 50, None),
]


@pytest.mark.parametrize("case", PLANT, ids=[c[0] for c in PLANT])
def test_decode_planted_boundary_ties(gpu_lib, case):
    label, B, Hq, Hkv, S, d, dt, r, k, R = case
    print(f"\n[ties {label}] B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} {dt} r={r} k={k} R={R}", flush=True)
    cfg = CONFIGS["C3"].replace(name=label, cfg_no=57, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt, r=r, k=k)
    y, planted = plant_boundary_ties(make_inputs(cfg), cfg)
    assert planted
    # the planted ties sit at each planted head's k-th score, inside the band
    _, s_o = oracle.select(y["q"], y["P"], y["K_rot"], r, k, return_scores=True)
    for b, h, jk, ja, jb in planted:
        sstar = np.sort(s_o[b, h])[::-1][k - 1]
        assert s_o[b, h, ja] == s_o[b, h, jk]
        assert abs(s_o[b, h, jb] - s_o[b, h, jk]) <= 1e-5 * abs(sstar)
        assert abs(s_o[b, h, jk] - sstar) <= 1e-5 * abs(sstar)
    _, idx_g, differ = run_decode(gpu_lib, y, r, k, R=R)
    ig = idx_g.cpu().numpy()
    # exact ties go to the lower index: of jk and ja, only the lower one can
    # be kept without the other (bit-exact rule, no band needed)
    for b, h, jk, ja, jb in planted:
        lo, hi = min(jk, ja), max(jk, ja)
        assert not (hi in ig[b, h] and lo not in ig[b, h]), (b, h)
    print(f"[ties {label}] planted heads {len(planted)}, rows with band-equivalent sets: {len(differ)}", flush=True)


# ---------------------------------------------------------------- decode parity
FULL = {"C2", "C3", "C4", "C5"}


@pytest.mark.parametrize("name", [pytest.param(n, marks=pytest.mark.slow) if n in FULL else n
                                  for n in DECODE_CASES])
def test_decode_workloads(gpu_lib, name):
    cfg = DECODE_CASES[name]
    x = make_inputs(cfg)
    # full-size workloads run as the benchmark runs them: scores from a
    # leading-dims copy with R = r
    R = cfg.r if name in FULL else None
    print(f"\n[{name}] B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} S={cfg.S} d={cfg.d} r={cfg.r} k={cfg.k} R={R}",
          flush=True)
    _, _, differ = run_decode(gpu_lib, x, cfg.r, cfg.k, R=R)
    print(f"[{name}] rows with band-equivalent sets: {len(differ)}", flush=True)


EDGE = [
    # (label, B, Hq, Hkv, S, d, dtype, r, k)
    ("S1", 1, 2, 1, 1, 128, "bf16", 8, 1),
    ("k_eq_S", 1, 4, 2, 300, 128, "bf16", 16, 300),
    ("k1", 2, 4, 4, 500, 64, "f32", 8, 1),
    ("r_eq_d", 1, 4, 1, 777, 128, "bf16", 128, 40),
    ("r1", 1, 2, 2, 1000, 64, "bf16", 1, 100),
    ("r5_ragged", 2, 6, 2, 1000, 128, "f32", 5, 33),
    ("r13_G3", 1, 6, 2, 2049, 64, "bf16", 13, 200),
    ("G16", 1, 16, 1, 1500, 128, "bf16", 32, 64),
    ("G8_f32_d128", 1, 16, 2, 1111, 128, "f32", 24, 128),
    ("d64_bf16_r64", 3, 8, 8, 640, 64, "bf16", 64, 64),
    ("chunked_select", 1, 4, 2, 40000, 128, "bf16", 32, 1500),
    # the first stage fused with the scores (>= 256 blocks of query head x chunk)
    ("chunked_fused_r40", 2, 64, 8, 40000, 128, "bf16", 40, 1500),
    ("chunked_fused_d64_G4", 3, 32, 8, 50000, 64, "bf16", 64, 3000),
    # k near the largest two-stage k (C k <= 32768): the last chunk (7232 tokens) is all candidates; r = d
    ("chunked_fused_k10000_r128", 3, 32, 8, 40000, 128, "bf16", 128, 10000),
    ("global_select", 1, 2, 1, 40000, 64, "bf16", 16, 20000),
    # fused score+select path (MHA, >= 256 heads, S <= 16384)
    ("fused_ragged_r24", 16, 16, 16, 1000, 128, "bf16", 24, 77),
    ("fused_d64_r40", 32, 8, 8, 3001, 64, "bf16", 40, 300),
    ("fused_r128_k1", 8, 32, 32, 777, 128, "bf16", 128, 1),
    ("fused_S16384", 4, 64, 64, 16384, 128, "bf16", 32, 700),
    ("many_heads_G4", 16, 16, 4, 1000, 128, "bf16", 24, 77),
    # fused path for pairs of grouped heads (G even, >= 512 query heads, S <= 16384)
    ("pair_ragged_r24", 16, 32, 8, 1000, 128, "bf16", 24, 77),
    ("pair_G2_d64_r40", 32, 16, 8, 3001, 64, "bf16", 40, 300),
    ("pair_G8_r128_k1", 16, 32, 4, 777, 128, "bf16", 128, 1),
    ("pair_k_eq_S", 8, 64, 16, 300, 128, "bf16", 16, 300),
    ("pair_G16_r1", 32, 16, 1, 2049, 64, "bf16", 1, 500),
    ("pair_S16384", 8, 64, 16, 16384, 128, "bf16", 32, 700),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_decode_edge_cases(gpu_lib, case):
    label, B, Hq, Hkv, S, d, dt, r, k = case
    print(f"\n[{label}] B={B} Hq={Hq} Hkv={Hkv} S={S} d={d} {dt} r={r} k={k}", flush=True)
    cfg = CONFIGS["C3"].replace(name=label, cfg_no=50, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt,
                                r=r, k=k)
    x = make_inputs(cfg)
    run_decode(gpu_lib, x, r, k)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("pk", ["identity", "signed_perm"])
def test_decode_exact_ties(gpu_lib, dt, pk):
    # integer-valued inputs: every score is an exact integer on both sides, so
    # the kept sets must agree bit for bit, ties broken towards lower indices
    x = make_integer_inputs(2, 8, 2, 128, 3000, dt, seed=3, P_kind=pk)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    for r, k in ((8, 100), (3, 777), (128, 5)):
        _, idx_g = gpu_lib.loki_decode(q, P, Kr, V, r=r, k=k)
        idx_o = oracle.select(x["q"], x["P"], x["K_rot"], r, k)
        assert np.array_equal(idx_g.cpu().numpy(), idx_o), (r, k)


def test_decode_all_equal_keys(gpu_lib):
    B, Hq, Hkv, S, d = 1, 4, 2, 5000, 128
    Kr = torch.ones((B, Hkv, S, d), dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(0)
    V = torch.randn((B, Hkv, S, d), generator=g).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g).to(torch.bfloat16)
    P = torch.eye(d).expand(Hkv, d, d).contiguous().to(torch.bfloat16)
    k = 1234
    out_g, idx_g = gpu_lib.loki_decode(dev(q), dev(P), dev(Kr), dev(V), r=16, k=k)
    assert np.array_equal(idx_g.cpu().numpy(), np.broadcast_to(np.arange(k), (B, Hq, k)))
    out_o = oracle.attend(q, P, Kr, V, np.broadcast_to(np.arange(k), (B, Hq, k)))
    assert max_abs(out_g, out_o) <= OUT_TOL[torch.bfloat16]


def test_decode_all_equal_keys_fused(gpu_lib):
    B, Hq, Hkv, S, d = 64, 4, 4, 2000, 128  # 256 MHA heads: fused path
    Kr = torch.ones((B, Hkv, S, d), dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(1)
    V = torch.randn((B, Hkv, S, d), generator=g).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g).to(torch.bfloat16)
    P = torch.eye(d).expand(Hkv, d, d).contiguous().to(torch.bfloat16)
    k = 333
    out_g, idx_g = gpu_lib.loki_decode(dev(q), dev(P), dev(Kr), dev(V), r=32, k=k,
                                       K_lead=dev(Kr[..., :32].contiguous()))
    assert np.array_equal(idx_g.cpu().numpy(), np.broadcast_to(np.arange(k), (B, Hq, k)))
    out_o = oracle.attend(q, P, Kr, V, np.broadcast_to(np.arange(k), (B, Hq, k)))
    assert max_abs(out_g, out_o) <= OUT_TOL[torch.bfloat16]


def test_fused_matches_two_kernel_path(gpu_lib):
    # the same heads decoded with 256 query heads (scores and selection fused
    # per head) and 128 (scores, then selection and attention per head): the
    # score arithmetic is the same, so the kept sets are bit-identical; the
    # attention sums in another order, so each output is checked against the
    # oracle
    cfg = cfg_case("C2", S=4096, B=8)
    x = make_inputs(cfg)
    _, i_all, _ = run_decode(gpu_lib, x, cfg.r, cfg.k)
    half = {n: x[n][:4].contiguous() for n in ("q", "K_rot", "V")}
    half["P"] = x["P"]
    _, i_half, _ = run_decode(gpu_lib, half, cfg.r, cfg.k)
    assert torch.equal(i_all[:4], i_half)


def test_pair_fused_rank_and_radix_heads(gpu_lib):
    # pair-fused path (512 grouped query heads) with every even head's query
    # zero: its scores all tie (threshold bin crowded, radix tie path, lowest
    # indices kept) while the odd head of the same pair ranks a few candidates
    cfg = cfg_case("C3", S=2048, B=16)
    x = make_inputs(cfg)
    x = dict(x)
    q = x["q"].clone()
    q[:, 0::2, :] = 0
    x["q"] = q
    _, idx_g, _ = run_decode(gpu_lib, x, cfg.r, cfg.k, R=cfg.r)
    ig = idx_g.cpu().numpy()
    assert np.array_equal(ig[:, 0::2], np.broadcast_to(np.arange(cfg.k), ig[:, 0::2].shape))


@pytest.mark.parametrize("order", ["best_first", "best_last"])
def test_pair_fused_score_order(gpu_lib, order):
    # pair-fused path (512 grouped query heads).  The selection first estimates
    # each head's threshold bin from the first 4096 tokens (two score batches)
    # and visits only the tokens at or above it; here every group's rows are
    # sorted by the scores of its first query head.  best_first: that head's
    # best tokens fill the sample, the estimate lies above the real threshold
    # and the full selection runs; best_last: the sample holds its worst
    # tokens, whose range fixes the bins, so the best tokens crowd the top end
    # bin and the full selection (its exact radix path) runs as well.  With
    # the natural order every block takes the marked tokens only.  Either way
    # the result is the oracle's.  S = 8192 keeps the sample a strict part of
    # the sequence, so that best_first really misses: the sample's want-th
    # largest (want about 0.69 k) lies above the k-th
    cfg = cfg_case("C3", S=8192, B=16)
    x = dict(make_inputs(cfg))
    _, s_o = oracle.select(x["q"], x["P"], x["K_rot"], cfg.r, cfg.k, return_scores=True)
    G = cfg.Hq // cfg.Hkv
    Kr, V = x["K_rot"].clone(), x["V"].clone()
    for b in range(cfg.B):
        for kv in range(cfg.Hkv):
            s = s_o[b, kv * G]
            perm = np.argsort(-s, kind="stable") if order == "best_first" else np.argsort(s, kind="stable")
            perm = torch.from_numpy(perm.copy())
            Kr[b, kv] = Kr[b, kv][perm]
            V[b, kv] = V[b, kv][perm]
    x["K_rot"], x["V"] = Kr, V
    run_decode(gpu_lib, x, cfg.r, cfg.k, R=cfg.r)


def test_decode_all_equal_keys_pair(gpu_lib):
    B, Hq, Hkv, S, d = 16, 32, 8, 2000, 128  # 512 grouped heads: pair-fused path
    Kr = torch.ones((B, Hkv, S, d), dtype=torch.bfloat16)
    g = torch.Generator().manual_seed(2)
    V = torch.randn((B, Hkv, S, d), generator=g).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g).to(torch.bfloat16)
    P = torch.eye(d).expand(Hkv, d, d).contiguous().to(torch.bfloat16)
    k = 700
    out_g, idx_g = gpu_lib.loki_decode(dev(q), dev(P), dev(Kr), dev(V), r=32, k=k,
                                       K_lead=dev(Kr[..., :32].contiguous()))
    assert np.array_equal(idx_g.cpu().numpy(), np.broadcast_to(np.arange(k), (B, Hq, k)))
    out_o = oracle.attend(q, P, Kr, V, np.broadcast_to(np.arange(k), (B, Hq, k)))
    assert max_abs(out_g, out_o) <= OUT_TOL[torch.bfloat16]


def test_pair_fused_matches_two_kernel_path(gpu_lib):
    # grouped heads: 512 query heads (the whole step of each pair of heads in
    # one kernel) against the first 256 of them (rotation, scores, selection
    # and attention kernels).  The score arithmetic is the same, so the kept
    # sets are bit-identical; the attention sums in another order, so each
    # output is checked against the oracle
    cfg = cfg_case("C3", S=4096, B=16)
    x = make_inputs(cfg)
    o_all, i_all, _ = run_decode(gpu_lib, x, cfg.r, cfg.k, R=cfg.r)
    half = {n: x[n][:8].contiguous() for n in ("q", "K_rot", "V")}
    half["P"] = x["P"]
    o_half, i_half, _ = run_decode(gpu_lib, half, cfg.r, cfg.k, R=cfg.r)
    assert torch.equal(i_all[:8], i_half)


def test_decode_deterministic(gpu_lib):
    cfg = cfg_case("C3", S=8192, B=2)
    x = make_inputs(cfg)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    o1, i1 = gpu_lib.loki_decode(q, P, Kr, V, r=cfg.r, k=cfg.k)
    o2, i2 = gpu_lib.loki_decode(q, P, Kr, V, r=cfg.r, k=cfg.k)
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))




# ---------------------------------------------------------------- lead-dims layout


LEAD_CASES = [
    # (label, cfg, R)
    ("C1_R16", CONFIGS["C1"], 16),
    ("C3_R32", CONFIGS["C3"].scaled(S=4096, B=2), 32),
    ("C3_R64", CONFIGS["C3"].scaled(S=4096, B=1), 64),
    ("C4_R16", CONFIGS["C4"].scaled(S=16384), 16),
    ("C5_R64", CONFIGS["C5"].scaled(S=8192, B=1), 64),
    ("f32_d128_R8_r5", CONFIGS["C3"].replace(name="l8", cfg_no=55, B=1, Hq=4, Hkv=2, S=999, dtype="f32", r=5, k=33), 8),
]


@pytest.mark.parametrize("case", LEAD_CASES, ids=[c[0] for c in LEAD_CASES])
def test_decode_lead_layout(gpu_lib, case):
    label, cfg, R = case
    x = make_inputs(cfg)
    out_l, idx_l, _ = run_decode(gpu_lib, x, cfg.r, cfg.k, R=R)
    # the lead copy holds the same values, so the result is bit-identical to
    # decoding from K_rot's own rows
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    out_r, idx_r = gpu_lib.loki_decode(q, P, Kr, V, r=cfg.r, k=cfg.k)
    assert torch.equal(idx_l, idx_r)
    assert torch.equal(out_l.view(torch.int16) if out_l.dtype == torch.bfloat16 else out_l,
                       out_r.view(torch.int16) if out_r.dtype == torch.bfloat16 else out_r)


@pytest.mark.parametrize("dt,d,R", [("bf16", 128, 32), ("bf16", 128, 16), ("bf16", 64, 64), ("f32", 64, 16), ("f32", 128, 4)])
def test_project_lead_copy(gpu_lib, dt, d, R):
    K, P = _proj_inputs(2, 3, 777, d, dt, "random", seed=4)
    Kr, Kl = gpu_lib.loki_project_keys(dev(K), dev(P), R=R)
    Kr2 = gpu_lib.loki_project_keys(dev(K), dev(P))
    assert torch.equal(Kr.view(torch.int16) if dt == "bf16" else Kr, Kr2.view(torch.int16) if dt == "bf16" else Kr2)
    assert torch.equal(Kl, Kr[..., :R].contiguous())


@pytest.mark.slow
@pytest.mark.parametrize("k", [16, 64])
def test_decode_maximum_cache_length(gpu_lib, k):
    # the largest cache the library accepts (2^24 tokens; one more is
    # rejected): k = 16 takes the chunked two-stage selection (1024 chunks of
    # 16384 tokens), k = 64 overflows its candidate list and takes the
    # global-memory selection
    cfg = CONFIGS["C1"].replace(B=1, Hq=2, Hkv=1, d=64, S=1 << 24, r=16, k=k, dtype="bf16", tau=8.0)
    print(f"\n[max S] S={cfg.S} k={k}", flush=True)
    x = make_inputs(cfg)
    _, _, differ = run_decode(gpu_lib, x, cfg.r, cfg.k)
    print(f"[max S] rows with band-equivalent sets: {len(differ)}", flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_decode_ignores_stale_workspace(gpu_lib, case):
    # every kernel writes what it later reads: a workspace full of 0xFF
    # bytes (and one full of zeros) gives bit for bit the same step, with
    # and without per-sequence lengths, on every dispatch path
    label, B, Hq, Hkv, S, d, dt, r, k, R = case
    cfg = CONFIGS["C3"].replace(name=label, cfg_no=52, B=B, Hq=Hq, Hkv=Hkv, S=S, d=d, dtype=dt, r=r, k=k)
    x = make_inputs(cfg)
    q, P, Kr, V = (dev(x[n]) for n in ("q", "P", "K_rot", "V"))
    Kl = Kr[..., :R].contiguous() if R else None
    nb = gpu_lib.loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, q.dtype)
    lens = dev(torch.tensor([max(1, S - 37 * b) for b in range(B)], dtype=torch.int32))
    for ln in (None, lens):
        results = []
        for fill in (0x00, 0xFF):
            ws = torch.full((nb,), fill, dtype=torch.uint8, device="cuda")
            out, idx = gpu_lib.loki_decode(q, P, Kr, V, r, k, workspace=ws, K_lead=Kl, lens=ln)
            torch.cuda.synchronize()
            results.append((out.clone(), idx.clone()))
        assert torch.equal(results[0][1], results[1][1])
        assert torch.equal(_bits(results[0][0]), _bits(results[1][0]))


def test_concurrent_streams_match_sequential(gpu_lib):
    # the library keeps no state between calls: four decodes of different
    # inputs issued on four streams at once, each with its own workspace,
    # equal the same decodes run one after the other
    cases = [cfg_case("C3", S=2048, B=16), cfg_case("C2", S=2048, B=8), cfg_case("C3", S=4096, B=2),
             cfg_case("C5", S=4096, B=1)]
    inputs = []
    for cfg in cases:
        x = make_inputs(cfg)
        inputs.append((cfg, *(dev(x[n]) for n in ("q", "P", "K_rot", "V"))))
    seq = []
    for cfg, q, P, Kr, V in inputs:
        out, idx = gpu_lib.loki_decode(q, P, Kr, V, cfg.r, cfg.k)
        seq.append((out.clone(), idx.clone()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in inputs]
    wss = [torch.empty(gpu_lib.loki_decode_workspace_bytes(c.B, c.Hq, c.Hkv, c.S, c.d, c.r, c.k, q.dtype),
                       dtype=torch.uint8, device="cuda") for c, q, *_ in inputs]
    outs = [torch.empty_like(q) for _, q, *_ in inputs]
    idxs = [torch.empty((c.B, c.Hq, c.k), dtype=torch.int32, device="cuda") for c, *_ in inputs]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (cfg, q, P, Kr, V) in enumerate(inputs):
            with torch.cuda.stream(streams[i]):
                gpu_lib.loki_decode(q, P, Kr, V, cfg.r, cfg.k, out=outs[i], idx=idxs[i], workspace=wss[i])
        torch.cuda.synchronize()
        for i in range(len(inputs)):
            assert torch.equal(idxs[i], seq[i][1]), (rep, i)
            assert torch.equal(_bits(outs[i]), _bits(seq[i][0])), (rep, i)


# ---------------------------------------------------------------- memory-system reference kernels


@pytest.mark.parametrize("nbytes", [16, 16 * 1000 + 16, 64 << 20])
def test_bench_copy_and_read(gpu_lib, nbytes):
    # the copy moves every byte; the read's sink is the XOR of every 32-bit word
    g = torch.Generator().manual_seed(nbytes % 1000)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    s, d = dev(src), torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    gpu_lib.loki_bench_copy(s, d)
    sink = gpu_lib.loki_bench_read(s)
    torch.cuda.synchronize()
    assert torch.equal(d.cpu(), src)
    want = np.bitwise_xor.reduce(src.numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


_DEBUG_RUN = """
import sys, torch
sys.path.insert(0, {root!r})
import rank_key_sparse_amd as rks
from loki_inputs import CONFIGS, make_inputs
cfg = CONFIGS["C3"].scaled(S=2048, B={B})
x = {{n: v.to("cuda") for n, v in make_inputs(cfg).items() if n in ("q", "P", "K_rot", "V")}}
out, idx = rks.loki_decode(x["q"], x["P"], x["K_rot"], x["V"], cfg.r, cfg.k)
torch.cuda.synchronize()
torch.save({{"out": out.cpu(), "idx": idx.cpu()}}, {path!r})
"""


@pytest.mark.parametrize("B", [2, 16])  # two-kernel path, and the fused pair path
def test_debug_mode_same_results(gpu_lib, B, tmp_path):
    # LOKI_DEBUG=1 waits for the stream after every launch step and checks the
    # runtime's error; the results are the default mode's, bit for bit
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = str(tmp_path / "dbg.pt")
    env = dict(os.environ, LOKI_DEBUG="1")
    r = subprocess.run([sys.executable, "-c", _DEBUG_RUN.format(root=root, B=B, path=path)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    got = torch.load(path, weights_only=True)
    cfg = CONFIGS["C3"].scaled(S=2048, B=B)
    x = make_inputs(cfg)
    out, idx = gpu_lib.loki_decode(dev(x["q"]), dev(x["P"]), dev(x["K_rot"]), dev(x["V"]), cfg.r, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(got["idx"], idx.cpu())
    assert torch.equal(got["out"].view(torch.int16), out.cpu().view(torch.int16))
