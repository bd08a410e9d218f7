"""The C ABI library on the CPU: it loads, exports every entry point that
include/loki.h declares, and rejects every invalid argument with the
documented status before touching HIP (so none of these calls needs a GPU)."""

import ctypes
import os
import re

import pytest

import rank_key_sparse_amd as rks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F32, BF16 = 0, 1
OK, NULL, SHAPE, RANGE, DTYPE, ALIGN, WORKSPACE, UNSUPPORTED, HIP = range(9)

# fake, 16-byte aligned, non-null device addresses: only ever passed to calls
# that must fail validation before any HIP call
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)
NULLP = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return rks.load_library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "loki.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(loki_\w+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert "loki_decode" in names and "loki_project_keys" in names
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(rks.EXPORTED) == names


def test_abi_version_and_status_strings(lib):
    assert lib.loki_abi_version() == 1
    for s in range(10):
        assert lib.loki_status_str(s)
    assert lib.loki_status_str(12345) == b"unknown status"


def decode(lib, q=A, P=A, K=A, V=A, out=A, idx=A, B=1, Hq=4, Hkv=2, S=100, d=128, r=8, k=10,
           dt=BF16, ws=A2, wsb=1 << 30):
    return lib.loki_decode(q, P, K, V, out, idx, B, Hq, Hkv, S, d, r, k, dt, ws, wsb, NULLP)


@pytest.mark.parametrize("kw,want", [
    (dict(q=NULLP), NULL), (dict(P=NULLP), NULL), (dict(K=NULLP), NULL), (dict(V=NULLP), NULL),
    (dict(out=NULLP), NULL), (dict(idx=NULLP), NULL),
    (dict(B=0), SHAPE), (dict(Hq=0), SHAPE), (dict(Hkv=0), SHAPE), (dict(S=0), SHAPE),
    (dict(Hq=5, Hkv=2), SHAPE), (dict(S=(1 << 24) + 1, k=1), SHAPE), (dict(B=70000, Hq=1, Hkv=1), SHAPE),
    (dict(r=0), RANGE), (dict(r=129), RANGE), (dict(k=0), RANGE), (dict(k=101), RANGE),
    (dict(dt=7), DTYPE),
    (dict(d=96), UNSUPPORTED), (dict(Hq=34, Hkv=2), UNSUPPORTED),
    (dict(q=MIS), ALIGN), (dict(V=MIS), ALIGN), (dict(idx=MIS), ALIGN), (dict(ws=MIS), ALIGN),
    (dict(wsb=16), WORKSPACE), (dict(ws=NULLP), NULL),
])
def test_decode_rejects(lib, kw, want):
    assert decode(lib, **kw) == want


def test_project_rejects(lib):
    f = lib.loki_project_keys
    assert f(NULLP, A, A, 1, 1, 8, 128, BF16, NULLP) == NULL
    assert f(A, A, A, 0, 1, 8, 128, BF16, NULLP) == SHAPE
    assert f(A, A, A, 1, 1, 8, 100, BF16, NULLP) == UNSUPPORTED
    assert f(A, A, MIS, 1, 1, 8, 128, BF16, NULLP) == ALIGN
    assert f(A, A, A, 1, 1, 8, 128, 3, NULLP) == DTYPE


def test_append_rejects(lib):
    f = lib.loki_append_kv
    # (k_new, v_new, P, pos, K_rot, V, K_lead, R, B, Hkv, S, d, dt, stream)
    for i in range(6):
        args = [A] * 6
        args[i] = NULLP
        assert f(*args, NULLP, 0, 2, 2, 64, 128, BF16, NULLP) == NULL, i
    assert f(A, A, A, A, A, A, NULLP, 0, 0, 2, 64, 128, BF16, NULLP) == SHAPE
    assert f(A, A, A, A, A, A, NULLP, 0, 2, 2, 0, 128, BF16, NULLP) == SHAPE
    assert f(A, A, A, A, A, A, NULLP, 0, 2, 2, 64, 96, BF16, NULLP) == UNSUPPORTED
    assert f(A, MIS, A, A, A, A, NULLP, 0, 2, 2, 64, 128, BF16, NULLP) == ALIGN
    assert f(A, A, A, A, A, MIS, NULLP, 0, 2, 2, 64, 128, BF16, NULLP) == ALIGN
    assert f(A, A, A, A, A, A, A, 0, 2, 2, 64, 128, BF16, NULLP) == RANGE
    assert f(A, A, A, A, A, A, A, 129, 2, 2, 64, 128, BF16, NULLP) == RANGE
    assert f(A, A, A, A, A, A, A, 12, 2, 2, 64, 128, BF16, NULLP) == UNSUPPORTED
    assert f(A, A, A, A, A, A, MIS, 32, 2, 2, 64, 128, BF16, NULLP) == ALIGN
    assert f(A, A, A, A, A, A, NULLP, 0, 2, 2, 64, 128, 7, NULLP) == DTYPE


def test_decode_varlen_rejects(lib):
    f = lib.loki_decode_varlen
    # (q, P, K_rot, K_lead, R, V, lens, out, idx, B, Hq, Hkv, S, d, r, k, dt, ws, wsb, stream)
    assert f(A, A, A, NULLP, 0, A, NULLP, A, A, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 1 << 30, NULLP) == NULL
    assert f(NULLP, A, A, NULLP, 0, A, A, A, A, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 1 << 30, NULLP) == NULL
    assert f(A, A, A, NULLP, 0, A, A, A, A, 1, 4, 2, 100, 128, 8, 101, BF16, A2, 1 << 30, NULLP) == RANGE
    assert f(A, A, A, A, 4, A, A, A, A, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 1 << 30, NULLP) == RANGE
    assert f(A, A, A, NULLP, 0, A, A, A, A, 1, 5, 2, 100, 128, 8, 10, BF16, A2, 1 << 30, NULLP) == SHAPE
    assert f(A, A, A, NULLP, 0, A, A, A, A, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 16, NULLP) == WORKSPACE


def test_stage_entry_points_reject(lib):
    assert lib.loki_scores(A, A, A, NULLP, 1, 1, 1, 8, 64, 4, F32, A2, 1 << 20, NULLP) == NULL
    assert lib.loki_scores(A, A, A, A, 1, 1, 1, 8, 64, 65, F32, A2, 1 << 20, NULLP) == RANGE
    assert lib.loki_select_topk(A, A, 4, 100, 0, A2, 1 << 20, NULLP) == RANGE
    assert lib.loki_select_topk(A, A, 0, 100, 5, A2, 1 << 20, NULLP) == SHAPE
    assert lib.loki_select_topk(A, MIS, 4, 100, 5, A2, 1 << 20, NULLP) == ALIGN
    assert lib.loki_select_topk(A, A, 4, 100, 5, A2, 8, NULLP) == WORKSPACE
    assert lib.loki_attend(A, A, A, A, NULLP, A, 1, 2, 1, 50, 64, 5, BF16, A2, 1 << 20, NULLP) == NULL
    assert lib.loki_attend(A, A, A, A, A, A, 1, 2, 1, 50, 64, 51, BF16, A2, 1 << 20, NULLP) == RANGE


def test_workspace_sizes(lib):
    ws = lib.loki_decode_workspace_bytes
    assert ws(1, 4, 2, 100, 128, 8, 10, BF16) > 0
    assert ws(1, 4, 2, 100, 128, 0, 10, BF16) == 0
    assert ws(1, 4, 2, 100, 96, 8, 10, BF16) == 0
    assert ws(1, 5, 2, 100, 128, 8, 10, BF16) == 0
    # must hold at least the fp32 keys and the rotated queries of every head
    B, Hq, Hkv, S, d = 16, 32, 8, 16384, 128
    n = ws(B, Hq, Hkv, S, d, 32, 1024, BF16)
    assert n >= B * Hq * S * 4 + B * Hq * d * 4
    assert n % 256 == 0
    # independent of r and k (one workspace serves every stage entry point)
    assert n == ws(B, Hq, Hkv, S, d, 1, 1, BF16) == ws(B, Hq, Hkv, S, d, d, S, BF16)
    assert lib.loki_select_workspace_bytes(4, 100, 5) >= 4 * 100 * 4
    assert lib.loki_select_workspace_bytes(4, 100, 101) == 0


def test_python_binding_validates_before_the_library():
    import torch
    with pytest.raises(ValueError):
        rks.loki_decode(torch.zeros(1, 1, 64), torch.zeros(1, 64, 64), torch.zeros(1, 1, 8, 64),
                        torch.zeros(1, 1, 8, 64), r=4, k=2)  # CPU tensors are rejected


def test_lead_entry_points_reject(lib):
    f = lib.loki_decode_lead
    def call(Kl=A, R=32, r=8, d=128, dt=BF16):
        return f(A, A, A, Kl, R, A, A, A, 1, 4, 2, 100, d, r, 10, dt, A2, 1 << 30, NULLP)
    assert call(Kl=NULLP) == NULL
    assert call(R=0) == RANGE
    assert call(R=129) == RANGE
    assert call(R=8, r=9) == RANGE
    assert call(R=12) == UNSUPPORTED       # 24 bytes per token: not a multiple of 16
    assert call(Kl=MIS) == ALIGN
    g = lib.loki_project_keys_lead
    assert g(A, A, A, NULLP, 32, 1, 1, 8, 128, BF16, NULLP) == NULL
    assert g(A, A, A, A, 200, 1, 1, 8, 128, BF16, NULLP) == RANGE
    assert g(A, A, A, A, 6, 1, 1, 8, 128, F32, NULLP) == UNSUPPORTED


def test_calibrate_rejects(lib):
    f = lib.loki_calibrate_pca
    # (K, P, eigvals, B, Hkv, S, d, dt, ws, wsb, stream)
    big = 1 << 40
    assert f(NULLP, A, A, 1, 2, 512, 128, BF16, A2, big, NULLP) == NULL
    assert f(A, NULLP, A, 1, 2, 512, 128, BF16, A2, big, NULLP) == NULL
    assert f(A, A, A, 0, 2, 512, 128, BF16, A2, big, NULLP) == SHAPE
    assert f(A, A, A, 1, 0, 512, 128, BF16, A2, big, NULLP) == SHAPE
    assert f(A, A, A, 1, 2, 0, 128, BF16, A2, big, NULLP) == SHAPE
    assert f(A, A, A, 1 << 16, 2, 1 << 16, 128, BF16, A2, big, NULLP) == SHAPE  # B*S >= 2^31
    assert f(A, A, A, 1, 2, 512, 96, BF16, A2, big, NULLP) == UNSUPPORTED
    assert f(A, A, A, 1, 2, 512, 128, 5, A2, big, NULLP) == DTYPE
    assert f(MIS, A, A, 1, 2, 512, 128, BF16, A2, big, NULLP) == ALIGN
    assert f(A, MIS, A, 1, 2, 512, 128, BF16, A2, big, NULLP) == ALIGN
    assert f(A, A, ctypes.c_void_p(0x10004), 1, 2, 512, 128, BF16, A2, big, NULLP) == ALIGN
    need = lib.loki_calibrate_workspace_bytes(1, 2, 512, 128)
    assert need >= 3 * 2 * 128 * 128 * 8
    assert f(A, A, A, 1, 2, 512, 128, BF16, A2, need - 1, NULLP) == WORKSPACE
    assert f(A, A, A, 1, 2, 512, 128, BF16, NULLP, need, NULLP) == NULL
    assert lib.loki_calibrate_workspace_bytes(1, 2, 512, 100) == 0
    assert lib.loki_calibrate_workspace_bytes(1 << 16, 2, 1 << 16, 128) == 0
    g = lib.loki_calibrate_pca_profiled
    assert g(A, A, A, 1, 2, 512, 128, BF16, A2, big, NULLP, NULLP) == NULL


def test_decode_aqua_rejects(lib):
    f = lib.loki_decode_aqua
    # (q, P, K_rot, V, lens, out, idx, dims, info, B, Hq, Hkv, S, d, r, k, dt, ws, wsb, stream)
    base = [A, A, A, A, NULLP, A, A, NULLP, NULLP, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 1 << 30, NULLP]

    def call(**kw):
        a = list(base)
        names = ["q", "P", "K", "V", "lens", "out", "idx", "dims", "info", "B", "Hq", "Hkv", "S", "d", "r", "k",
                 "dt", "ws", "wsb"]
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a)

    for n in ("q", "P", "K", "V", "out", "idx"):
        assert call(**{n: NULLP}) == NULL, n
    assert call(r=0) == RANGE
    assert call(r=129) == RANGE
    assert call(k=101) == RANGE
    assert call(Hq=5) == SHAPE
    assert call(d=96) == UNSUPPORTED
    assert call(dt=9) == DTYPE
    assert call(dims=ctypes.c_void_p(0x10002)) == ALIGN
    assert call(info=ctypes.c_void_p(0x10001)) == ALIGN
    assert call(out=MIS) == ALIGN
    assert call(wsb=16) == WORKSPACE


def test_decode_asym_rejects(lib):
    f = lib.loki_decode_asym
    # (q, A, K_idx, R, K, V, lens, out, idx, B, Hq, Hkv, S, d, r, k, dt, ws, wsb, stream)
    names = ["q", "A", "K_idx", "R", "K", "V", "lens", "out", "idx", "B", "Hq", "Hkv", "S", "d", "r", "k", "dt",
             "ws", "wsb"]
    base = [A, A, A, 32, A, A, NULLP, A, A, 1, 4, 2, 100, 128, 8, 10, BF16, A2, 1 << 30]

    def call(**kw):
        a = list(base)
        for n, v in kw.items():
            a[names.index(n)] = v
        return f(*a, NULLP)

    for n in ("q", "A", "K_idx", "K", "V", "out", "idx"):
        assert call(**{n: NULLP}) == NULL, n
    assert call(r=33) == RANGE          # r > R
    assert call(R=0) == RANGE
    assert call(R=12) == UNSUPPORTED    # R * 2 bytes not a multiple of 16
    assert call(K_idx=MIS) == ALIGN
    assert call(k=0) == RANGE
    assert call(wsb=8) == WORKSPACE
    assert lib.loki_decode_asym_profiled(*base, NULLP, NULLP) == NULL


def test_project_lead_only_rejects(lib):
    f = lib.loki_project_keys_lead
    # K_rot may be NULL; K_lead then carries the output checks
    assert f(A, A, NULLP, NULLP, 32, 1, 1, 8, 128, BF16, NULLP) == NULL
    assert f(A, A, NULLP, MIS, 32, 1, 1, 8, 128, BF16, NULLP) == ALIGN
    assert f(A, A, NULLP, A, 0, 1, 1, 8, 128, BF16, NULLP) == RANGE


def test_calibrate_asym_rejects(lib):
    f = lib.loki_calibrate_asym
    # (q_samples, K, A, Bm, N, Hq, B, Hkv, S, d, r, dt, ws, wsb, stream)
    big = 1 << 40
    assert f(NULLP, A, A, A, 100, 4, 1, 2, 50, 128, 8, BF16, A2, big, NULLP) == NULL
    assert f(A, A, A, NULLP, 100, 4, 1, 2, 50, 128, 8, BF16, A2, big, NULLP) == NULL
    assert f(A, A, A, A, 100, 5, 1, 2, 50, 128, 8, BF16, A2, big, NULLP) == SHAPE
    assert f(A, A, A, A, 0, 4, 1, 2, 50, 128, 8, BF16, A2, big, NULLP) == SHAPE
    assert f(A, A, A, A, 100, 4, 1, 2, 50, 96, 8, BF16, A2, big, NULLP) == UNSUPPORTED
    assert f(A, A, A, A, 100, 4, 1, 2, 50, 128, 0, BF16, A2, big, NULLP) == RANGE
    assert f(A, A, A, A, 100, 4, 1, 2, 50, 128, 129, BF16, A2, big, NULLP) == RANGE
    assert f(A, A, MIS, A, 100, 4, 1, 2, 50, 128, 8, BF16, A2, big, NULLP) == ALIGN
    assert f(A, A, A, A, 100, 4, 1, 2, 50, 128, 8, 3, A2, big, NULLP) == DTYPE
    need = lib.loki_calibrate_asym_workspace_bytes(100, 4, 1, 2, 50, 128, 8)
    assert need > 0
    assert f(A, A, A, A, 100, 4, 1, 2, 50, 128, 8, BF16, A2, need - 1, NULLP) == WORKSPACE


def test_bench_kernels_reject(lib):
    Z = ctypes.c_size_t
    assert lib.loki_bench_copy(A, A2, Z(100), NULLP) == SHAPE          # not a multiple of 16
    assert lib.loki_bench_copy(NULLP, A2, Z(64), NULLP) == NULL
    assert lib.loki_bench_copy(A, NULLP, Z(64), NULLP) == NULL
    assert lib.loki_bench_copy(MIS, A2, Z(64), NULLP) == ALIGN
    assert lib.loki_bench_copy(NULLP, NULLP, Z(0), NULLP) == OK         # nothing to do
    assert lib.loki_bench_read(A, Z(24), A2, NULLP) == SHAPE
    assert lib.loki_bench_read(NULLP, Z(64), A2, NULLP) == NULL
    assert lib.loki_bench_read(A, Z(64), NULLP, NULLP) == NULL
    assert lib.loki_bench_read(MIS, Z(64), A2, NULLP) == ALIGN
    assert lib.loki_bench_read(A, Z(64), ctypes.c_void_p(0x20002), NULLP) == ALIGN


def test_decode_noalloc_rejects_before_hip(lib):
    def call(B=1, Hq=4, Hkv=2, S=100, d=128, r=8, k=10, dt=BF16):
        return lib.loki_decode_noalloc(A, A, A, NULLP, 0, A, A, A, B, Hq, Hkv, S, d, r, k, dt, NULLP)
    assert call(B=0) == SHAPE
    assert call(Hq=5) == SHAPE
    assert call(d=96) == UNSUPPORTED
    assert call(r=0) == RANGE and call(k=101) == RANGE
    assert call(dt=7) == DTYPE
    # a workspace beyond the fixed scratch (48 MiB) is rejected before any HIP call
    assert lib.loki_decode_workspace_bytes(16, 32, 8, 65536, 128, 32, 1024, BF16) > (48 << 20)
    assert call(B=16, Hq=32, Hkv=8, S=65536, r=32, k=1024) == WORKSPACE
