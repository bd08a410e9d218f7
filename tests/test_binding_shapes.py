"""The Python binding's argument checks on the CPU: every tensor the kernels
write (out, idx, dims, info_loss, the factors A and Bm, the projected caches)
must have exactly the shape the call's sizes give, every input must match the
others, and all of this is checked before the device and before the library
is called.  With CPU tensors of the right shapes the call then stops at the
device check; with one wrong shape it stops at that tensor."""

import pytest
import torch

import rank_key_sparse_amd as rks

B, Hq, Hkv, S, d, r, k = 2, 4, 2, 64, 64, 8, 5
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def decode_args():
    return dict(q=t(B, Hq, d), P=t(Hkv, d, d), K_rot=t(B, Hkv, S, d), V=t(B, Hkv, S, d))


def expect(msg, fn, *a, **kw):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **kw)


def test_decode_right_shapes_reach_the_device_check():
    expect("GPU device", rks.loki_decode, **decode_args(), r=r, k=k,
           out=t(B, Hq, d), idx=t(B, Hq, k, dtype=torch.int32), K_lead=t(B, Hkv, S, r),
           lens=t(B, dtype=torch.int32), workspace=t(100, dtype=torch.uint8))


@pytest.mark.parametrize("name,bad", [
    ("out", t(B, Hq, d - 1)), ("out", t(B, Hq + 1, d)), ("idx", t(B, Hq, k - 1, dtype=torch.int32)),
    ("idx", t(B, Hq, k + 1, dtype=torch.int32)), ("K_lead", t(B, Hkv, S - 1, r)), ("K_lead", t(B, Hkv, S)),
    ("lens", t(B + 1, dtype=torch.int32)), ("workspace", t(4, 25, dtype=torch.uint8)),
])
def test_decode_rejects_wrong_shapes(name, bad):
    expect(name, rks.loki_decode, **decode_args(), r=r, k=k, **{name: bad})


@pytest.mark.parametrize("name,bad", [
    ("P", t(Hkv, d, d - 1)), ("P", t(Hkv + 1, d, d)), ("V", t(B, Hkv, S + 1, d)), ("K_rot", t(B + 1, Hkv, S, d)),
])
def test_decode_rejects_inconsistent_inputs(name, bad):
    a = decode_args()
    a[name] = bad
    expect(name, rks.loki_decode, **a, r=r, k=k)


@pytest.mark.parametrize("name,bad", [
    ("out", t(B, Hq, d + 1)), ("idx", t(B, Hq, k - 1, dtype=torch.int32)), ("dims", t(B, Hq, r - 1, dtype=torch.int32)),
    ("dims", t(B, Hq, r + 1, dtype=torch.int32)), ("info_loss", t(B, Hq + 1, dtype=torch.float32)),
    ("info_loss", t(B * Hq, dtype=torch.float32)),
])
def test_decode_aqua_rejects_wrong_shapes(name, bad):
    expect(name, rks.loki_decode_aqua, **decode_args(), r=r, k=k, **{name: bad})


def test_decode_aqua_right_shapes_reach_the_device_check():
    expect("GPU device", rks.loki_decode_aqua, **decode_args(), r=r, k=k, out=t(B, Hq, d),
           idx=t(B, Hq, k, dtype=torch.int32), dims=t(B, Hq, r, dtype=torch.int32),
           info_loss=t(B, Hq, dtype=torch.float32))


def asym_args():
    return dict(q=t(B, Hq, d), A=t(Hkv, d, d), K_idx=t(B, Hkv, S, r), K=t(B, Hkv, S, d), V=t(B, Hkv, S, d))


@pytest.mark.parametrize("name,bad", [
    ("out", t(B, Hq, d - 1)), ("idx", t(B, Hq, k + 1, dtype=torch.int32)), ("K_idx", t(B, Hkv, S * r)),
    ("K_idx", t(B, Hkv, S + 1, r)), ("A", t(Hkv, d, r)),
])
def test_decode_asym_rejects_wrong_shapes(name, bad):
    a = asym_args()
    if name in a:
        a[name] = bad
        expect(name, rks.loki_decode_asym, **a, r=r, k=k)
    else:
        expect(name, rks.loki_decode_asym, **a, r=r, k=k, **{name: bad})


def test_decode_asym_right_shapes_reach_the_device_check():
    expect("GPU device", rks.loki_decode_asym, **asym_args(), r=r, k=k)


@pytest.mark.parametrize("name,bad", [("A", t(Hkv, d, r)), ("Bm", t(Hkv + 1, d, d)), ("A", t(Hkv * d, d))])
def test_calibrate_asym_rejects_wrong_factor_shapes(name, bad):
    expect(name, rks.loki_calibrate_asym, t(16, Hq, d), t(B, Hkv, S, d), r, **{name: bad})


def test_calibrate_asym_right_shapes_reach_the_device_check():
    expect("GPU device", rks.loki_calibrate_asym, t(16, Hq, d), t(B, Hkv, S, d), r,
           A=t(Hkv, d, d), Bm=t(Hkv, d, d))


@pytest.mark.parametrize("name,bad", [("P", t(Hkv, d, d + 1)), ("eigvals", t(Hkv, d - 1, dtype=torch.float64))])
def test_calibrate_pca_rejects_wrong_shapes(name, bad):
    expect(name, rks.loki_calibrate_pca, t(B, Hkv, S, d), **{name: bad})


@pytest.mark.parametrize("kw", [dict(K_rot=t(B, Hkv, S - 1, d)), dict(R=r, K_lead=t(B, Hkv, S, r + 1)),
                                dict(R=r, K_lead=t(B, Hkv, S, r + 1), lead_only=True)])
def test_project_rejects_wrong_output_shapes(kw):
    name = "K_rot" if "K_rot" in kw else "K_lead"
    expect(name, rks.loki_project_keys, t(B, Hkv, S, d), t(Hkv, d, d), **kw)


def test_append_rejects_wrong_shapes():
    args = dict(k_new=t(B, Hkv, d), v_new=t(B, Hkv, d), P=t(Hkv, d, d), pos=t(B, dtype=torch.int32),
                K_rot=t(B, Hkv, S, d), V=t(B, Hkv, S, d))
    expect("GPU device", rks.loki_append_kv, **args, K_lead=t(B, Hkv, S, r))
    for name, bad in (("v_new", t(B, Hkv, d - 1)), ("pos", t(B + 1, dtype=torch.int32)), ("V", t(B, Hkv, S - 1, d))):
        a = dict(args)
        a[name] = bad
        expect(name, rks.loki_append_kv, **a)
    expect("K_lead", rks.loki_append_kv, **args, K_lead=t(B, Hkv, S + 1, r))


def test_attend_rejects_idx_of_another_head_count():
    expect("idx", rks.loki_attend, *decode_args().values(), t(B, Hq - 1, k, dtype=torch.int32))
    expect("GPU device", rks.loki_attend, *decode_args().values(), t(B, Hq, k, dtype=torch.int32))
