"""The no-allocation decode entry point (loki_decode_noalloc, scratch in a
fixed device array of the library) against the workspace entry point it
varies (loki_decode / loki_decode_lead), through the C ABI: bit-identical
outputs and kept sets on two calls in a row, the second with a smaller
input, on the pair-fused path (with the lead-dims copy) and on a path whose
kernels use the scratch (two-kernel selection and attention partials)."""

import pytest
import torch

import rank_key_sparse_amd as rks
from loki_inputs import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _dev(x):
    return {n: x[n].to("cuda") for n in ("q", "P", "K_rot", "V")}


def _both(gpu_lib, cfg, lead):
    x = _dev(make_inputs(cfg))
    Kl = x["K_rot"][..., :cfg.r].contiguous() if lead else None
    o_ref, i_ref = gpu_lib.loki_decode(x["q"], x["P"], x["K_rot"], x["V"], cfg.r, cfg.k, K_lead=Kl)
    out = torch.full_like(x["q"], float("nan"))
    idx = torch.full((cfg.B, cfg.Hq, cfg.k), -7, dtype=torch.int32, device="cuda")
    gpu_lib.loki_decode_noalloc(x["q"], x["P"], x["K_rot"], x["V"], cfg.r, cfg.k, out, idx, K_lead=Kl)
    torch.cuda.synchronize()
    assert torch.equal(idx, i_ref)
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       o_ref.view(torch.int16) if o_ref.dtype == torch.bfloat16 else o_ref)


@pytest.mark.parametrize("case", [
    ("two_kernel", [CONFIGS["C3"].scaled(S=8192, B=4), CONFIGS["C3"].scaled(S=2048, B=2)], False),
    ("pair_fused_lead", [CONFIGS["C3"].scaled(S=4096, B=16), CONFIGS["C3"].scaled(S=1024, B=16)], True),
    ("f32", [CONFIGS["C1"].replace(B=3, Hq=4, Hkv=2, S=3000, k=200), CONFIGS["C1"]], False),
], ids=lambda c: c[0])
def test_noalloc_matches_workspace_entry_point(gpu_lib, case):
    _, cfgs, lead = case
    for cfg in cfgs:  # two calls in a row, the second smaller
        print(f"\n[noalloc {case[0]}] B={cfg.B} Hq={cfg.Hq} S={cfg.S} r={cfg.r} k={cfg.k}", flush=True)
        _both(gpu_lib, cfg, lead)


def test_noalloc_rejects_sizes_beyond_the_scratch(gpu_lib):
    # C3's shape at 4x the cache length needs more workspace than the fixed array
    lib = rks.load_library()
    need = lib.loki_decode_workspace_bytes(16, 32, 8, 65536, 128, 32, 1024, 1)
    assert need > (48 << 20)
    A = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = rks._ptr(A)
    st = lib.loki_decode_noalloc(p, p, p, None, 0, p, p, p, 16, 32, 8, 65536, 128, 32, 1024, 1, None)
    assert st == 6  # LOKI_ERR_WORKSPACE, before any launch
