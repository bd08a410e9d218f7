"""Python binding of libloki, the gfx950 low-rank-key sparse decode-attention library.

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory and the current HIP stream.  The entry points
mirror the C ABI (``include/loki.h``) name for name:

* :func:`loki_calibrate_pca` -- the basis ``P`` itself: principal directions of sampled keys;
* :func:`loki_project_keys` -- ``K_rot = K P`` per key/value head;
* :func:`loki_append_kv` -- one decode step's new key (rotated) and value written into the caches;
* :func:`loki_decode` -- one Loki decode step -> ``(out, idx)``;
* :func:`loki_scores`, :func:`loki_select_topk`, :func:`loki_attend` -- the
  decode stages alone (same kernels), for stage-level checks;
* :func:`loki_bench_copy`, :func:`loki_bench_read` -- memory-system reference
  kernels (measurement only).

If the built library is missing the calls raise; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libloki.so")

LOKI_F32, LOKI_BF16 = 0, 1
_DT = {torch.float32: LOKI_F32, torch.bfloat16: LOKI_BF16}

_STATUS = {
    0: "LOKI_OK", 1: "LOKI_ERR_NULL", 2: "LOKI_ERR_SHAPE", 3: "LOKI_ERR_RANGE",
    4: "LOKI_ERR_DTYPE", 5: "LOKI_ERR_ALIGN", 6: "LOKI_ERR_WORKSPACE",
    7: "LOKI_ERR_UNSUPPORTED", 8: "LOKI_ERR_HIP", 9: "LOKI_ERR_INTERNAL",
}


class LokiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t

_SIGS = {
    "loki_abi_version": ([], ctypes.c_int),
    "loki_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "loki_project_keys": ([_P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P], ctypes.c_int),
    "loki_decode_workspace_bytes": ([_I, _I, _I, _I, _I, _I, _I, ctypes.c_int], _Z),
    "loki_append_kv": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P], ctypes.c_int),
    "loki_project_keys_lead": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_int, _P], ctypes.c_int),
    "loki_decode": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P],
                    ctypes.c_int),
    "loki_decode_lead": ([_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int,
                          _P, _Z, _P], ctypes.c_int),
    "loki_decode_varlen": ([_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int,
                            _P, _Z, _P], ctypes.c_int),
    "loki_decode_profiled": ([_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                              ctypes.c_int, _P, _Z, _P, _P], ctypes.c_int),
    "loki_scores": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P], ctypes.c_int),
    "loki_select_workspace_bytes": ([_I, _I, _I], _Z),
    "loki_select_topk": ([_P, _P, _I, _I, _I, _P, _Z, _P], ctypes.c_int),
    "loki_attend": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P],
                    ctypes.c_int),
    "loki_decode_aqua": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P],
                         ctypes.c_int),
    "loki_decode_aqua_profiled": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int,
                                   _P, _Z, _P, _P], ctypes.c_int),
    "loki_decode_asym": ([_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P],
                         ctypes.c_int),
    "loki_decode_asym_profiled": ([_P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int,
                                   _P, _Z, _P, _P], ctypes.c_int),
    "loki_calibrate_asym_workspace_bytes": ([_I, _I, _I, _I, _I, _I, _I], _Z),
    "loki_calibrate_asym": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P], ctypes.c_int),
    "loki_calibrate_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "loki_calibrate_pca": ([_P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P], ctypes.c_int),
    "loki_calibrate_pca_profiled": ([_P, _P, _P, _I, _I, _I, _I, ctypes.c_int, _P, _Z, _P, _P], ctypes.c_int),
    "loki_decode_noalloc": ([_P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, ctypes.c_int, _P],
                            ctypes.c_int),
    "loki_bench_copy": ([_P, _P, _Z, _P], ctypes.c_int),
    "loki_bench_read": ([_P, _Z, _P, _P], ctypes.c_int),
}

EXPORTED = tuple(_SIGS)


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of libloki.so (the in-tree
    build, or the file that the LOKI_LIBRARY environment variable names, e.g.
    a host-sanitized build of the same sources)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LOKI_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libloki.so not built ({p}); run `python -m rank_key_sparse_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().loki_status_str(status).decode()
        raise LokiError(status, msg)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None, shape=None):
    """Metadata checks of one tensor argument: type, dtype, rank, exact shape
    (every buffer the kernels write is sized from the call's sizes, so an
    output of another shape would be written out of bounds), contiguity and
    the device of the call.  That the call's device is a GPU is checked once
    per call by _gpu, after all of these."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _gpu(t: torch.Tensor, name: str) -> None:
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype} (fp32 or bf16)")
    return _DT[t.dtype]


def loki_project_keys(K: torch.Tensor, P: torch.Tensor, K_rot: torch.Tensor | None = None,
                      R: int | None = None, K_lead: torch.Tensor | None = None, lead_only: bool = False):
    """``K_rot[b, kv] = K[b, kv] @ P[kv]``; K [B,Hkv,S,d], P [Hkv,d,d].

    With ``R``, also writes the lead-dims copy ``K_lead = K_rot[..., :R]``
    (contiguous) in the same pass and returns ``(K_rot, K_lead)``; with
    ``lead_only`` only ``K_lead`` is written and returned (a key index).
    """
    if lead_only:
        if R is None:
            raise ValueError("lead_only needs R")
        _need(K, "K", ndim=4)
        B, Hkv, S, d = K.shape
        _need(P, "P", dtype=K.dtype, device=K.device, shape=(Hkv, d, d))
        if K_lead is None:
            K_lead = torch.empty((B, Hkv, S, R), dtype=K.dtype, device=K.device)
        _need(K_lead, "K_lead", dtype=K.dtype, device=K.device, shape=(B, Hkv, S, R))
        _gpu(K, "K")
        _check(load_library().loki_project_keys_lead(_ptr(K), _ptr(P), None, _ptr(K_lead), R, B, Hkv, S, d,
                                                     _dtype_code(K), _stream(K)))
        return K_lead
    _need(K, "K", ndim=4)
    B, Hkv, S, d = K.shape
    _need(P, "P", dtype=K.dtype, device=K.device, shape=(Hkv, d, d))
    if K_rot is None:
        K_rot = torch.empty_like(K)
    _need(K_rot, "K_rot", dtype=K.dtype, device=K.device, shape=K.shape)
    if R is not None:
        if K_lead is None:
            K_lead = torch.empty((B, Hkv, S, R), dtype=K.dtype, device=K.device)
        _need(K_lead, "K_lead", dtype=K.dtype, device=K.device, shape=(B, Hkv, S, R))
    _gpu(K, "K")
    lib = load_library()
    if R is None:
        _check(lib.loki_project_keys(_ptr(K), _ptr(P), _ptr(K_rot), B, Hkv, S, d, _dtype_code(K), _stream(K)))
        return K_rot
    _check(lib.loki_project_keys_lead(_ptr(K), _ptr(P), _ptr(K_rot), _ptr(K_lead), R, B, Hkv, S, d,
                                      _dtype_code(K), _stream(K)))
    return K_rot, K_lead


def loki_decode_aqua(q, P, K_rot, V, r: int, k: int, lens=None, out=None, idx=None, workspace=None,
                     dims=None, info_loss=None, events=None):
    """Decode step whose approximate scores use, per query head, the ``r``
    rotated dims where the query is largest in magnitude (the token selection
    and exact attention are as in :func:`loki_decode`).  Returns ``(out, idx,
    dims [B,Hq,r] int32, info_loss [B,Hq] float32)``."""
    B, Hq, Hkv, S, d = _shapes(q, P, K_rot)
    dev = q.device
    _need(V, "V", dtype=q.dtype, device=dev, shape=K_rot.shape)
    out = torch.empty_like(q) if out is None else out
    idx = torch.empty((B, Hq, k), dtype=torch.int32, device=dev) if idx is None else idx
    dims = torch.empty((B, Hq, r), dtype=torch.int32, device=dev) if dims is None else dims
    info_loss = torch.empty((B, Hq), dtype=torch.float32, device=dev) if info_loss is None else info_loss
    _need(out, "out", dtype=q.dtype, device=dev, shape=(B, Hq, d))
    _need(idx, "idx", dtype=torch.int32, device=dev, shape=(B, Hq, k))
    _need(dims, "dims", dtype=torch.int32, device=dev, shape=(B, Hq, r))
    _need(info_loss, "info_loss", dtype=torch.float32, device=dev, shape=(B, Hq))
    if lens is not None:
        _need(lens, "lens", dtype=torch.int32, device=dev, shape=(B,))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    _gpu(q, "q")
    dt = _dtype_code(q)
    lib = load_library()
    if workspace is None:
        workspace = torch.empty(max(1, loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, q.dtype)),
                                dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(P), _ptr(K_rot), _ptr(V), _ptr(lens), _ptr(out), _ptr(idx), _ptr(dims), _ptr(info_loss),
            B, Hq, Hkv, S, d, r, k, dt, _ptr(workspace), workspace.numel())
    if events is None:
        _check(lib.loki_decode_aqua(*args, _stream(q)))
    else:
        if len(events) != 6:
            raise ValueError("events must hold 6 torch.cuda.Event objects")
        arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check(lib.loki_decode_aqua_profiled(*args, arr, _stream(q)))
    return out, idx, dims, info_loss


def loki_decode_asym(q, A, K_idx, K, V, r: int, k: int, lens=None, out=None, idx=None, workspace=None,
                     events=None):
    """Decode step with an asymmetric scoring index: scores ``(q A[kv])[:r] .
    K_idx[..., :r]``, the k best tokens, exact attention with ``q`` over the
    unrotated keys ``K``.  A [Hkv,d,d] (first r columns used), K_idx
    [B,Hkv,S,R].  Returns ``(out, idx)``."""
    B, Hq, Hkv, S, d = _shapes(q, A, K, "A", "K")
    dev = q.device
    _need(K_idx, "K_idx", dtype=q.dtype, ndim=4, device=dev)
    R = K_idx.shape[3]
    _need(K_idx, "K_idx", shape=(B, Hkv, S, R))
    _need(V, "V", dtype=q.dtype, device=dev, shape=K.shape)
    out = torch.empty_like(q) if out is None else out
    idx = torch.empty((B, Hq, k), dtype=torch.int32, device=dev) if idx is None else idx
    _need(out, "out", dtype=q.dtype, device=dev, shape=(B, Hq, d))
    _need(idx, "idx", dtype=torch.int32, device=dev, shape=(B, Hq, k))
    if lens is not None:
        _need(lens, "lens", dtype=torch.int32, device=dev, shape=(B,))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    _gpu(q, "q")
    lib = load_library()
    if workspace is None:
        workspace = torch.empty(max(1, loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, q.dtype)),
                                dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(A), _ptr(K_idx), R, _ptr(K), _ptr(V), _ptr(lens), _ptr(out), _ptr(idx), B, Hq, Hkv, S,
            d, r, k, _dtype_code(q), _ptr(workspace), workspace.numel())
    if events is None:
        _check(lib.loki_decode_asym(*args, _stream(q)))
    else:
        if len(events) != 6:
            raise ValueError("events must hold 6 torch.cuda.Event objects")
        arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check(lib.loki_decode_asym_profiled(*args, arr, _stream(q)))
    return out, idx


def loki_calibrate_asym(q_samples, K, r: int, A=None, Bm=None, workspace=None):
    """Asymmetric scoring index factors from query samples [N,Hq,d] and keys
    [B,Hkv,S,d]: ``(A, Bm)``, each [Hkv,d,d] in the keys' dtype with the
    rank-r factors in the first r columns (zeros after)."""
    _need(q_samples, "q_samples", ndim=3)
    dev = q_samples.device
    _need(K, "K", dtype=q_samples.dtype, ndim=4, device=dev)
    N, Hq, d = q_samples.shape
    B, Hkv, S, dk = K.shape
    if dk != d:
        raise ValueError("inconsistent head dims")
    A = torch.empty((Hkv, d, d), dtype=K.dtype, device=dev) if A is None else A
    Bm = torch.empty((Hkv, d, d), dtype=K.dtype, device=dev) if Bm is None else Bm
    _need(A, "A", dtype=K.dtype, device=dev, shape=(Hkv, d, d))
    _need(Bm, "Bm", dtype=K.dtype, device=dev, shape=(Hkv, d, d))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    _gpu(K, "K")
    lib = load_library()
    if workspace is None:
        nb = int(lib.loki_calibrate_asym_workspace_bytes(N, Hq, B, Hkv, S, d, r))
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    _check(lib.loki_calibrate_asym(_ptr(q_samples), _ptr(K), _ptr(A), _ptr(Bm), N, Hq, B, Hkv, S, d, r,
                                   _dtype_code(K), _ptr(workspace), workspace.numel(), _stream(K)))
    return A, Bm


def loki_calibrate_workspace_bytes(B: int, Hkv: int, S: int, d: int) -> int:
    return int(load_library().loki_calibrate_workspace_bytes(B, Hkv, S, d))


def loki_calibrate_pca(K: torch.Tensor, P: torch.Tensor | None = None, eigvals: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, events=None):
    """Principal basis of sampled keys K [B,Hkv,S,d] (cache layout), per key head:
    returns ``(P [Hkv,d,d] in K's dtype, eigvals [Hkv,d] float64)``, columns of P in
    decreasing eigenvalue order of ``A^T A`` (A = the head's key rows), each
    column's largest-magnitude entry positive.  ``events``: 4 torch.cuda.Event
    recorded at the stage boundaries (measurement)."""
    _need(K, "K", ndim=4)
    B, Hkv, S, d = K.shape
    dev = K.device
    if P is None:
        P = torch.empty((Hkv, d, d), dtype=K.dtype, device=dev)
    _need(P, "P", dtype=K.dtype, device=dev, shape=(Hkv, d, d))
    if eigvals is None:
        eigvals = torch.empty((Hkv, d), dtype=torch.float64, device=dev)
    _need(eigvals, "eigvals", dtype=torch.float64, device=dev, shape=(Hkv, d))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    _gpu(K, "K")
    lib = load_library()
    nbytes = int(lib.loki_calibrate_workspace_bytes(B, Hkv, S, d))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    if events is None:
        _check(lib.loki_calibrate_pca(_ptr(K), _ptr(P), _ptr(eigvals), B, Hkv, S, d, _dtype_code(K),
                                      _ptr(workspace), workspace.numel(), _stream(K)))
    else:
        if len(events) != 4:
            raise ValueError("events must hold 4 torch.cuda.Event objects")
        arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check(lib.loki_calibrate_pca_profiled(_ptr(K), _ptr(P), _ptr(eigvals), B, Hkv, S, d, _dtype_code(K),
                                               _ptr(workspace), workspace.numel(), arr, _stream(K)))
    return P, eigvals


def loki_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, P: torch.Tensor, pos: torch.Tensor,
                   K_rot: torch.Tensor, V: torch.Tensor, K_lead: torch.Tensor | None = None) -> None:
    """Writes one new token per (b, kv) into the caches in place:
    ``K_rot[b, kv, pos[b]] = k_new[b, kv] @ P[kv]``, ``V[b, kv, pos[b]] = v_new[b, kv]``
    and, with ``K_lead``, its leading ``R = K_lead.shape[-1]`` dims.  ``pos`` is an int32
    device tensor [B]; positions outside [0, S) write nothing."""
    _need(k_new, "k_new", ndim=3)
    dev = k_new.device
    B, Hkv, d = k_new.shape
    _need(K_rot, "K_rot", dtype=k_new.dtype, ndim=4, device=dev)
    S = K_rot.shape[2]
    _need(K_rot, "K_rot", shape=(B, Hkv, S, d))
    _need(v_new, "v_new", dtype=k_new.dtype, device=dev, shape=(B, Hkv, d))
    _need(P, "P", dtype=k_new.dtype, device=dev, shape=(Hkv, d, d))
    _need(pos, "pos", dtype=torch.int32, device=dev, shape=(B,))
    _need(V, "V", dtype=k_new.dtype, device=dev, shape=(B, Hkv, S, d))
    R = 0
    if K_lead is not None:
        _need(K_lead, "K_lead", dtype=k_new.dtype, ndim=4, device=dev)
        R = K_lead.shape[-1]
        _need(K_lead, "K_lead", shape=(B, Hkv, S, R))
    _gpu(k_new, "k_new")
    _check(load_library().loki_append_kv(_ptr(k_new), _ptr(v_new), _ptr(P), _ptr(pos), _ptr(K_rot), _ptr(V),
                                         _ptr(K_lead), R, B, Hkv, S, d, _dtype_code(k_new), _stream(k_new)))


def loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, dtype) -> int:
    return int(load_library().loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, _DT[dtype]))


def _shapes(q, P, K_rot, pname="P", kname="K_rot"):
    """Sizes of a decode-family call from q [B,Hq,d] and the cache [B,Hkv,S,d];
    the basis (or query-side matrix) must be [Hkv,d,d]."""
    _need(q, "q", ndim=3)
    _need(K_rot, kname, dtype=q.dtype, ndim=4, device=q.device)
    B, Hq, d = q.shape
    Hkv, S = K_rot.shape[1], K_rot.shape[2]
    _need(K_rot, kname, shape=(B, Hkv, S, d))
    _need(P, pname, dtype=q.dtype, device=q.device, shape=(Hkv, d, d))
    return B, Hq, Hkv, S, d


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    return workspace


def loki_decode(q, P, K_rot, V, r: int, k: int, out=None, idx=None, workspace=None, K_lead=None,
                events=None, lens=None):
    """One Loki decode step.  Returns ``(out [B,Hq,d], idx [B,Hq,k] int32 ascending)``.

    With ``K_lead`` ([B,Hkv,S,R], the leading R >= r dims of K_rot) the
    approximate scores stream from it instead of from K_rot's rows.  With
    ``events`` (six recorded-once torch.cuda.Event objects) the instrumented
    entry point records them at the stage boundaries.  With ``lens`` (int32
    [B] on the device) sequence b holds only its first ``lens[b]`` cached
    tokens; idx rows of sequences shorter than k end with -1.
    """
    B, Hq, Hkv, S, d = _shapes(q, P, K_rot)
    dev = q.device
    _need(V, "V", dtype=q.dtype, device=dev, shape=K_rot.shape)
    if out is None:
        out = torch.empty_like(q)
    if idx is None:
        idx = torch.empty((B, Hq, k), dtype=torch.int32, device=dev)
    _need(out, "out", dtype=q.dtype, device=dev, shape=(B, Hq, d))
    _need(idx, "idx", dtype=torch.int32, device=dev, shape=(B, Hq, k))
    if K_lead is not None:
        _need(K_lead, "K_lead", dtype=q.dtype, ndim=4, device=dev)
        _need(K_lead, "K_lead", shape=(B, Hkv, S, K_lead.shape[3]))
    if lens is not None:
        _need(lens, "lens", dtype=torch.int32, device=dev, shape=(B,))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=dev)
    _gpu(q, "q")
    lib = load_library()
    dt = _dtype_code(q)
    nbytes = int(lib.loki_decode_workspace_bytes(B, Hq, Hkv, S, d, r, k, dt))
    ws = _workspace(nbytes, dev, workspace)
    if events is not None:
        if len(events) != 6:
            raise ValueError("events must hold 6 torch.cuda.Event objects")
        arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        _check(lib.loki_decode_profiled(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(K_lead),
                                        0 if K_lead is None else K_lead.shape[3], _ptr(V), _ptr(lens),
                                        _ptr(out), _ptr(idx), B, Hq, Hkv, S, d, r, k, dt, _ptr(ws), ws.numel(),
                                        arr, _stream(q)))
    elif lens is not None:
        _check(lib.loki_decode_varlen(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(K_lead),
                                      0 if K_lead is None else K_lead.shape[3], _ptr(V), _ptr(lens), _ptr(out),
                                      _ptr(idx), B, Hq, Hkv, S, d, r, k, dt, _ptr(ws), ws.numel(), _stream(q)))
    elif K_lead is None:
        _check(lib.loki_decode(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(V), _ptr(out), _ptr(idx),
                               B, Hq, Hkv, S, d, r, k, dt, _ptr(ws), ws.numel(), _stream(q)))
    else:
        _check(lib.loki_decode_lead(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(K_lead), K_lead.shape[3],
                                    _ptr(V), _ptr(out), _ptr(idx), B, Hq, Hkv, S, d, r, k, dt,
                                    _ptr(ws), ws.numel(), _stream(q)))
    return out, idx


def loki_scores(q, P, K_rot, r: int, workspace=None):
    """Approximate scores ``[B,Hq,S]`` fp32 over the leading ``r`` rotated dims."""
    B, Hq, Hkv, S, d = _shapes(q, P, K_rot)
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
    _gpu(q, "q")
    lib = load_library()
    dt = _dtype_code(q)
    nbytes = int(lib.loki_decode_workspace_bytes(B, Hq, Hkv, S, d, max(1, min(r, d)), 1, dt))
    ws = _workspace(nbytes, q.device, workspace)
    s = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib.loki_scores(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(s), B, Hq, Hkv, S, d, r, dt,
                           _ptr(ws), ws.numel(), _stream(q)))
    return s


def loki_select_topk(scores: torch.Tensor, k: int, workspace=None) -> torch.Tensor:
    """Top-k indices (ascending, ties -> lower index) of each row of fp32 ``scores [..., S]``."""
    _need(scores, "scores", dtype=torch.float32)
    if scores.dim() < 1:
        raise ValueError("scores must have a last (token) dim")
    S = scores.shape[-1]
    rows = scores.numel() // max(S, 1)
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=scores.device)
    _gpu(scores, "scores")
    lib = load_library()
    nbytes = int(lib.loki_select_workspace_bytes(rows, S, k))
    ws = _workspace(nbytes, scores.device, workspace)
    idx = torch.empty((*scores.shape[:-1], k), dtype=torch.int32, device=scores.device)
    _check(lib.loki_select_topk(_ptr(scores), _ptr(idx), rows, S, k, _ptr(ws), ws.numel(),
                                _stream(scores)))
    return idx


def loki_attend(q, P, K_rot, V, idx, workspace=None):
    """Exact softmax attention over a given kept set ``idx [B,Hq,k]`` (int32)."""
    B, Hq, Hkv, S, d = _shapes(q, P, K_rot)
    _need(V, "V", dtype=q.dtype, device=q.device, shape=K_rot.shape)
    _need(idx, "idx", dtype=torch.int32, ndim=3, device=q.device)
    k = idx.shape[-1]
    _need(idx, "idx", shape=(B, Hq, k))
    if workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, ndim=1, device=q.device)
    _gpu(q, "q")
    lib = load_library()
    dt = _dtype_code(q)
    nbytes = int(lib.loki_decode_workspace_bytes(B, Hq, Hkv, S, d, d, k, dt))
    ws = _workspace(nbytes, q.device, workspace)
    out = torch.empty_like(q)
    _check(lib.loki_attend(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(V), _ptr(idx), _ptr(out),
                           B, Hq, Hkv, S, d, k, dt, _ptr(ws), ws.numel(), _stream(q)))
    return out


def loki_bench_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Plain copy of src's bytes into dst (same number of bytes, a multiple of
    16): the reference kernel for the memory-system figures."""
    _need(src, "src")
    _need(dst, "dst", device=src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    _gpu(src, "src")
    _check(load_library().loki_bench_copy(_ptr(src), _ptr(dst), nbytes, _stream(src)))


def loki_bench_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Plain streaming read of src's bytes; returns the device uint32 sink
    (int32 tensor of one element, zeroed first) that holds the XOR of every
    32-bit word read."""
    _need(src, "src")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    _need(sink, "sink", dtype=torch.int32, device=src.device, shape=(1,))
    _gpu(src, "src")
    _check(load_library().loki_bench_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src)))
    return sink


def loki_decode_noalloc(q, P, K_rot, V, r: int, k: int, out, idx, K_lead=None):
    """loki_decode (with K_lead: loki_decode_lead) with the library's own fixed
    device scratch instead of a workspace: for callers that cannot allocate.
    out [B,Hq,d] and idx [B,Hq,k] int32 are the caller's; this call allocates
    nothing.  Calls that overlap on one GPU share the scratch and race."""
    B, Hq, Hkv, S, d = _shapes(q, P, K_rot)
    dev = q.device
    _need(V, "V", dtype=q.dtype, device=dev, shape=K_rot.shape)
    _need(out, "out", dtype=q.dtype, device=dev, shape=(B, Hq, d))
    _need(idx, "idx", dtype=torch.int32, device=dev, shape=(B, Hq, k))
    R = 0
    if K_lead is not None:
        _need(K_lead, "K_lead", dtype=q.dtype, ndim=4, device=dev)
        R = K_lead.shape[3]
        _need(K_lead, "K_lead", shape=(B, Hkv, S, R))
    _gpu(q, "q")
    _check(load_library().loki_decode_noalloc(_ptr(q), _ptr(P), _ptr(K_rot), _ptr(K_lead), R, _ptr(V), _ptr(out),
                                              _ptr(idx), B, Hq, Hkv, S, d, r, k, _dtype_code(q), _stream(q)))
    return out, idx
