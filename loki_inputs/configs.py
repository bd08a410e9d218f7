"""Workload shapes for low-rank-key (Loki-style) sparse decode attention.

Five decode workloads are defined, each with the shape of a real model's
attention layer and a synthetic key spectrum that stands in for the low-rank
structure of real keys (Loki, arXiv 2406.02542, abstract: keys lie in a much
lower-dimensional space than the head dimension).  No dataset or model weight
is used; the spectra ``exp(-j/tau)`` give the rotated key dimensions a
geometric variance decay so that the leading ``r`` rotated dimensions carry
most of the key energy.

Names (notation of the AQUA page's preliminaries, eqs. 1-5): ``B`` batch,
``Hq`` query heads, ``Hkv`` key/value heads (``G = Hq/Hkv`` queries share one
key head), ``d`` head dimension, ``S`` cached tokens, ``r`` leading rotated
dimensions used for approximate scores, ``k`` tokens kept per query head.
"""

from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg_no: int          # seed namespace; one per workload family
    B: int
    Hq: int
    Hkv: int
    d: int
    S: int
    r: int
    k: int
    dtype: str           # "f32" or "bf16": storage dtype of q, P, K, K_rot, V, out
    tau: float           # key/query spectrum: std of rotated dim j is exp(-j/tau)
    heavy: int = 0       # planted heavy tokens per query head
    noise: float = 0.0   # isotropic key noise std (added to every key dim)
    projection: bool = False  # the workload includes the prefill key projection

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    def scaled(self, S: int | None = None, B: int | None = None, k: int | None = None,
               heavy: int | None = None) -> "Config":
        """Same workload family at a smaller size (for parity cases that the
        oracle finishes in seconds).  ``k`` keeps the family's k/S ratio
        unless given."""
        S2 = self.S if S is None else S
        k2 = k if k is not None else max(1, (self.k * S2) // self.S)
        hv = self.heavy if heavy is None else heavy
        if hv:
            hv = min(hv, max(1, k2 // 2))
        return self.replace(name=f"{self.name}@S{S2}", S=S2, k=k2,
                            B=self.B if B is None else B, heavy=hv)


CONFIGS = {
    # Single head, batch 1, fp32, d_head 64.
    "C1": Config("C1", 1, B=1, Hq=1, Hkv=1, d=64, S=1024, r=16, k=64,
                 dtype="f32", tau=8.0),
    # Llama-2-7B-shaped decode (MHA), bf16 cache.
    "C2": Config("C2", 2, B=1, Hq=32, Hkv=32, d=128, S=4096, r=32, k=512,
                 dtype="bf16", tau=16.0),
    # Llama-3-8B-shaped GQA decode, 16 sequences of 16K tokens.
    "C3": Config("C3", 3, B=16, Hq=32, Hkv=8, d=128, S=16384, r=32, k=1024,
                 dtype="bf16", tau=16.0),
    # Long-context GQA decode with 64 planted heavy tokens per query head.
    "C4": Config("C4", 4, B=1, Hq=32, Hkv=8, d=128, S=131072, r=16, k=2048,
                 dtype="bf16", tau=12.0, heavy=64),
    # Prefill key projection then one decode step; noisy keys.
    "C5": Config("C5", 5, B=4, Hq=32, Hkv=8, d=128, S=32768, r=64, k=2048,
                 dtype="bf16", tau=24.0, noise=0.05, projection=True),
}


def config(name: str) -> Config:
    return CONFIGS[name]
