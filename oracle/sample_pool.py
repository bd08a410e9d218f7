"""The oracle's decode on several host cores at once, for a throughput figure.

TEST INFRASTRUCTURE ONLY: the benchmark's CPU-baseline leg starts this module
as child processes (``python -m oracle.sample_pool SPEC_JSON``), one per core,
each single-threaded.  It adds no arithmetic of its own: every worker calls the
oracle's ``select`` + ``attend`` (or ``decode_varlen`` for a ragged batch) on
whole batch elements, exactly as the single-threaded leg does.

The parent writes the inputs once as float32 ``.npy`` files (exact for bf16
and fp32 values) into a scratch folder; the workers map them read-only.  The
spec names that folder, ``r``, ``k``, the batch size, this worker's number and
the worker count, the wall-clock start time shared by every worker, and the
seconds each one keeps decoding.  Worker ``w`` takes batch elements ``w, w + n,
w + 2n, ...`` (mod ``B``) until its time is up and prints one JSON line:
``{"done": decodes, "elapsed": seconds}``.
"""

from __future__ import annotations

import json
import os
import sys
import time

import numpy as np


def _worker(spec: dict) -> dict:
    from . import loki

    folder = spec["folder"]
    arr = {n: np.load(os.path.join(folder, n + ".npy"), mmap_mode="r") for n in ("q", "P", "K_rot", "V")}
    lens_path = os.path.join(folder, "lens.npy")
    lens = np.load(lens_path) if os.path.exists(lens_path) else None
    r, k, B, w, nw = spec["r"], spec["k"], spec["B"], spec["worker"], spec["workers"]
    while time.time() < spec["start"]:  # every worker begins together, after its imports
        time.sleep(0.001)
    t0 = time.perf_counter()
    done = 0
    while True:
        b = (w + done * nw) % B
        sl = {n: arr[n][b:b + 1] for n in ("q", "K_rot", "V")}
        if lens is None:
            idx = loki.select(sl["q"], arr["P"], sl["K_rot"], r, k)
            loki.attend(sl["q"], arr["P"], sl["K_rot"], sl["V"], idx)
        else:
            loki.decode_varlen(sl["q"], arr["P"], sl["K_rot"], sl["V"], lens[b:b + 1], r, k)
        done += 1
        if time.perf_counter() - t0 >= spec["seconds"]:
            break
    return {"done": done, "elapsed": time.perf_counter() - t0}


if __name__ == "__main__":
    print(json.dumps(_worker(json.loads(sys.argv[1]))), flush=True)
