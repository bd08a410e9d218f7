#!/usr/bin/env python3
"""One-GPU benchmark of low-rank-key (Loki-style) sparse decode attention.

Default run: the Llama-3-8B-shaped GQA decode workload (batch 16, 32 query
heads sharing 8 key/value heads, head dim 128, 16384 cached tokens per
sequence, leading r = 32 rotated dims for the approximate scores, k = 1024
kept tokens per query head, bf16 cache).  One step = one ``loki_decode``
over every (batch, query head): query rotation, approximate scores, top-k,
exact attention over the kept rows, merge.

Measurement:
* inputs are resident in HBM before timing; NBUF copies of the caches are
  rotated so every step reads a cache last touched NBUF-1 steps earlier,
  with more data touched in between than the 256 MB Infinity Cache holds;
* region A times exactly ``--steps`` plain steps (wall clock between two
  device synchronisations): value, ms_per_step;
* region B re-times the same steps through the instrumented entry point,
  whose HIP events on the library's stream give each kernel's average
  duration -> the roofline of the dominant kernel;
* the CPU baseline runs the float64 oracle, single-threaded, on a bounded
  sample of the same workload (whole batch elements) on the host, and also
  confirms the GPU output on that sample.

The line also reports the memory-system reference of this GPU, measured
live with the library's own kernels: a plain streaming read of 2 GiB (the
practical read ceiling next to the nominal peak) and a plain copy.

Also: ``--calibrate-copy`` runs the library's copy kernel over 1 GiB (for
rocprofv3 counter scaling), ``--summarize-trace DB`` and ``--summarize-pmc FETCH_DB WRITE_DB``
turn rocprofv3 result databases into the summaries kept under profiles/.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sqlite3
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
STAGES = ["qrot", "scores", "select", "attend", "merge"]


# the sources of the decode kernels whose counters profiles/traffic_*.json holds
DECODE_SOURCES = ("common.h", "select_core.h", "mfma_common.h", "attend_core.h", "mfma_kernels.hip",
                  "pair_kernels.hip", "select_attend_kernels.hip", "decode_kernels.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "rank_key_sparse_amd", "csrc", name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- profiles tooling


def summarize_trace(db: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, end from kernels").fetchall()
    agg: dict = {}
    for name, st, en in rows:
        agg.setdefault(name.split("(")[0], []).append((en - st) / 1000.0)
    tot = sum(sum(v) for v in agg.values())
    out = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{name}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                   f"{100 * sum(v) / tot:.1f}% |")
    return "\n".join(out)


def trace_json(db: str) -> dict:
    """Average duration per kernel (us) from a rocprofv3 kernel-trace database,
    keyed by the kernel's name without its argument list, with the decode
    sources' hash (the bench line uses it only while the sources match)."""
    con = sqlite3.connect(db)
    agg: dict = {}
    for name, st, en in con.execute("select name, start, end from kernels").fetchall():
        agg.setdefault(name.split("(")[0], []).append((en - st) / 1000.0)
    return {"source_hash": kernel_source_hash(),
            "kernels": {k: {"calls": len(v), "avg_us": sum(v) / len(v)} for k, v in agg.items()}}


def load_trace_us(workload: str, kernel_name: str):
    """The committed kernel trace's average duration (us) of `kernel_name`, or
    None when absent or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"trace_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash():
        return None
    hits = [v for key, v in t.get("kernels", {}).items() if key.split("<")[0].endswith(kernel_name)]
    # the timed variant: the one launched most (a bench also makes one full-rank reference call)
    return max(hits, key=lambda v: v["calls"])["avg_us"] if hits else None


def _pmc(db: str, counter: str) -> dict:
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, value from counters_collection where counter_name=?",
                       (counter,)).fetchall()
    agg: dict = {}
    for kn, gs, v in rows:
        agg.setdefault((kn.split("(")[0], gs), []).append(v)
    return {k: sum(v) / len(v) for k, v in agg.items()}


def summarize_pmc(fetch_db: str, write_db: str, copy_bytes: int = 1 << 30) -> dict:
    """Per-kernel HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB),
    each scaled by what the counter reads for the calibration copy."""
    fetch, write = _pmc(fetch_db, "FETCH_SIZE"), _pmc(write_db, "WRITE_SIZE")
    kib = copy_bytes / 1024.0

    def copy_entry(d):
        # the calibration copy: the library's copy kernel over 1 GiB (one read, one write)
        cands = [(v, k) for k, v in d.items() if "bench_copy_kernel" in k[0]]
        return max(cands)[1] if cands else None

    cf, cw = copy_entry(fetch), copy_entry(write)
    f_scale = kib / fetch[cf] if cf else None
    w_scale = kib / write[cw] if cw else None
    kernels = {}
    for (name, gs), v in fetch.items():
        if "loki" not in name or "bench_" in name:
            continue
        w = write.get((name, gs))
        kernels[f"{name}|grid={gs}"] = {
            "fetch_kib": v, "write_kib": w,
            "fetch_bytes": v * 1024.0 * f_scale if f_scale else None,
            "write_bytes": (w * 1024.0 * w_scale) if (w is not None and w_scale) else None,
        }
    return {"source_hash": kernel_source_hash(), "copy_kernel_fetch": cf and cf[0],
            "copy_kernel_write": cw and cw[0], "copy_bytes": copy_bytes,
            "fetch_scale": f_scale, "write_scale": w_scale, "kernels": kernels}


def load_traffic(workload: str, kernel_name: str):
    """Scaled HBM bytes per dispatch of `kernel_name` from the committed PMC
    summary, or None when absent or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash():
        return None
    for key, v in t.get("kernels", {}).items():
        if key.split("|")[0].split("<")[0].endswith(kernel_name) and v.get("fetch_bytes") is not None:
            return v["fetch_bytes"] + (v.get("write_bytes") or 0.0)
    return None


# ----------------------------------------------------------------------------- benchmark


def memory_reference(read_bytes: int = 2 << 30, copy_bytes: int = 1 << 30, reps: int = 5) -> dict:
    """Rates of the library's own reference kernels on this GPU: a plain
    streaming read of `read_bytes` (larger than the 256 MB Infinity Cache, so
    it streams from HBM) and a plain copy of `copy_bytes` (read + write
    counted), median of `reps` timed runs each (HIP events)."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    src = torch.empty(read_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    dst = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda")

    def timed(fn, n):
        out = []
        for _ in range(n + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(1e-3 * e0.elapsed_time(e1))
        return float(np.median(out[1:]))  # the first run warms up

    t_read = timed(lambda: rks.loki_bench_read(src, sink), reps)
    t_copy = timed(lambda: rks.loki_bench_copy(src[:copy_bytes], dst), reps)
    del src, dst
    return {"read_gbs": round(read_bytes / t_read / 1e9, 1), "copy_gbs": round(2 * copy_bytes / t_copy / 1e9, 1),
            "read_bytes": read_bytes, "copy_bytes": copy_bytes}


def union_rows(idx, G: int) -> int:
    """Number of distinct kept tokens per (b, kv) group, summed (the -1
    padding of sequences shorter than k not counted)."""
    import torch
    B, Hq, k = idx.shape
    Hkv = Hq // G
    grp = idx.view(B, Hkv, G * k).to(torch.int64)
    srt, _ = torch.sort(grp, dim=-1)
    distinct = 1 + (srt[..., 1:] != srt[..., :-1]).sum(dim=-1) - (srt[..., 0] < 0).to(torch.int64)
    return int(distinct.sum().item())


def ragged_lengths(B: int, S: int):
    """Per-sequence cache lengths of the ragged mode: spread evenly from S down
    to a little over S/2."""
    return [S - (b * S) // (2 * B) for b in range(B)]


def cpu_baseline(x, cfg, out_gpu, idx_gpu, seconds: float, lens=None):
    """The float64 oracle, one thread, on whole batch elements until `seconds`
    of CPU work; also checks the GPU result on that sample.  With `lens` each
    element is a decode over its own cache prefix."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_helpers import OUT_TOL, check_index_sets

    done, t_used, ok = 0, 0.0, True
    with threadpool_limits(limits=1):
        while t_used < seconds or done == 0:
            b = done % cfg.B
            sl = {n: x[n][b:b + 1] for n in ("q", "K_rot", "V")}
            t = time.perf_counter()
            if lens is None:
                idx_o, s_o = oracle.select(sl["q"], x["P"], sl["K_rot"], cfg.r, cfg.k, return_scores=True)
                out_o = oracle.attend(sl["q"], x["P"], sl["K_rot"], sl["V"], idx_o)
            else:
                out_o, idx_o, s_o = oracle.decode_varlen(sl["q"], x["P"], sl["K_rot"], sl["V"], lens[b:b + 1],
                                                         cfg.r, cfg.k, return_scores=True)
            t_used += time.perf_counter() - t
            if done < cfg.B:  # first pass over the batch: confirm the GPU result
                try:
                    differ = check_index_sets(idx_gpu[b:b + 1].astype(np.int64), idx_o, s_o, cfg.k)
                    err = np.abs(out_gpu[b:b + 1] - out_o)
                    for bb, h in differ:
                        err[bb, h] = 0.0
                    ok = ok and float(err.max()) <= OUT_TOL[x["q"].dtype]
                except AssertionError:
                    ok = False
            done += 1
    per_step = t_used / done * cfg.B
    single = {"value": round(1.0 / per_step, 4), "cores": 1,
              "sample": f"{done} batch-element decodes of the same workload ({done / cfg.B:.2f} full steps, "
                        f"{done * cfg.Hq} query heads), {t_used:.1f} s single-threaded"}
    many = oracle_all_cores(x, cfg, seconds, lens)
    res = {"value": many["value"], "unit": "steps/s", "cores": many["cores"], "kind": "oracle",
           "sample": many["sample"], "cpu_model": cpu_model(), "single_core": single,
           "gpu_matches_oracle_on_sample": ok}
    return res


def cpu_model() -> str:
    """The host CPU's model name and the cores this process may run on."""
    name = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name}; {len(os.sched_getaffinity(0))} cores available to the process"


def oracle_all_cores(x, cfg, seconds: float, lens=None, max_workers: int = 16) -> dict:
    """The oracle on every available host core (at most `max_workers`, one
    single-threaded process each) for `seconds` of wall-clock time, decoding
    whole batch elements of the same workload; the rate is the decodes of all
    workers over the longest worker's time."""
    import shutil
    import subprocess
    import tempfile

    import numpy as np

    nw = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    folder = tempfile.mkdtemp(prefix="loki_oracle_", dir=shm)
    procs = []
    try:
        for n in ("q", "P", "K_rot", "V"):  # float32 holds bf16 and fp32 values exactly
            np.save(os.path.join(folder, n + ".npy"), x[n].float().numpy())
        if lens is not None:
            np.save(os.path.join(folder, "lens.npy"), np.asarray(lens, dtype=np.int64))
        env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
                   PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
        start = time.time() + 3.0
        for w in range(nw):
            spec = {"folder": folder, "r": cfg.r, "k": cfg.k, "B": cfg.B, "worker": w, "workers": nw,
                    "start": start, "seconds": seconds}
            procs.append(subprocess.Popen([sys.executable, "-m", "oracle.sample_pool", json.dumps(spec)],
                                          cwd=ROOT, env=env, stdout=subprocess.PIPE, text=True))
        outs = []
        for p_ in procs:
            so, _ = p_.communicate(timeout=seconds + 120)
            if p_.returncode != 0:
                raise RuntimeError(f"oracle worker exited with status {p_.returncode}")
            outs.append(json.loads(so.strip().splitlines()[-1]))
    finally:
        for p_ in procs:
            if p_.poll() is None:
                p_.kill()
                p_.wait()
        shutil.rmtree(folder, ignore_errors=True)
    done = sum(o["done"] for o in outs)
    wall = max(o["elapsed"] for o in outs)
    return {"value": round(done / wall / cfg.B, 4), "cores": nw,
            "sample": f"{done} batch-element decodes of the same workload ({done / cfg.B:.2f} full steps) "
                      f"by {nw} single-threaded processes in {wall:.1f} s wall-clock"}


def score_stage_kernel(cfg) -> str:
    """The kernel that runs the score stage of a bf16 decode (the library's
    dispatch rule): scores and selection fused, one block per query head, when
    every query head has its own key head; fused per pair of query heads of a
    group when the group size is even; for heads longer than 32768 tokens
    selected in two stages, the scores fused with the first stage, one block
    per query head and 16384-token chunk, when that gives 256 blocks;
    otherwise the score kernel alone (the selection then runs as its own
    stage)."""
    G = cfg.Hq // cfg.Hkv
    if cfg.dtype == "bf16" and cfg.S <= 16384:
        if cfg.Hq == cfg.Hkv and cfg.B * cfg.Hq >= 256:
            return "score_select_kernel"
        if G % 2 == 0 and cfg.B * cfg.Hq >= 512 and cfg.r <= 128:
            return "score_select_pair_kernel"
    C = -(-cfg.S // 16384)
    if (cfg.dtype == "bf16" and cfg.S > 32768 and cfg.k < cfg.S and cfg.k <= 16384 and C * cfg.k <= 32768
            and cfg.B * cfg.Hq * C >= 256 and cfg.r <= 128):
        return "score_select_chunk_kernel"
    return "score_mfma_kernel"


def run(args) -> dict:
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = time.perf_counter()
    x = make_inputs(cfg)
    gen_s = time.perf_counter() - t
    print(f"[bench] inputs for {cfg.name} generated in {gen_s:.1f} s", file=sys.stderr, flush=True)
    q = x["q"].to(dev)
    P = x["P"].to(dev)
    R = cfg.r if args.layout == "lead" else 0
    bufs = []
    for i in range(args.buffers):
        Kr = x["K_rot"].to(dev)
        V = x["V"].to(dev)
        Kl = Kr[..., :R].contiguous() if R else None
        bufs.append((Kr, V, Kl))
    nbytes = rks.loki_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.d, cfg.r, cfg.k, q.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    idx = torch.empty((cfg.B, cfg.Hq, cfg.k), dtype=torch.int32, device=dev)
    lens_h = ragged_lengths(cfg.B, cfg.S) if args.ragged else None
    lens = None if lens_h is None else torch.tensor(lens_h, dtype=torch.int32, device=dev)

    def step(i, events=None):
        Kr, V, Kl = bufs[i % len(bufs)]
        rks.loki_decode(q, P, Kr, V, cfg.r, cfg.k, out=out, idx=idx, workspace=ws, K_lead=Kl, events=events,
                        lens=lens)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    headline = step
    if args.graph:
        # one HIP graph per cache copy (its kernels in one launch), replayed in turn
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        for i in range(len(bufs)):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(gr, stream=side):
                    step(i)
            graphs.append(gr)
        torch.cuda.current_stream().wait_stream(side)
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        headline = lambda i: graphs[i % len(graphs)].replay()  # noqa: E731

    # region A: the headline
    t0 = time.perf_counter()
    for i in range(args.steps):
        headline(i)
    t_enq = time.perf_counter() - t0  # host time to enqueue the steps (diagnostic)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    print(f"[bench] region A: {args.steps} steps in {wall * 1e3:.2f} ms", file=sys.stderr, flush=True)

    # region A': the same plain steps with one event between consecutive
    # steps (no events inside a step): per-step percentiles of the headline
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e_ in ev_a:
        e_.record()
    torch.cuda.synchronize()
    ev_a[0].record()
    for i in range(args.steps):
        headline(i)
        ev_a[i + 1].record()
    torch.cuda.synchronize()
    plain_us = np.sort([1e3 * ev_a[i].elapsed_time(ev_a[i + 1]) for i in range(args.steps)])
    pct_plain = {"p10": float(np.percentile(plain_us, 10)), "p50": float(np.percentile(plain_us, 50)),
                 "p90": float(np.percentile(plain_us, 90))}

    # region B: per-kernel durations from stage events on the library's stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in evs:  # create the underlying events
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=evs[i])
    torch.cuda.synchronize()
    stage_us = {s: 0.0 for s in STAGES}
    for row in evs:
        for j, s in enumerate(STAGES):
            stage_us[s] += 1e3 * row[j].elapsed_time(row[j + 1])
    stage_us = {s: v / args.steps for s, v in stage_us.items()}
    # whole-step durations from the same events (first to last): percentiles
    step_us = np.sort([1e3 * row[0].elapsed_time(row[5]) for row in evs])
    pct = {"p10": float(np.percentile(step_us, 10)), "p50": float(np.percentile(step_us, 50)),
           "p90": float(np.percentile(step_us, 90))}

    # quality context (not timed): how many of the exact top-k tokens the
    # kept set holds, the exact top-k from the library's full-rank decode
    Kr0, V0, _ = bufs[0]
    step(0)
    idx_kept = idx.clone()
    _, idx_exact = rks.loki_decode(q, P, Kr0, V0, cfg.d, cfg.k, lens=lens)
    torch.cuda.synchronize()
    a_k, a_x = idx_kept.cpu().numpy(), idx_exact.cpu().numpy()
    recall = float(np.mean([np.intersect1d(a_k[b, h][a_k[b, h] >= 0], a_x[b, h][a_x[b, h] >= 0]).size
                            / max(1, int((a_x[b, h] >= 0).sum())) for b in range(cfg.B) for h in range(cfg.Hq)]))

    # algorithmic bytes (what the method must move; intermediates excluded)
    e = cfg.elem_bytes
    U = union_rows(idx, cfg.G)
    tokens = cfg.B * cfg.S if lens_h is None else sum(lens_h)
    by_prefix = tokens * cfg.Hkv * cfg.r * e
    by_gather = U * cfg.d * 2 * e
    by_step = by_prefix + by_gather + cfg.Hkv * cfg.d * cfg.d * e + 2 * cfg.B * cfg.Hq * cfg.d * e \
        + cfg.B * cfg.Hq * cfg.k * 4
    whole = score_stage_kernel(cfg) == "score_select_pair_kernel"
    # the pair kernel runs the whole step (its later stage events are empty):
    # its bytes per launch are the step's
    per_kernel_bytes = {"scores": by_step if whole else by_prefix, "attend": by_gather}
    dom = max(("scores", "attend"), key=lambda s: stage_us[s])
    dom_kernel = {"scores": score_stage_kernel(cfg), "attend": "attend_mfma_kernel"}[dom]
    achieved = per_kernel_bytes[dom] / (stage_us[dom] * 1e-6) / 1e9
    traffic = load_traffic(args.workload, dom_kernel)
    trace_us = None if args.ragged else load_trace_us(args.workload, dom_kernel)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic, 0),
                "kernel": dom_kernel, "alg_bytes_per_launch": per_kernel_bytes[dom],
                "avg_launch_us": round(stage_us[dom], 2),
                # the same kernel's average duration in the committed rocprofv3
                # trace (no events around it), and the fraction it gives
                "trace_avg_us": None if trace_us is None else round(trace_us, 2),
                "frac_trace": None if trace_us is None else
                round(per_kernel_bytes[dom] / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    step_gbs = by_step / (ms_per_step * 1e-3) / 1e9
    mem = memory_reference()

    res = {
        "metric": "decode attention steps/s (all heads) and achieved HBM GB/s vs ~8 TB/s peak",
        "value": round(1e3 / ms_per_step, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Llama-3-8B-shaped GQA decode" if cfg.name == "C3" else cfg.name,
                   "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.d,
                   "cached_tokens": cfg.S, "r": cfg.r, "k": cfg.k, "score_source":
                   f"K_lead (R={R})" if R else "K_rot rows", "cache_copies_rotated": args.buffers,
                   "launch": "HIP graph per step" if args.graph else "one call per step",
                   "lengths": "full" if lens_h is None else
                   f"ragged {lens_h[0]}..{lens_h[-1]} (mean {sum(lens_h) / len(lens_h):.0f})"},
        "hbm_gbs_step": round(step_gbs, 1),
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "frac_of_read_ceiling_step": round(step_gbs / mem["read_gbs"], 4),
        "memory_reference": mem,
        "step_us_plain": {k_: round(v_, 2) for k_, v_ in pct_plain.items()},
        "host_enqueue_us_per_step": round(1e6 * t_enq / args.steps, 2),
        "step_us_events": {k_: round(v_, 2) for k_, v_ in pct.items()},
        "recall_at_k_vs_exact_topk": round(recall, 4),
        "alg_bytes_per_step": by_step,
        "union_rows": U,
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        res["cpu_baseline"] = cpu_baseline(x, cfg, out.float().cpu().numpy().astype(np.float64),
                                           idx.cpu().numpy(), args.cpu_seconds,
                                           None if lens_h is None else np.array(lens_h))
    else:
        res["cpu_baseline"] = None
    return res


def run_project(args) -> dict:
    """The key projection K_rot = K P (and the leading-dims copy K_lead) on the
    prefill-plus-decode workload's cache: HBM GB/s, MFMA TFLOP/s."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(cfg, need_K=True)
    P = x["P"].to(dev)
    R = cfg.r if args.layout == "lead" else 0
    bufs = []
    for i in range(max(2, args.buffers)):
        K = x["K"].to(dev)
        Kr = torch.empty_like(K)
        Kl = torch.empty(K.shape[:-1] + (R,), dtype=K.dtype, device=dev) if R else None
        bufs.append((K, Kr, Kl))

    def step(i):
        K, Kr, Kl = bufs[i % len(bufs)]
        rks.loki_project_keys(K, P, K_rot=Kr, R=R if R else None, K_lead=Kl)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    # the same calls between events on the current stream: the kernel's average duration
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / args.steps
    e = cfg.elem_bytes
    rows = cfg.B * cfg.Hkv * cfg.S
    by = 2 * rows * cfg.d * e + cfg.Hkv * cfg.d * cfg.d * e + rows * R * e
    flop = 2.0 * rows * cfg.d * cfg.d
    gbs = by / (us * 1e-6) / 1e9
    tflops = flop / (us * 1e-6) / 1e12
    # oracle on one (b, kv) slice, single-threaded, scaled to the whole cache
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t < min(args.cpu_seconds, 5.0):
            oracle.project(x["K"][n % cfg.B:n % cfg.B + 1, :1], x["P"][:1])
            n += 1
        per_slice = (time.perf_counter() - t) / n
    # the reference copy of the same bytes (K in, K_rot out) with the library's own copy kernel
    K0, Kr0, _ = bufs[0]
    nb = K0.numel() * K0.element_size()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for i in range(args.steps):
        rks.loki_bench_copy(bufs[i % len(bufs)][0], bufs[i % len(bufs)][1])
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nb / (1e-3 * c0.elapsed_time(c1) / args.steps) / 1e9
    step(0)
    torch.cuda.synchronize()
    got = bufs[0][1][:1, :1].double().cpu().numpy()
    want = oracle.project(x["K"][:1, :1], x["P"][:1])
    ok = bool(np.max(np.abs(got - want)) <= 2e-2)
    return {
        "metric": "key projection K_rot = K P (+ leading-dims copy): achieved HBM GB/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} cache projection", "batch": cfg.B, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.d, "cached_tokens": cfg.S, "lead_dims": R, "buffers": len(bufs)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "project_bf16_kernel",
                     "alg_bytes_per_launch": by, "avg_launch_us": round(us, 2)},
        "mfma": {"tflops": round(tflops, 2), "peak_tflops": 2500.0, "util": round(tflops / 2500.0, 4),
                 "flop_per_launch": flop},
        "copy_reference": {"gbs": round(copy_gbs, 1), "bytes_moved": 2 * nb,
                           "frac_of_copy": round(gbs / copy_gbs, 4)},
        "cpu_baseline": {"value": round(1.0 / (per_slice * cfg.B * cfg.Hkv), 4), "unit": "projections/s",
                         "cores": 1, "kind": "oracle",
                         "sample": f"{n} (b, kv) slices of {cfg.S}x{cfg.d} in float64, scaled to the cache",
                         "gpu_matches_oracle_on_slice": ok},
    }


def run_aqua(args) -> dict:
    """Decode steps whose approximate scores use each query head's r rotated
    dims of largest |q_rot| (loki_decode_aqua) on the decode workload."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(cfg)
    q, P = x["q"].to(dev), x["P"].to(dev)
    bufs = [(x["K_rot"].to(dev), x["V"].to(dev)) for _ in range(args.buffers)]
    ws = torch.empty(rks.loki_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.d, cfg.r, cfg.k, q.dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    idx = torch.empty((cfg.B, cfg.Hq, cfg.k), dtype=torch.int32, device=dev)
    dims = torch.empty((cfg.B, cfg.Hq, cfg.r), dtype=torch.int32, device=dev)
    info = torch.empty((cfg.B, cfg.Hq), dtype=torch.float32, device=dev)

    def step(i, events=None):
        Kr, V = bufs[i % len(bufs)]
        rks.loki_decode_aqua(q, P, Kr, V, cfg.r, cfg.k, out=out, idx=idx, workspace=ws, dims=dims, info_loss=info,
                             events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in evs:
        for ev in row:
            ev.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=evs[i])
    torch.cuda.synchronize()
    stage_us = {s: 0.0 for s in STAGES}
    for row in evs:
        for j, s_ in enumerate(STAGES):
            stage_us[s_] += 1e3 * row[j].elapsed_time(row[j + 1]) / args.steps
    # quality context (untimed): recall of the exact top-k (the library's
    # full-rank decode) by these dims and by the leading r dims of the basis
    Kr0, V0 = bufs[0]
    step(0)
    idx_aq = idx.clone()
    _, idx_exact = rks.loki_decode(q, P, Kr0, V0, cfg.d, cfg.k)
    _, idx_lead = rks.loki_decode(q, P, Kr0, V0, cfg.r, cfg.k)
    torch.cuda.synchronize()
    ex = idx_exact.cpu().numpy()

    def recall(ii):
        a = ii.cpu().numpy()
        return float(np.mean([np.intersect1d(a[b, h], ex[b, h]).size / cfg.k
                              for b in range(cfg.B) for h in range(cfg.Hq)]))
    e = cfg.elem_bytes
    # the dims the method reads: per (b, kv) group the union of its heads' dims
    dg = dims.view(cfg.B, cfg.Hkv, cfg.G * cfg.r).cpu().numpy()
    union_dims = int(sum(len(np.unique(dg[b, kv])) for b in range(cfg.B) for kv in range(cfg.Hkv)))
    by_scores = union_dims * cfg.S * e
    by_rows = cfg.B * cfg.Hkv * cfg.S * cfg.d * e  # what the kernel streams: whole rotated rows
    U = union_rows(idx, cfg.G)
    by_gather = U * cfg.d * 2 * e
    by_step = by_scores + by_gather + cfg.Hkv * cfg.d * cfg.d * e + 2 * cfg.B * cfg.Hq * cfg.d * e \
        + cfg.B * cfg.Hq * cfg.k * 4
    per = {"scores": by_scores, "attend": by_gather}
    dom = max(("scores", "attend"), key=lambda s_: stage_us[s_])
    kern = {"scores": "score_mfma_kernel" if cfg.dtype == "bf16" else "score_kernel",
            "attend": "attend_mfma_kernel"}[dom]
    ach = per[dom] / (stage_us[dom] * 1e-6) / 1e9
    res = {
        "metric": "decode steps/s with query-magnitude score dims (all heads)",
        "value": round(1e3 / ms, 1), "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode, query-magnitude dims", "batch": cfg.B, "q_heads": cfg.Hq,
                   "kv_heads": cfg.Hkv, "head_dim": cfg.d, "cached_tokens": cfg.S, "r": cfg.r, "k": cfg.k},
        "stage_us": {s_: round(v, 2) for s_, v in stage_us.items()},
        "union_dims_per_group": round(union_dims / (cfg.B * cfg.Hkv), 2),
        "score_rows_streamed_bytes": by_rows,
        "info_loss_mean": round(float(info.mean()), 5),
        "recall_at_k_vs_exact_topk": {"query_magnitude_dims": round(recall(idx_aq), 4),
                                      "leading_dims": round(recall(idx_lead), 4)},
        "hbm_gbs_step": round(by_step / (ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kern,
                     "alg_bytes_per_launch": per[dom], "avg_launch_us": round(stage_us[dom], 2)},
    }
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
        return res
    # oracle on whole batch elements (bounded), single-threaded; also the
    # leading-dims information loss of the same queries for comparison
    import oracle
    from oracle import aqua
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_helpers import check_index_sets
    ig = idx.cpu().numpy().astype(np.int64)
    done, used, ok = 0, 0.0, True
    with threadpool_limits(limits=1):
        while used < args.cpu_seconds or done == 0:
            b = done % cfg.B
            sl = {n: x[n][b:b + 1] for n in ("q", "K_rot", "V")}
            t = time.perf_counter()
            idx_o, s_o = aqua.select(sl["q"], x["P"], sl["K_rot"], cfg.r, cfg.k, return_scores=True)
            oracle.attend(sl["q"], x["P"], sl["K_rot"], sl["V"], idx_o)
            used += time.perf_counter() - t
            if done < cfg.B:
                dims_o = aqua.query_dims(sl["q"], x["P"], cfg.r)
                same = np.all(dims_o == dg.reshape(cfg.B, cfg.Hq, cfg.r)[b:b + 1], axis=-1)[0]
                for h in np.nonzero(same)[0]:
                    try:
                        check_index_sets(ig[b:b + 1, h:h + 1], idx_o[:, h:h + 1], s_o[:, h:h + 1], cfg.k)
                    except AssertionError:
                        ok = False
            done += 1
    lead = np.broadcast_to(np.arange(cfg.r), (cfg.B, cfg.Hq, cfg.r))
    res["info_loss_leading_dims_mean"] = round(float(aqua.info_loss(x["q"], x["P"], lead).mean()), 5)
    res["cpu_baseline"] = {"value": round(1.0 / (used / done * cfg.B), 4), "unit": "steps/s", "cores": 1,
                           "kind": "oracle", "sample": f"{done} batch-element decodes, {used:.1f} s single-threaded",
                           "gpu_matches_oracle_on_sample": ok}
    return res


def run_asym(args) -> dict:
    """Decode steps with an asymmetric scoring index (loki_decode_asym) on the
    decode workload: the factors calibrated on the GPU from seeded query
    samples and the keys, the key index written by the projection kernel
    (both timed once, outside the steps), then the timed decode steps."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs, make_query_samples

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(cfg, need_K=True)
    if args.queries == "mismatched":
        # queries (and the calibration samples) drawn in another basis than
        # the keys: the query and key second moments differ
        both = make_query_samples(cfg, 512 + cfg.B, seed=1)
        qs, x["q"] = both[:512].to(dev), both[512:].contiguous()
    else:
        qs = make_query_samples(cfg, 512).to(dev)
    q = x["q"].to(dev)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    bufs = []
    for i in range(args.buffers):
        K, V = x["K"].to(dev), x["V"].to(dev)
        if i == 0:
            e0.record()
            A, Bm = rks.loki_calibrate_asym(qs, K, cfg.r)
            e1.record()
        Ki = rks.loki_project_keys(K, Bm, R=cfg.r, lead_only=True)
        if i == 0:
            e2.record()
        bufs.append((K, V, Ki))
    torch.cuda.synchronize()
    calib_ms, index_ms = e0.elapsed_time(e1), e1.elapsed_time(e2)
    ws = torch.empty(rks.loki_decode_workspace_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.d, cfg.r, cfg.k, q.dtype),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    idx = torch.empty((cfg.B, cfg.Hq, cfg.k), dtype=torch.int32, device=dev)

    def step(i, events=None):
        K, V, Ki = bufs[i % len(bufs)]
        rks.loki_decode_asym(q, A, Ki, K, V, cfg.r, cfg.k, out=out, idx=idx, workspace=ws, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for row in evs:
        for ev in row:
            ev.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(i, events=evs[i])
    torch.cuda.synchronize()
    stage_us = {s_: 0.0 for s_ in STAGES}
    for row in evs:
        for j, s_ in enumerate(STAGES):
            stage_us[s_] += 1e3 * row[j].elapsed_time(row[j + 1]) / args.steps
    # quality context (untimed): recall of the exact top-k (the library's
    # full-rank decode with an identity basis) by this index and by Loki's
    # leading dims of the keys' own principal basis, both at rank r
    K0, V0, _ = bufs[0]
    step(0)
    idx_asym = idx.clone()
    eye = torch.eye(cfg.d, dtype=q.dtype, device=dev).expand(cfg.Hkv, cfg.d, cfg.d).contiguous()
    _, idx_exact = rks.loki_decode(q, eye, K0, V0, cfg.d, cfg.k)
    P_pca, _ = rks.loki_calibrate_pca(K0)
    K_rot_pca = rks.loki_project_keys(K0, P_pca)
    _, idx_pca = rks.loki_decode(q, P_pca, K_rot_pca, V0, cfg.r, cfg.k)
    torch.cuda.synchronize()
    ex = idx_exact.cpu().numpy()

    def recall(ii):
        a = ii.cpu().numpy()
        return float(np.mean([np.intersect1d(a[b, h], ex[b, h]).size / cfg.k
                              for b in range(cfg.B) for h in range(cfg.Hq)]))
    e = cfg.elem_bytes
    U = union_rows(idx, cfg.G)
    by_scores = cfg.B * cfg.Hkv * cfg.S * cfg.r * e
    by_gather = U * cfg.d * 2 * e
    by_step = by_scores + by_gather + cfg.Hkv * cfg.d * cfg.d * e + 2 * cfg.B * cfg.Hq * cfg.d * e \
        + cfg.B * cfg.Hq * cfg.k * 4
    # the pair kernel runs the whole step (its later stage events are empty):
    # its bytes per launch are the step's
    whole = score_stage_kernel(cfg) == "score_select_pair_kernel"
    per = {"scores": by_step if whole else by_scores, "attend": by_gather}
    dom = max(("scores", "attend"), key=lambda s_: stage_us[s_])
    kern = {"scores": score_stage_kernel(cfg), "attend": "attend_mfma_kernel"}[dom]
    ach = per[dom] / (stage_us[dom] * 1e-6) / 1e9
    res = {
        "metric": "decode steps/s with an asymmetric scoring index (all heads)",
        "value": round(1e3 / ms, 1), "unit": "steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} decode, asymmetric index", "batch": cfg.B, "q_heads": cfg.Hq,
                   "kv_heads": cfg.Hkv, "head_dim": cfg.d, "cached_tokens": cfg.S, "r": cfg.r, "k": cfg.k,
                   "calibration_queries_per_head": 512, "queries": args.queries},
        "recall_at_k_vs_exact_topk": {"asymmetric_index": round(recall(idx_asym), 4),
                                      "key_pca_leading_dims": round(recall(idx_pca), 4)},
        "stage_us": {s_: round(v, 2) for s_, v in stage_us.items()},
        "calibration_ms": round(calib_ms, 3), "index_projection_ms": round(index_ms, 3),
        "hbm_gbs_step": round(by_step / (ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kern,
                     "alg_bytes_per_launch": per[dom], "avg_launch_us": round(stage_us[dom], 2)},
    }
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
        return res
    # the oracle's own pipeline (its factors from the same query samples and
    # keys, then per batch element the index, selection and attention),
    # single-threaded on whole batch elements for a bounded time; the factors
    # are set up outside the timed part, as on the GPU
    import oracle
    from oracle import asym
    from threadpoolctl import threadpool_limits
    A_o, B_o = asym.calibrate(qs.cpu(), x["K"], cfg.r)
    eye = np.broadcast_to(np.eye(cfg.d), (cfg.Hkv, cfg.d, cfg.d))
    done, used = 0, 0.0
    with threadpool_limits(limits=1):
        while used < args.cpu_seconds or done == 0:
            b = done % cfg.B
            t = time.perf_counter()
            Ki = np.einsum("hsd,hdr->hsr", x["K"][b].double().numpy(), B_o)[None]
            ii = asym.select(x["q"][b:b + 1], A_o, Ki, cfg.r, cfg.k)
            oracle.attend(x["q"][b:b + 1], eye, x["K"][b:b + 1], x["V"][b:b + 1], ii)
            used += time.perf_counter() - t
            done += 1
    res["cpu_baseline"] = {"value": round(1.0 / (used / done * cfg.B), 4), "unit": "steps/s", "cores": 1,
                           "kind": "oracle", "sample": f"{done} batch-element decodes (index, selection, attention), "
                                                       f"{used:.1f} s single-threaded"}
    return res


def run_calibrate(args) -> dict:
    """Offline calibration of the basis (loki_calibrate_pca) on the workload's
    whole key cache: Gram matrix of each key head's rows (MFMA), fixed-order
    sum of the partials, Jacobi eigensolver.  The Gram kernel streams the
    cache (HBM roofline); the eigensolver is one block per key head."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(cfg, need_K=True)
    K = x["K"].to(dev)
    P = torch.empty((cfg.Hkv, cfg.d, cfg.d), dtype=K.dtype, device=dev)
    lam = torch.empty((cfg.Hkv, cfg.d), dtype=torch.float64, device=dev)
    ws = torch.empty(rks.loki_calibrate_workspace_bytes(cfg.B, cfg.Hkv, cfg.S, cfg.d), dtype=torch.uint8,
                     device=dev)

    def step(events=None):
        rks.loki_calibrate_pca(K, P, lam, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    names = ("gram", "reduce", "eigensolver")
    stage_us = {n: 0.0 for n in names}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in evs:
        for ev in row:
            ev.record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    for row in evs:
        for j, n in enumerate(names):
            stage_us[n] += 1e3 * row[j].elapsed_time(row[j + 1]) / args.steps
    e = cfg.elem_bytes
    rows = cfg.B * cfg.Hkv * cfg.S
    by = rows * cfg.d * e  # the keys, read once
    flop = 2.0 * rows * cfg.d * cfg.d
    gbs = by / (stage_us["gram"] * 1e-6) / 1e9
    tflops = flop / (stage_us["gram"] * 1e-6) / 1e12
    # oracle (float64 SVD) on one key head, single-threaded, scaled to all heads;
    # its result also checks the GPU's leading directions and eigenvalues there
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        P_o, lam_o = oracle.calibrate(x["K"][:, :1])
        per_head = time.perf_counter() - t
    Pg = P.double().cpu().numpy()[0]
    cos = np.abs(np.sum(Pg[:, :cfg.r] * P_o[0][:, :cfg.r], axis=0))
    ok = bool(np.min(cos) > 0.999 and np.max(np.abs(lam.cpu().numpy()[0] - lam_o[0])) <= 1e-4 * lam_o[0, 0])
    return {
        "metric": "basis calibration (principal directions of the key cache, per key head): calls/s",
        "value": round(1e3 / ms, 3), "unit": "calls/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} key-cache calibration", "batch": cfg.B, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.d, "cached_tokens": cfg.S},
        "stage_us": {n: round(v, 2) for n, v in stage_us.items()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "gram_bf16_kernel",
                     "alg_bytes_per_launch": by, "avg_launch_us": round(stage_us["gram"], 2),
                     "note": "the eigensolver (one block per key head, latency-bound) takes most of the call"},
        "mfma": {"tflops": round(tflops, 2), "peak_tflops": 2500.0, "util": round(tflops / 2500.0, 4),
                 "flop_per_launch": flop},
        "cpu_baseline": {"value": round(1.0 / (per_head * cfg.Hkv), 5), "unit": "calls/s", "cores": 1,
                         "kind": "oracle",
                         "sample": f"one key head ({cfg.B * cfg.S}x{cfg.d} float64 SVD, {per_head:.1f} s), "
                                   f"scaled to {cfg.Hkv} heads",
                         "gpu_matches_oracle_on_sample": ok},
    }


def run_append(args) -> dict:
    """One decode step's cache append (loki_append_kv): the new key of every
    (b, kv) rotated into the basis and written with its value and lead dims
    at the sequence's position, on the workload's caches."""
    import numpy as np
    import torch

    import rank_key_sparse_amd as rks
    from loki_inputs import CONFIGS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    rks.load_library()
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(cfg)
    P = x["P"].to(dev)
    Kr, V = x["K_rot"].to(dev), x["V"].to(dev)
    R = cfg.r if args.layout == "lead" else 0
    Kl = Kr[..., :R].contiguous() if R else None
    g = torch.Generator().manual_seed(9)
    tdt = Kr.dtype
    k_new = torch.randn((cfg.B, cfg.Hkv, cfg.d), generator=g).to(tdt).to(dev)
    v_new = torch.randn((cfg.B, cfg.Hkv, cfg.d), generator=g).to(tdt).to(dev)
    # each sequence appends at its own position (a ragged batch)
    pos = torch.tensor([cfg.S - 1 - (b % 7) for b in range(cfg.B)], dtype=torch.int32, device=dev)

    def step(i):
        rks.loki_append_kv(k_new, v_new, P, pos, Kr, V, Kl)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # host-inclusive: one Python call per append (the launch, not the kernel, sets the pace)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    # device throughput: `steps` appends captured in one HIP graph, one replay timed by events
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for i in range(args.steps):
                step(i)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / args.steps
    e = cfg.elem_bytes
    rows = cfg.B * cfg.Hkv
    # read k_new, v_new, P, pos; write the K_rot, V and K_lead rows
    by = 2 * rows * cfg.d * e + cfg.Hkv * cfg.d * cfg.d * e + cfg.B * 4 + rows * (2 * cfg.d + R) * e
    gbs = by / (us * 1e-6) / 1e9
    # oracle: the same rotations in float64, single-threaded
    import oracle
    from threadpoolctl import threadpool_limits
    kn, vn = k_new.cpu(), v_new.cpu()
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t < min(args.cpu_seconds, 3.0):
            oracle.project(kn[:, :, None, :], x["P"])
            n += 1
        per_call = (time.perf_counter() - t) / n
    want = oracle.project(kn[:, :, None, :], x["P"])[:, :, 0, :]
    got = torch.stack([Kr[b, :, int(pos[b])] for b in range(cfg.B)]).double().cpu().numpy()
    ok = bool(np.max(np.abs(got - want)) <= 2e-2) and bool(
        torch.equal(torch.stack([V[b, :, int(pos[b])] for b in range(cfg.B)]).cpu(), vn))
    return {
        "metric": "cache append per decode step (rotated key, value, lead dims): appends/ms on the device",
        "value": round(1e3 / us, 1), "unit": "appends/ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us * 1e-3, 5), "host_call_ms": round(ms, 5),
        "timing": "one HIP graph of `steps` appends, replay timed by events", "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name} cache append", "batch": cfg.B, "kv_heads": cfg.Hkv,
                   "head_dim": cfg.d, "cached_tokens": cfg.S, "lead_dims": R},
        "roofline": {"bound": "latency", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "append_kv_kernel",
                     "alg_bytes_per_launch": by, "avg_launch_us": round(us, 2)},
        "cpu_baseline": {"value": round(1e-3 / per_call, 4), "unit": "appends/ms", "cores": 1, "kind": "oracle",
                         "sample": f"{n} calls of the float64 projection of the {rows} new keys",
                         "gpu_matches_oracle": ok},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="C3", choices=["C2", "C3", "C4", "C5"])
    ap.add_argument("--layout", default="lead", choices=["lead", "rowmajor"])
    ap.add_argument("--buffers", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--queries", default="matched", choices=["matched", "mismatched"],
                    help="--op asym: queries drawn in the keys' basis, or in another one")
    ap.add_argument("--ragged", action="store_true",
                    help="decode a ragged batch: per-sequence cache lengths from S down to about S/2")
    ap.add_argument("--graph", action="store_true",
                    help="decode: time steps replayed from HIP graphs (one launch per step)")
    ap.add_argument("--op", default="decode", choices=["decode", "project", "append", "calibrate", "aqua", "asym"],
                    help="project: time the key projection instead (use --workload C5); "
                         "append: time one decode step's cache append")
    ap.add_argument("--summarize-trace", metavar="DB")
    ap.add_argument("--trace-json", metavar="DB", help="per-kernel average durations of a trace as JSON")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return 0
    if args.trace_json:
        print(json.dumps(trace_json(args.trace_json), indent=1))
        return 0
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode shards over (batch, kv head) groups with no exchange between GPUs)",
              file=sys.stderr)
        return 2
    if args.calibrate_copy:
        import torch

        import rank_key_sparse_amd as rks
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            rks.loki_bench_copy(src, dst)  # the library's copy kernel: 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
    res = {"project": run_project, "append": run_append, "calibrate": run_calibrate, "aqua": run_aqua, "asym": run_asym}.get(args.op, run)(args)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
