"""Host-side parts of the benchmark (CPU): the all-cores oracle baseline, the
committed-profile readers and the trace summary."""

import json
import os
import sqlite3
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from loki_inputs import CONFIGS, make_inputs  # noqa: E402


def test_oracle_all_cores_runs_whole_decodes():
    # two single-threaded worker processes on the small fp32 workload: every
    # worker decodes at least one batch element, the rate is positive and the
    # scratch folder is gone afterwards
    cfg = CONFIGS["C1"]
    x = make_inputs(cfg)
    before = set(os.listdir("/dev/shm")) if os.path.isdir("/dev/shm") else set()
    res = bench.oracle_all_cores(x, cfg, 0.3, max_workers=2)
    assert res["cores"] == min(2, len(os.sched_getaffinity(0)))
    assert res["value"] > 0
    assert "single-threaded processes" in res["sample"]
    if os.path.isdir("/dev/shm"):
        assert not any(n.startswith("loki_oracle_") for n in set(os.listdir("/dev/shm")) - before)


def test_oracle_all_cores_ragged():
    cfg = CONFIGS["C1"].replace(B=3)
    x = make_inputs(cfg)
    res = bench.oracle_all_cores(x, cfg, 0.2, lens=[cfg.S, 5, cfg.k + 1], max_workers=2)
    assert res["value"] > 0


def test_cpu_model_names_the_host():
    s = bench.cpu_model()
    assert "cores available to the process" in s and len(s) > 30


def test_trace_json_and_reader(tmp_path, monkeypatch):
    # a minimal rocprofv3-shaped kernel table: the reader takes the variant
    # launched most, and only while the decode sources match the stored hash
    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, end integer)")
    rows = [("void loki::score_select_pair_kernel<1, 8, 128, 1>(args)", 0, 88000)] * 3 + \
           [("void loki::score_select_pair_kernel<4, 2, 128, 1>(args)", 0, 174000)]
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    t = bench.trace_json(str(db))
    assert t["source_hash"] == bench.kernel_source_hash()
    k = t["kernels"]["void loki::score_select_pair_kernel<1, 8, 128, 1>"]
    assert k["calls"] == 3 and abs(k["avg_us"] - 88.0) < 1e-9
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "trace_CX.json").write_text(json.dumps(t))
    assert abs(bench.load_trace_us("CX", "score_select_pair_kernel") - 88.0) < 1e-9
    t["source_hash"] = "0" * 16
    (tmp_path / "trace_CX.json").write_text(json.dumps(t))
    assert bench.load_trace_us("CX", "score_select_pair_kernel") is None
    assert bench.load_trace_us("CY", "score_select_pair_kernel") is None


def test_committed_profiles_name_the_current_sources():
    # the committed counter and trace summaries were taken on the decode
    # sources now in the tree (else the bench line would report null)
    for name in ("traffic_C3.json", "trace_C3.json"):
        with open(os.path.join(ROOT, "profiles", name)) as fh:
            assert json.load(fh)["source_hash"] == bench.kernel_source_hash(), name


def test_union_rows_counts_distinct_rows_per_group():
    import torch
    idx = torch.tensor(np.array([[[0, 1, 2], [1, 2, 3], [5, 6, 7], [7, 8, -1]]]), dtype=torch.int32)
    assert bench.union_rows(idx, 2) == 4 + 4  # {0,1,2,3} and {5,6,7,8}
