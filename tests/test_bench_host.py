"""Host logic of bench.py (no GPU): the per-stage source hashes that tie a
committed byte-counter summary to the kernels it was taken on, and the
algorithmic work the roofline fractions divide by."""
import importlib.util
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    bench = _bench()
    prof = tmp_path / "profiles"
    prof.mkdir()
    good, stale = bench.source_hash("logits"), "0" * 16
    (prof / "traffic_cfgx.txt").write_text(
        "# header\n"
        f"kernel_source_sha logits {good}\n"
        f"kernel_source_sha topk {stale}\n"
        "traffic_bytes_per_launch logits 123456\n"
        "traffic_bytes_per_launch topk 789\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # source_hash reads the kernel sources under ROOT: point it back at the repository's
    real = _bench()
    monkeypatch.setattr(bench, "source_hash", real.source_hash)
    assert bench.measured_traffic("cfgx", "logits") == 123456.0
    assert bench.measured_traffic("cfgx", "topk") is None      # taken on other sources
    assert bench.measured_traffic("cfgx", "gather") is None    # not measured
    assert bench.measured_traffic("nosuch", "logits") is None  # no summary


def test_stage_hashes_follow_their_sources():
    bench = _bench()
    h = {s: bench.source_hash(s) for s in ("logits", "topk", "gather")}
    assert len(set(h.values())) == 3 and all(len(v) == 16 for v in h.values())
    assert bench.source_hash() not in h.values()  # all of csrc/ differs from any one stage


def test_algorithmic_work_counts_valid_pairs():
    import workloads
    bench = _bench()
    x = workloads.inputs("tiny")
    cfg = x["cfg"]
    w = bench.algorithmic_work(x)
    n_valid = np.clip(x["limit"].astype(np.int64) + 1, 0, cfg.K)
    assert w["pairs"] == int(n_valid.sum())
    assert w["logits_flops"] == w["pairs"] * 2 * 64 * 128
    assert w["topk_bytes"] == w["pairs"] * 4 + cfg.rows * cfg.topk * 4
    assert w["gather_bytes"] == cfg.rows * cfg.topk * (256 + 4) + w["distinct_rows"] * 68
