"""Host-side logic of bench.py (no GPU): the one-GPU contract, the flop convention and the lookup
of recorded HBM traffic by source digest."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_flop_convention():
    # FA convention: 4 B H N^2 d, halved when causal; the benchmark shape gives 549.76 GFLOP forward
    assert bench.fwd_flops(1, 32, 8192, 128, True) == 4 * 32 * 8192 ** 2 * 128 / 2 == 549755813888
    assert bench.fwd_flops(1, 1, 128, 64, False) == 4 * 128 * 128 * 64


def test_recorded_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    digest = bench.sources_digest("dkdv")
    f = tmp_path / "traffic.md"
    f.write_text("| kernel | sources digest | fetched MB | written MB | traffic MB | alg | ratio |\n"
                 "|---|---|---|---|---|---|---|\n"
                 f"| dkdv | {digest} | 700.0 | 100.0 | 800.0 | 1 + 1 | 2.0 |\n"
                 "| dq | 0123456789abcdef | 1.0 | 1.0 | 2.0 | 1 + 1 | 1.0 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("dkdv") == 800.0e6
    assert bench.recorded_traffic("dq") is None  # recorded for other sources: not reported
    assert bench.recorded_traffic("fwd") is None


def test_cpu_baseline_reports_parity_of_given_outputs():
    """The cpu_baseline leg times the oracle and, on the heads it computes, sets the timed step's
    outputs against it: exact oracle values pass, a perturbed O fails the bar."""
    import numpy as np
    import torch
    import oracle
    from inputs import CONFIGS, make_inputs
    cfg = CONFIGS[1]
    t = make_inputs(cfg)
    x = {k: v[0, 0].to(torch.float64).numpy() for k, v in t.items()}
    fr = oracle.forward(x["q"], x["k"], x["v"], cfg.causal, cfg.scale, 1.25, 1)
    br = oracle.backward(x["q"], x["k"], x["v"], x["do"], cfg.causal, cfg.scale, o=fr.o, lse=fr.lse)
    gpu = {"o": fr.o[None, None], "lse": fr.lse[None, None], "dq": br.dq[None, None],
           "dk": br.dk[None, None], "dv": br.dv[None, None], "dup": fr.rs[None, None],
           "m": fr.m[None, None]}
    res = bench.cpu_baseline(cfg, t, 1, gpu, budget_s=0.0)
    par = res["parity_of_timed_step"]
    assert par["pass"] and par["heads_checked"] == 1 and par["dupcnt_rows_differing"] == 0
    assert par["shift_m_max_rel_err_where_counts_agree"] == 0.0
    assert res["host_cpu_count"] == os.cpu_count() and res["kind"] == "oracle"
    bad = dict(gpu, o=gpu["o"] + 0.05)
    assert not bench.cpu_baseline(cfg, t, 1, bad, budget_s=0.0)["parity_of_timed_step"]["pass"]
    bad = dict(gpu, dup=gpu["dup"] + 1)
    assert bench.cpu_baseline(cfg, t, 1, bad, budget_s=0.0)["parity_of_timed_step"]["dupcnt_rows_differing"] == 128
    bad = dict(gpu, dq=gpu["dq"] * 1.1)
    assert not bench.cpu_baseline(cfg, t, 1, bad, budget_s=0.0)["parity_of_timed_step"]["pass"]
