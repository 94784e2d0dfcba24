"""CPU checks of the benchmark's contract and of its algorithmic work counts
(no GPU: only the argument handling and the arithmetic of the counters)."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_latent_kv_04_amd.workloads import WORKLOADS, make_problem  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_refused_combinations_exit_before_touching_the_gpu():
    # the non-absorbed kernel is bf16 only; the FP8 cache serves the absorbed form
    r = _run("--attention", "non-absorbed", "--workload", "v2lite_f32_L256")
    assert r.returncode == 2 and "bf16" in r.stderr
    r = _run("--cache", "fp8", "--attention", "non-absorbed", "--workload",
             "v2_bf16_prefill_6144+2048")
    assert r.returncode == 2 and "absorbed" in r.stderr


def test_decode_work_counts_every_key_once():
    prob = make_problem(WORKLOADS["v2lite_bf16_B64_L4096"], B=3, ctx=[100, 7, 64])
    by, fl = bench.algorithmic_work(prob)
    keys = 171
    n_h = prob.wl.n_h
    assert by == keys * 576 * 2 + 3 * n_h * 576 * 2 + 3 * n_h * 513 * 4
    assert fl == keys * n_h * (2 * 576 + 2 * 512)


def test_prefill_work_counts_the_causal_pairs():
    prob = make_problem(WORKLOADS["v2_bf16_prefill_6144+2048"], ctx=10, q_len=4, n_h=2)
    # rows see 7, 8, 9, 10 keys
    pairs = 7 + 8 + 9 + 10
    _, fl = bench.algorithmic_work(prob)
    assert fl == pairs * 2 * (2 * 576 + 2 * 512)
    assert bench.non_absorbed_flops(prob) == (2 * (2 * 512 * 128) * 10 * 2 +
                                              pairs * 2 * (2 * 192 + 2 * 128))


def test_full_prefill_flop_counts():
    prob = make_problem(WORKLOADS["v2_bf16_prefill_6144+2048"])
    assert abs(bench.algorithmic_work(prob)[1] / 1e12 - 4.089) < 1e-3
    assert abs(bench.non_absorbed_flops(prob) / 1e12 - 1.4776) < 1e-4


def test_producer_work():
    kv_by, q_by, kv_fl, q_fl = bench.producer_work(128, 128, 5120, 1536, 2)
    assert kv_by == (128 * 5120 + 576 * 5120 + 128 * 576) * 2 + 512 * 4
    assert q_by == (128 * 5120 + 1536 * 5120 + 128 * 192 * 1536 + 128 * 128 * 192) * 2 + 1536 * 4
    assert kv_fl == 2 * 128 * 576 * 5120 and q_fl == 2 * 128 * (1536 * 5120 + 128 * 192 * 1536)
    # without query compression the queries come straight from h
    _, q_by2, _, q_fl2 = bench.producer_work(64, 16, 2048, None, 2)
    assert q_by2 == (64 * 2048 + 16 * 192 * 2048 + 64 * 16 * 192) * 2
    assert q_fl2 == 2 * 64 * 16 * 192 * 2048


def test_traffic_record_applies_only_to_the_sources_it_was_taken_on():
    path = os.path.join(ROOT, "profiles", "decode_traffic_v2_bf16_B128_L1k-8k.json")
    with open(path) as f:
        rec = json.load(f)
    got = bench.load_traffic("v2_bf16_B128_L1k-8k")
    if rec["source_sha"] == bench.source_sha():
        assert got == rec["hbm_bytes_per_launch"]
    else:
        assert got is None
    assert bench.load_traffic("v2lite_f32_L256") is None       # no record
    assert rec["hbm_bytes_per_launch"] >= rec["algorithmic_bytes_per_launch"] * 0.9
    # the non-absorbed prefill times another kernel: its own record, keyed on
    # that kernel's sources
    wl = "v2_bf16_prefill_6144+2048"
    with open(os.path.join(ROOT, "profiles", f"prefill_mha_traffic_{wl}.json")) as f:
        rec2 = json.load(f)
    got2 = bench.load_traffic(wl, "prefill_mha")
    if rec2["source_sha"] == bench.source_sha("prefill_mha"):
        assert got2 == rec2["hbm_bytes_per_launch"]
    else:
        assert got2 is None
    assert bench.source_sha("prefill_mha") != bench.source_sha("decode")
