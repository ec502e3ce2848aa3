"""CPU checks of the benchmark's arithmetic against figures the pages print.

The FLOP formula of "Xe2 ... Flash Attention -- HD=256" (section "Performance Testing")
must reproduce the roofline percentages printed in the "Xe2 Sdp Bf16" page's performance
table from its times, and the headline figure of the HD=256 page must be consistent with
its stated peak (tests/golden/page_perf_figures.json, each entry with its citation).
"""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "page_perf_figures.json")


@pytest.fixture(scope="module")
def figures():
    with open(GOLDEN) as f:
        return json.load(f)


def test_pages_formula_reproduces_printed_roofline(figures):
    peak = figures["peak_tflops"]
    for row in figures["rows"]:
        fl = bench.flops_pages(row["q_len"], row["kv_len"], row["hd"], row["heads_q"])
        pct = 100 * fl / (row["ms"] * 1e-3) / 1e12 / peak
        assert abs(pct - row["roofline_pct"]) <= 0.1, (row["cite"], pct)


def test_headline_consistent_with_peak(figures):
    h = figures["headline"]
    assert round(h["pct"] / 100 * figures["peak_tflops"]) == h["tflops"]


def test_headline_formula_and_softmax_term():
    B, Hq, Lq, Lk, D = 1, 32, 16384, 16384, 256
    fl = bench.flops_headline(B, Hq, Lq, Lk, D)
    assert fl == 8796093022208  # 4 * 32 * 16384^2 * 256
    # the pages' count adds 2 flops per score for the softmax
    assert bench.flops_pages(Lq, Lk, D, Hq, B) - fl == 2 * B * Hq * Lq * Lk


def test_peak_is_mi355x_dense_fp16():
    # 256 CUs x 2.4 GHz x 4096 dense fp16 flop per clock per CU
    assert abs(bench.PEAK_TFLOPS - 2516.58) < 0.01


def test_visible_pairs_brute_force():
    # row i sees key j iff j <= i + Lk - Lq: counted pair by pair on small shapes
    for Lq, Lk in [(5, 8), (8, 5), (7, 7), (1, 9), (9, 1), (3, 3)]:
        brute = sum(1 for i in range(Lq) for j in range(Lk) if j <= i + Lk - Lq)
        assert bench.visible_pairs(Lq, Lk, True) == brute, (Lq, Lk)
        assert bench.visible_pairs(Lq, Lk, False) == Lq * Lk
    n = 16384
    assert bench.visible_pairs(n, n, True) == n * (n + 1) // 2


def test_algorithmic_bytes_and_bound():
    import attn_inputs
    w = attn_inputs.WORKLOADS["gqa16k_d256"]
    # Q + K + V + O (16-bit) + LSE (fp32): the 572,522,496 bytes of the headline shape
    assert bench.algorithmic_bytes(w) == 572522496
    balance = bench.PEAK_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert 314 < balance < 315
    ai = {n: bench.flops_workload(x) / bench.algorithmic_bytes(x)
          for n, x in attn_inputs.WORKLOADS.items()}
    assert ai["gqa16k_d256"] > 15000 and ai["gqa8k_d128_bf16"] > balance
    assert ai["decode16x16k_d256"] < balance and ai["decode1x64k_d128_bf16"] < 5


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_vs_baseline_uses_the_pages_figure(figures):
    # the pages' own TFLOPS for the headline workload (another GPU's: context only)
    assert bench.PAGES_TFLOPS == {"gqa16k_d256": figures["headline"]["tflops"]}
