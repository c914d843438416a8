"""The counter records bench.py attaches to its line (profiles/*.json) match the
committed score source, and the bench's algorithmic flop counts agree with the
closed form of one causal QK^T, 2*d*G*(W(T-W) + W(W+1)/2) per head (CPU only)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from eviction_window_qk_amd import synth  # noqa: E402


HEADLINE = "llama8b_t128k"   # bench.py's default workload


def test_bench_default_is_the_largest_workload():
    wl = synth.WORKLOADS[HEADLINE]
    assert all(wl.n_heads * wl.T >= w.n_heads * w.T for w in synth.WORKLOADS.values())
    assert "--workload\", default=\"llama8b_t128k\"" in open(bench.__file__).read()


def test_headline_records_are_current():
    tr = bench.recorded_traffic(HEADLINE)
    mf = bench.recorded_mfma(HEADLINE)
    assert tr is not None and tr > 0
    assert mf is not None
    # pass 1, and pass 2 in whichever variant the workload takes (streamed or LDS-resident)
    assert len(mf["mfma_busy"]) == 2 and "k_rowstats" in mf["mfma_busy"]
    assert any(k.startswith("k_colsum") for k in mf["mfma_busy"])
    assert all(0.0 < v < 1.0 for v in mf["mfma_busy"].values())


def test_executed_flops_cover_two_passes():
    alg = bench.algorithmic(synth.WORKLOADS[HEADLINE])
    mf = bench.recorded_mfma(HEADLINE)
    # each pass runs the causal QK^T once, diagonal 32x32 blocks whole
    assert 2 * alg["flops"] <= mf["executed_flops_per_launch"] <= 2.1 * alg["flops"]


@pytest.mark.parametrize("name,flops", [("qwen7b_t768", 289.6e9), ("qwen7b_t1536_ema", 2.421e12),
                                        ("llama8b_global_t16k", 549.2e9),
                                        ("llama8b_t128k", 4.396e12)])
def test_algorithmic_flops_match_closed_form(name, flops):
    # NH * 2*d*G*(W(T-W) + W(W+1)/2) for each workload's shape
    assert bench.algorithmic(synth.WORKLOADS[name])["flops"] == pytest.approx(flops, rel=2e-3)


@pytest.mark.parametrize("name,nbytes", [("qwen7b_t768", 0.7688e9), ("llama8b_global_t16k", 4.3956e9)])
def test_score_stage_bytes(name, nbytes):
    # one read of K (NH*T*d*2) and of the window queries (NH*G*W*d*2), one write of u (NH*T*4)
    wl = synth.WORKLOADS[name]
    expect = wl.n_heads * (2.0 * wl.T * wl.head_dim + 2.0 * wl.group * wl.window * wl.head_dim + 4.0 * wl.T)
    assert expect == pytest.approx(nbytes, rel=1e-3)
    assert bench.algorithmic(wl)["b_score"] == pytest.approx(expect, rel=1e-12)


@pytest.mark.parametrize("name,bound", [("qwen7b_t768", "mfma"), ("qwen7b_t1536_ema", "mfma"),
                                        ("llama8b_t128k", "mfma"), ("llama8b_global_t16k", "hbm")])
def test_score_roofline_bound(name, bound):
    # the stage's bound is the slower of its flops at the MFMA peak and its bytes at the HBM peak
    alg = bench.algorithmic(synth.WORKLOADS[name])
    t_flop = alg["flops"] / (bench.PEAK_BF16_TFLOPS * 1e12)
    t_byte = alg["b_score"] / (bench.PEAK_HBM_GBS * 1e9)
    assert ("hbm" if t_byte > t_flop else "mfma") == bound
