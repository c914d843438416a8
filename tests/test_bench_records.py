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


def test_headline_records_are_current():
    tr = bench.recorded_traffic("qwen7b_t768")
    mf = bench.recorded_mfma("qwen7b_t768")
    assert tr is not None and tr > 0
    assert mf is not None
    assert set(mf["mfma_busy"]) == {"k_rowstats", "k_colsum"}
    assert all(0.0 < v < 1.0 for v in mf["mfma_busy"].values())


def test_executed_flops_cover_two_passes():
    alg = bench.algorithmic(synth.WORKLOADS["qwen7b_t768"])
    mf = bench.recorded_mfma("qwen7b_t768")
    # each pass runs the causal QK^T once, diagonal 32x32 blocks whole
    assert 2 * alg["flops"] <= mf["executed_flops_per_launch"] <= 2.1 * alg["flops"]


@pytest.mark.parametrize("name,flops", [("qwen7b_t768", 289.6e9), ("qwen7b_t1536_ema", 2.421e12),
                                        ("llama8b_global_t16k", 549.2e9),
                                        ("llama8b_t128k", 4.396e12)])
def test_algorithmic_flops_match_closed_form(name, flops):
    # NH * 2*d*G*(W(T-W) + W(W+1)/2) for each workload's shape
    assert bench.algorithmic(synth.WORKLOADS[name])["flops"] == pytest.approx(flops, rel=2e-3)
