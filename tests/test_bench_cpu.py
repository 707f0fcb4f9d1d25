"""Host-side checks of bench.py: the one-GPU contract, the byte accounting behind
the reported rate, and the guard that reports counter traffic only for the
sources it was taken on.  No GPU and no library calls."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_expert_bytes_follow_the_checkpoint_layout():
    # gate_up [5760, 90, 16] blocks + [5760, 90] scales + 5760 bf16 biases;
    # down [2880, 90, 16] + [2880, 90] + 2880 bf16
    gu, dn = bench.expert_bytes(2880, 2880)
    assert gu == 5760 * 90 * 16 + 5760 * 90 + 5760 * 2 == 8_824_320
    assert dn == 2880 * 90 * 16 + 2880 * 90 + 2880 * 2 == 4_412_160
    assert gu + dn == 13_236_480
    assert 128 * (gu + dn) == 1_694_269_440


def test_layer_accounting_counts_touched_experts_once():
    T, H, I, k = 3, 2880, 2880, 4
    ids = np.array([[0, 1, 2, 3], [3, 2, 1, 0], [0, 5, 7, 1]])
    acc = bench.moe_accounting(ids, T, H, I, 0)
    assert acc["touched"] == 6 and acc["pairs"] == T * k
    # weights of the touched experts, x in, fp32 logits, bf16 out
    assert acc["layer_bytes"] == 6 * 13_236_480 + T * H * 2 + T * 128 * 4 + T * H * 2
    # 2 flops per multiply-add: gate_up (2I x H) and down (H x I) per pair
    assert acc["flops"] == 2.0 * T * k * (2 * I * H + H * I)
    assert acc["flops"] / (T * k) == 49_766_400


def test_counter_traffic_is_reported_only_for_matching_sources(tmp_path, monkeypatch):
    srcs = ["gemm_bf16.hip", "common.hpp", "launch.hpp"]
    good = {"k": {"sources": srcs, "source_digest": bench.source_digest(srcs), "hbm_bytes_per_launch": 123}}
    stale = {"k": {"sources": srcs, "source_digest": "0000000000000000", "hbm_bytes_per_launch": 123}}
    p = tmp_path / "pmc.json"
    monkeypatch.setattr(bench, "PMC_FILE", str(p))
    p.write_text(json.dumps(good))
    assert bench.pmc_traffic("k") == 123
    assert bench.pmc_traffic("other") is None
    p.write_text(json.dumps(stale))
    assert bench.pmc_traffic("k") is None


def test_gate_up_h_bytes_follow_the_activation_mode():
    # h written by the gate_up kernel: bf16 hi + lo or fp32 = 4 B per element;
    # MXFP4 activations: E2M1 codes (1/2 B) and one E8M0 byte per 32 elements
    T, H, I = 2, 2880, 2880
    ids = np.array([[0, 1, 2, 3], [4, 5, 6, 7]])
    gu, _ = bench.expert_bytes(H, I)
    for act, xin, hb in ((0, T * H * 2, 8 * I * 4), (1, T * H, 8 * I * 4),
                         (2, T * H * 17 // 32, 8 * I * 17 // 32)):
        acc = bench.moe_accounting(ids, T, H, I, act)
        assert acc["gemm1_bytes"] == 8 * gu + xin + hb
    assert bench.h_bytes_written(8, I, 2) == 8 * 2880 // 32 * 17 == 12240
    # the logits term takes the layer's expert count
    a128 = bench.moe_accounting(ids, T, H, I, 0)
    a64 = bench.moe_accounting(ids, T, H, I, 0, E=64)
    assert a128["layer_bytes"] - a64["layer_bytes"] == T * 64 * 4


def test_tflops_fractions():
    # FP8 mode: 2/3 of the flops on the bf16 MFMA (2.5 PF), 1/3 at the FP8 rate (5 PF)
    assert abs(bench.issued_peak_tflops(1) - 3000.0) < 1e-9
    assert bench.issued_peak_tflops(2) == bench.MXFP4_PEAK_TFLOPS
    f = bench.tflops_fractions(1500.0, 2e12, 1e9, 2, ceiling_gbps=6000.0)
    assert f["flop_per_byte"] == 2000.0
    assert f["attainable_TFLOPs"] == min(10100.0, 2000.0 * 8000.0 / 1e3)
    assert abs(f["frac_attainable"] - 1500.0 / 10100.0) < 1e-12
    assert f["attainable_measured_TFLOPs"] == min(10100.0, 2000.0 * 6.0)
    assert abs(f["frac_mxfp4_peak"] - 1500.0 / 10100.0) < 1e-12


def test_dense_prefill_peaks_follow_the_issued_form():
    # E4M3 x E2M1 at the FP8 rate, E2M1 x E2M1 at the FP4 rate
    assert bench.dense_prefill_peak_tflops(1) == bench.FP8_PEAK_TFLOPS == 5000.0
    assert bench.dense_prefill_peak_tflops(2) == bench.MXFP4_PEAK_TFLOPS == 10100.0
