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
