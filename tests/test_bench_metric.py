"""The benchmark's metric code, pinned to the pages' Table 10, and its one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _rows(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_tflops_eff_reproduces_table10():
    for M, K, G, N, ms, printed in _rows("table10_tflops.txt"):
        M, K, G, N = int(M), int(K), int(G), int(N)
        pattern = [N, 3 * N // 4, N // 2, N // 4]          # repeated across the G groups
        sum_n = sum(pattern[g % 4] for g in range(G))
        got = bench.tflops_eff(M, K, sum_n, float(ms) * 1e-3)
        # latency printed to 3 decimals: +-0.0005 ms -> <= 0.08 % on the smallest latency
        assert got == pytest.approx(float(printed), rel=1e-3)


def test_weight_bytes_is_eq7():
    assert bench.weight_bytes(1536, 2048) == 1536 * 2048 * 2.75 / 8 == 1081344
    assert bench.weight_bytes(4096, 7168) == 10092544


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_fused_step_accounting():
    """The one-launch decode step's algorithmic bytes: every term once, by hand for the benchmark's
    decode configuration (E=128, K=2048, N=1536, T=16, top-8, fp32 tokens) with 81 active experts."""
    rows = 16 * 8
    by_hand = (81 * 1536 * 2048 * 11 / 32      # compressed weights of the experts with tokens
               + 16 * 2048 * 4                 # token rows, read once
               + rows * 4                      # ids
               + rows * 8 + (2 * 128 + 1) * 4  # sorted_slot + slot_pos, counts + offsets
               + rows * (1024 + 64)            # codes + block scales written
               + rows * 1536 * 2               # bf16 outputs
               + 2 * 128 * 4)                  # gamma_w, gamma_a
    assert bench.fused_step_bytes(81, 1536, 2048, 16, 8, 128) == by_hand


def test_fused_eligibility_matches_the_library_limits():
    import gen
    import dataclasses
    assert bench.fused_eligible(dataclasses.replace(gen.CONFIGS["c1"], T=2))   # 16 rows, E = 128
    assert bench.fused_eligible(dataclasses.replace(gen.CONFIGS["c1"], T=8))   # 64 rows: 2 T*k = E
    assert not bench.fused_eligible(dataclasses.replace(gen.CONFIGS["c1"], T=9))
    assert not bench.fused_eligible(gen.CONFIGS["c1"])       # 128 rows: two launches are faster
    assert not bench.fused_eligible(gen.CONFIGS["c2"])       # prefill
    assert not bench.fused_eligible(gen.CONFIGS["c3"])       # two projections, K = 7168
    assert not bench.fused_eligible(gen.CONFIGS["c3_mlp"])   # the MLP
