"""Host-side logic of bench.py (no GPU): the algorithmic work behind the roofline
line, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from synth.configs import C1

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_of_the_decode_layer():
    # every one of the 64 experts receives rows at T = 64
    w = bench.algorithmic_work(C1, np.ones(C1.N, dtype=np.int64))
    d, I, Is, T, N, R = C1.d, C1.inter, C1.I_s, C1.T, C1.N, C1.T * C1.K
    # gate/up stage: every routed expert's gate and up weights once, the shared
    # ones, x in, H out (bf16 throughout)
    assert w["gate_up"]["bytes"] == (N * 2 * d * I + 2 * d * Is + T * d + R * I + T * Is) * 2
    assert w["gate_up"]["bytes"] == 1_874_427_904
    # the whole layer: all expert and shared weights, the router weights, x and y
    assert w["layer"]["bytes"] == (N * 3 * d * I + 3 * d * Is + N * d + 2 * T * d) * 2
    assert w["layer"]["bytes"] == 2_809_528_320
    # 2*d*N (router) + 6*K*d*I (routed) + 6*d*I_s (shared) flops per token
    per_token = w["layer"]["flops"] / T
    assert per_token == 2 * d * N + 6 * C1.K * d * I + 6 * d * Is
    assert round(per_token / 1e6, 1) == 496.1
    assert w["active_experts"] == N
    # the experts (S4-S6): their weights, x in and y out
    assert w["experts"]["bytes"] == (N * 3 * d * I + 3 * d * Is + 2 * T * d) * 2
    assert w["experts"]["flops"] == 6 * R * d * I + 6 * T * d * Is


def test_idle_experts_read_no_weights():
    counts = np.zeros(C1.N, dtype=np.int64)
    counts[:10] = 1
    full = bench.algorithmic_work(C1, np.ones(C1.N, dtype=np.int64))
    part = bench.algorithmic_work(C1, counts)
    per_expert = 3 * C1.d * C1.inter * 2
    assert full["layer"]["bytes"] - part["layer"]["bytes"] == (C1.N - 10) * per_expert
    assert part["active_experts"] == 10


def test_int8_weights_count_one_byte_and_a_row_scale():
    ones = np.ones(C1.N, dtype=np.int64)
    w8 = bench.algorithmic_work(C1, ones, w8=True)
    d, I, Is, T, N, R = C1.d, C1.inter, C1.I_s, C1.T, C1.N, C1.T * C1.K
    expect = N * (2 * d * I + 2 * I * 4) + 2 * d * Is + 2 * Is * 4 + T * d * 2 + (R * I + T * Is) * 2
    assert w8["gate_up"]["bytes"] == expect
    # flops do not depend on the weight format
    assert w8["layer"]["flops"] == bench.algorithmic_work(C1, ones)["layer"]["flops"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_source_hash_is_stable():
    assert bench.ffn_source_hash("bf16") == bench.ffn_source_hash("bf16")
    assert bench.ffn_source_hash("bf16") != bench.ffn_source_hash("w8")


def test_source_hash_ignores_comments_only():
    code = "int f(int x) {  // doubles\n  return 2 * x;\n}\n"
    assert bench._code_only(code) == bench._code_only("// note\n" + code.replace("  // doubles", ""))
    assert bench._code_only(code) != bench._code_only(code.replace("2 * x", "3 * x"))
