"""Host-side logic of the benchmark (no GPU): the one-GPU refusal, the algorithmic byte
count behind its GB/s figures, and the rule that counted traffic is reported only for the
kernel source it was measured on."""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_algorithmic_bytes_of_the_million_token_layer():
    # 32 kv heads = 32 query heads, 2-bit keys and values, k = 2, one new token per step, at
    # a cache of 1000 tokens.  Per (token, kv head): key record 128*2/8 = 32 B plus 3 B per
    # outlier; value tile share 32 B, 3 B per outlier and a 2-byte scale; per (token, query
    # head) a 4-byte logit written by q.K^T and read by softmax.V.  The append reads the two
    # fp16 vectors (2 * 256 B) and writes the key record, the value codes (32 B each), 3 B per
    # outlier of each vector and the 2-byte scale.
    wl = synth.WORKLOADS["llama7b_1m_2bit"]
    assert (wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.k_bits, wl.v_bits, wl.n_outliers, wl.n_new) == (1, 32, 32, 2, 2, 2, 1)
    qk, pv, app = bench.algorithmic_bytes(wl, 1000)
    assert qk == 32 * 1000 * (32 + 6) + 32 * 1000 * 4 == 1_344_000
    assert pv == 32 * 1000 * (32 + 6 + 2) + 32 * 1000 * 4 == 1_408_000
    assert app == 32 * (512 + 32 + 32 + 12 + 2) == 18_880


def test_algorithmic_bytes_of_the_grouped_layer():
    # batch 16, 8 kv heads shared by 32 query heads (g = 4), 3-bit keys and values, k = 2:
    # 54 B of keys and 56 B of values per (token, kv head), 4 logits of 4 B each way
    wl = synth.WORKLOADS["llama3_8b_gqa_b16_64k"]
    assert (wl.batch, wl.n_kv_heads, wl.n_q_heads, wl.k_bits, wl.v_bits, wl.n_outliers) == (16, 8, 32, 3, 3, 2)
    L = 64
    qk, pv, _ = bench.algorithmic_bytes(wl, L)
    units = 16 * 8 * L
    assert qk == units * (54 + 4 * 4)
    assert pv == units * (56 + 4 * 4)


def test_traffic_is_reported_only_for_the_measured_source():
    wl = "llama7b_1m_2bit"
    stored = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[wl]["qk_lut_kernel"]
    assert bench.traffic_from_profile(wl, "qk_lut_kernel", stored["source_hash"]) == stored["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile(wl, "qk_lut_kernel", "0" * 16) is None
    assert bench.traffic_from_profile("no_such_workload", "qk_lut_kernel", stored["source_hash"]) is None
