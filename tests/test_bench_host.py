"""Host-side checks of the benchmark: its one-GPU contract and the algorithmic
byte counts its roofline figures divide by, written out by hand for the
Qwen3-8B-shaped metric workload (16 sequences x 32K tokens, 32 query / 8 KV
heads, D 128, 16-token blocks, K = 128)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from lookahead_sparse_kv_amd import workload as wlm  # noqa: E402

B, HQ, HKV, D, CTX, W, K = 16, 32, 8, 128, 32768, 2048, 128


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_exact_scoring_bytes():
    wl = wlm.WORKLOADS["qwen3_8b_32k"]
    keys = B * CTX * HKV * D * 2           # every key once: 1 GiB
    q_look = B * 1 * HQ * D * 2
    table = B * W * 4
    scores = B * HKV * W * 4
    ctx = B * 4
    assert keys == 1 << 30
    assert bench.score_bytes(wl) == keys + q_look + table + scores + ctx == 1_075_052_608


def test_attention_and_path_bytes():
    wl = wlm.WORKLOADS["qwen3_8b_32k"]
    rows = B * HKV
    kv = rows * K * 16 * D * 2 * 2         # the selected K and V tiles: 128 MiB
    q = out = B * HQ * D * 2
    lists = rows * K * 4 * 2               # block list + the page-table entries it names
    assert kv == 128 << 20
    assert bench.attn_bytes(wl) == kv + q + out + lists == 134_610_944
    select = rows * (W * 4 + K * 4)        # scores in, selection out
    assert bench.select_bytes(wl) == select
    total = bench.score_bytes(wl) + bench.select_bytes(wl) + bench.attn_bytes(wl)
    assert total == 1_210_777_664          # about 1.211 GB per layer-step


def test_compressed_scoring_bytes():
    wl = wlm.WORKLOADS["qwen3_8b_32k_minmax"]
    boxes = B * W * HKV * 2 * D * 2        # min and max rows of every block: 1/8 of the keys
    assert boxes == (1 << 30) // 8
    assert bench.score_bytes(wl) == boxes + B * HQ * D * 2 + B * HKV * W * 4 + B * 4 == 135_397_440
