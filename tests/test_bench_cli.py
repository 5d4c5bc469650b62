"""The benchmark's host-side contract: one GPU only, and the algorithmic byte count of
a layer (K/V rows read once per KV group, Q in and O out, S out)."""
import os
import subprocess
import sys

import numpy as np

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_layer_bytes_by_hand():
    w = wl.get_workload("tiny")     # 4 query heads, 4 KV heads, d = 64, N = 1024, k = 307
    d, n, k = w.head_dim, w.seq_lens[0], w.k_per_seq[0]
    attn, total = bench.layer_bytes(w, 0, None, d)          # layer 0: every head streams
    assert attn == 4 * 2 * n * d * 2 + 2 * 4 * d * 2
    assert total == attn + 4 * k * 4
    # layer 1: head 0 streams, heads 1..3 read their own sets (one KV head each)
    S = {(0, h): np.arange(h, h + 10) for h in range(4)}
    attn1, _ = bench.layer_bytes(w, 1, S, d)
    assert attn1 == 2 * n * d * 2 + 3 * 10 * 2 * d * 2 + 2 * 4 * d * 2
    # E4M3 codes: one byte per K/V element
    attn8, _ = bench.layer_bytes(w, 1, S, d, kv_elem=1)
    assert attn8 == (2 * n * d + 3 * 10 * 2 * d) + 2 * 4 * d * 2
