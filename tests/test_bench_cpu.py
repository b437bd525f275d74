"""The benchmark's contract on the host: one GPU only (a request for more exits with a message and
status 2 before any GPU work), and the byte accounting behind the roofline's algorithmic bytes,
checked against counts written out by hand."""
import os
import subprocess
import sys

import numpy as np

from query_aware_sparse_page_amd.accounting import selected_kv_bytes, summary_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no result line


def test_selected_bytes_count_valid_tokens_only():
    P, D, Hkv = 32, 128, 2
    lens = [3 * P + 5, P]  # sequence 0: its last page holds 5 tokens
    sel = np.array([[[0, 3, -1], [1, 2, 3]], [[0, -1, -1], [0, -1, -1]]])
    cnt = np.array([[2, 3], [1, 1]])
    # head 0 of seq 0: pages 0 (32) and 3 (5); head 1: 1, 2 (32 each) and 3 (5); seq 1: one
    # full page per head
    tokens = (32 + 5) + (32 + 32 + 5) + 32 + 32
    for esize in (1, 2, 4):
        assert selected_kv_bytes(lens, sel, cnt, Hkv, P, D, esize) == 2 * tokens * D * esize
    # the 32K workload's unit: 64 full pages per KV head, 8 KV heads, bf16
    full = np.tile(np.arange(64), (1, 8, 1))
    assert selected_kv_bytes([32768], full, np.full((1, 8), 64), 8, 32, 128, 2) == 8 * 1024 * 1024


def test_summary_bytes():
    # two lo / hi rows of D elements per (page, KV head); pages = ceil(L / P)
    assert summary_bytes([32768], 8, 32, 128, 2) == 1024 * 8 * 2 * 128 * 2
    assert summary_bytes([33, 0, 1], 2, 16, 64, 4) == (3 + 0 + 1) * 2 * 2 * 64 * 4
