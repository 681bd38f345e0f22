"""Host-side checks of bench.py (CPU only): the algorithmic work per launch behind `roofline.achieved`,
written out from the definitions of the measurement plan, and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def test_decode_full_layer_bytes():
    # one pass over K and V of every sequence: B * N rows * 2 tensors * row bytes
    a = bench.algorithmic(CONFIGS["decode128k"])
    assert a["full_attn"]["bytes"] == 8 * 131072 * 2 * (128 * 2)             # 536,870,912
    a = bench.algorithmic(CONFIGS["decode1m_fp8"])
    assert a["full_attn"]["bytes"] == 1 * 1048576 * 2 * (128 + 4)           # codes + fp32 row scale


def test_sparse_layer_units():
    # per query token: S rows of K and V, S int32 indices, the bf16 query and the fp32 output
    S, H, d = 1152, 32, 128
    for name, row in (("decode128k", 2 * d), ("decode1m_fp8", d + 4)):
        cfg = CONFIGS[name]
        a = bench.algorithmic(cfg)["sparse_attn"]
        rows = cfg.B * cfg.Tq
        assert a["bytes"] == rows * (S * 2 * row + 4 * S + 2 * H * d + 4 * H * d)
        assert a["flops"] == rows * 4 * H * d * S                             # 18.87 MFLOP per token
    assert S * 2 * 2 * d == 589_824 and S * 2 * (d + 4) == 304_128


def test_prefill_full_layer_flops():
    # 4 H d flops per visible (query, key) pair; query i of the chunk sees 65536 + i + 1 keys
    cfg = CONFIGS["prefill_chunk"]
    pairs = sum(65536 + i + 1 for i in range(4096))
    assert bench.algorithmic(cfg)["full_attn"]["flops"] == 4.0 * 32 * 128 * pairs
    assert abs(4.0 * 32 * 128 * pairs / 1e12 - 4.535) < 1e-3


def test_bridge_units():
    cfg = CONFIGS["prefill_exit256k"]
    a = bench.algorithmic(cfg)["bridge"]
    D, d, T = 2048, 128, 262144
    assert a["bytes"] == T * (2 * D + 4 * d) + 4 * D * d                     # 4,608 B per token + weights
    assert a["flops"] == 2.0 * T * D * 2 * d                                  # 1.05 MFLOP per token


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
