"""CPU: the float64 oracle against its pins, and proof that the pins catch planted mistakes."""
import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import hs2_oracle
from tests import oracle_pins as P

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)


def test_page_constants():
    g = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))
    assert oracle.K_GLOBAL == g["k_global"]["value"] == 1024
    assert oracle.WINDOW == g["window"]["value"] == 128
    # the pages' KV-cache figures: 12.09 GB -> 2.69 GB is the quoted 4.5x
    assert round(g["kv_cache_gb_hybrid_swa"]["value"] / g["kv_cache_gb_hysparse2"]["value"], 1) == \
        g["kv_cache_ratio"]["value"]
    from workloads import CONFIGS
    for cfg in CONFIGS.values():
        assert cfg.k_global == 1024 and cfg.window == 128 and cfg.S == 1152


def _mutant(old: str, new: str):
    src = open(hs2_oracle.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    # (description, old text, new text)
    ("dropped softmax scale", "s = sm * (q @ kk.T)", "s = (q @ kk.T)"),
    ("sign flip in logits", "s = sm * (q @ kk.T)", "s = -sm * (q @ kk.T)"),
    ("key range excludes t", "kk = k[: t + 1]", "kk = k[: t]"),
    ("score normalised over candidates only", "return p[:, :C].sum(axis=0)",
     "return (p[:, :C] / p[:, :C].sum(axis=1, keepdims=True)).sum(axis=0) if C else p[:, :C].sum(axis=0)"),
    ("candidate range off by one", "C = max(0, t - window + 1)", "C = max(0, t - window + 2)"),
    ("ties to the higher index", 'order = np.argsort(-score, kind="stable")',
     'order = (score.shape[0] - 1 - np.argsort(-score[::-1], kind="stable"))'),
    ("window off by one", "win = np.arange(max(0, t - window + 1), t + 1)",
     "win = np.arange(max(0, t - window), t)"),
    ("sparse keeps -1 entries", "sel = np.asarray(idx)[np.asarray(idx) >= 0]", "sel = np.asarray(idx)"),
    ("e4m3 bias 8", "(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    ("bridge uses Wv for K", "k[r0:r0 + row_block] = f64_to_bf16_bits_rne(h @ wk)",
     "k[r0:r0 + row_block] = f64_to_bf16_bits_rne(h @ wv)"),
    ("bridge truncates instead of RNE", "np.round(ax / spacing)", "np.floor(ax / spacing)"),
    ("bf16 decode drops the low byte", "u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
     "u = (np.asarray(u16, dtype=np.uint16).astype(np.uint32) & np.uint32(0xFF00)) << np.uint32(16)"),
    ("block score is the sum of its members", "min(C, (b + 1) * block)].max() for b in range(nb)",
     "min(C, (b + 1) * block)].sum() for b in range(nb)"),
    ("short last block runs past the candidates", "np.arange(b * block, min(C, (b + 1) * block))",
     "np.arange(b * block, (b + 1) * block)"),
    ("blocks shifted by one position", "score[b * block: min(C, (b + 1) * block)]",
     "score[b * block + 1: min(C, (b + 1) * block + 1)]"),
    ("e4m3 encoder ties to odd", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    ("fp8 scale from 240", "sc = (amax / np.float32(FP8_MAX)).astype(np.float32)",
     "sc = (amax / np.float32(240.0)).astype(np.float32)"),
    ("fp8 bridge projects V with Wk", "for w_b in (wk_b, wv_b):", "for w_b in (wk_b, wk_b):"),
    ("fp8 bridge rounds x to bf16 first", "x = (h @ w.T).astype(np.float32)",
     "x = f64_to_bf16_bits_rne(h @ w.T); x = bf16_bits_to_f64(x).astype(np.float32)"),
    ("sparse softmax without max shift cancels nothing but wrong normaliser",
     "p = e / e.sum(axis=1, keepdims=True)\n    return p @ v[sel]",
     "p = e / e.sum()\n    return p @ v[sel]"),
]


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new):
    mod = _mutant(old, new)
    failed = []
    for check in P.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught: {desc}"
