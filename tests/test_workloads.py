"""CPU: seeded generators (determinism, shapes, needles, FP8 round trip) and the oracle
on the tiny workload (planted needles must be picked)."""
import math

import numpy as np

import oracle
from workloads import CONFIGS, make_workload, small_config
from workloads.gen import quantize_fp8_rows


def test_deterministic_and_shapes():
    cfg = small_config("t", 101, B=2, N=700, Tq=3, H=4, d=64, n_sparse=2)
    a, b = make_workload(cfg), make_workload(cfg)
    assert a.q_full.dtype == np.uint16 and a.q_full.shape == (2, 3, 4, 64)
    assert a.k.shape == (2, 700, 64) and len(a.q_sparse) == 2
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q_sparse[1], b.q_sparse[1])
    assert a.q_pos.tolist() == [[697, 698, 699]] * 2 and a.kv_len.tolist() == [700, 700]
    # distinct tensor ids give distinct streams
    assert not np.array_equal(a.k, a.v)


def test_fp8_round_trip_bound():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((257, 128)).astype(np.float32)
    codes, scale = quantize_fp8_rows(x)
    dec = oracle.decode(codes, "fp8", scale)
    # E4M3 has 3 mantissa bits: RNE error <= 2^-4 relative for normals, and at most half of
    # the subnormal spacing 2^-9 (times the row scale) below 2^-6.
    err = np.abs(dec - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.allclose(np.abs(dec).max(axis=1), np.abs(x).max(axis=1), rtol=1e-6)


def test_tiny_needles_selected():
    cfg = CONFIGS["tiny"]
    wl = make_workload(cfg)
    assert len(wl.needles) == 8
    q = oracle.decode(wl.q_full, "f32")
    k = oracle.decode(wl.k, "f32")
    v = oracle.decode(wl.v, "f32")
    sm = 1.0 / math.sqrt(cfg.d)
    t0 = cfg.N - cfg.Tq
    for (b, t, h, p) in wl.needles:
        assert p <= t - cfg.window
        o, idx, score = oracle.full_attn_select_row(q[b, t - t0], k[b], v[b], t, sm)
        assert p in set(idx[: cfg.k_global].tolist())
        assert np.max(np.abs(o[h] - v[b, p])) < 1e-3


def test_spread64_plan():
    cfg = small_config("s", 102, B=1, N=8192 + 256, Tq=256, H=32, d=128, needles="spread64")
    wl = make_workload(cfg)
    assert len(wl.needles) == 64
    for (b, t, h, p) in wl.needles:
        assert 0 <= p <= t - cfg.window and t < cfg.N and h < cfg.H
    # c3's plan: positions 1024 i + 512, query positions 65536 + 64 i + 63, heads i mod 32
    big = CONFIGS["prefill_chunk"]
    from workloads.gen import _needle_plan
    plan = _needle_plan(big)
    assert plan[0] == (0, 65536 + 63, 0, 512) and plan[63] == (0, 65536 + 64 * 63 + 63, 31, 1024 * 63 + 512)


def test_agentic_phases_and_inputs():
    from workloads import AGENTIC, AgenticConfig, make_agentic
    cfg = AgenticConfig("t", 102, N0=50, turns=2, act=3, obs=7, H=2, d=64, D=64, n_sparse=2)
    ph = cfg.phases()
    # rounds of act single-token spans then one obs chunk, contiguous from N0 to N_final
    assert [k for (k, _, _) in ph] == ["act"] * 3 + ["obs"] + ["act"] * 3 + ["obs"]
    pos = cfg.N0
    for (kind, p, T) in ph:
        assert p == pos and T == (1 if kind == "act" else cfg.obs)
        pos += T
    assert pos == cfg.N_final == 50 + 2 * 10 and cfg.n_new == 20
    a, b = make_agentic(cfg), make_agentic(cfg)
    assert a.hidden.shape == (70, 64) and a.q_full.shape == (20, 2, 64) and len(a.q_sparse) == 2
    assert a.wk.shape == (64, 64) and np.array_equal(a.hidden, b.hidden)
    assert not np.array_equal(a.q_sparse[0], a.q_sparse[1])
    big = AGENTIC["agentic"]
    assert big.N_final == 131200 and big.n_new == 4 * (32 + 4096)
