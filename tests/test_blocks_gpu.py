"""GPU parity of the block-level selection (hs2_full_attn_select_blocks) against the oracle.

Protocol per query row (the token-level protocol lifted to blocks):
  * window segment of idx: exact;
  * block ids: min(k_b, #blocks) unique ids in [0, #blocks), ascending, then -1; the symmetric
    difference with the oracle's ids only holds blocks whose oracle block score is within 1e-6 of
    the oracle's k_b-th block score;
  * the global segment of idx is exactly the expansion of the returned block ids (every member,
    cut at the candidate count), then -1;
  * planted needles: the needle's block is always picked;
  * o within the token-level bars; the sparse layers run on the oracle's indices.
block = 1 must reproduce the token-level entry point's indices bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.hs2_harness import BAND, HipRun, OracleRun, _say, to_dev, tol_for
from workloads import CONFIGS, make_workload, small_config

pytestmark = pytest.mark.gpu


def check_block_row(bidx, idx, bid_o, idx_o, sc_o, t, kb, block, W, needles=()):
    K = kb * block
    assert np.array_equal(idx[K:], idx_o[K:]), f"window segment differs at t={t}"
    C = sc_o.shape[0]
    nb = -(-C // block)
    n = min(kb, nb)
    g = bidx[:n]
    assert np.all(bidx[n:] == -1), "block padding"
    assert np.all(g >= 0) and np.all(g < nb), "block id outside the candidate blocks"
    assert np.all(np.diff(g) > 0), "block ids not strictly ascending"
    exp = [j for b in g for j in range(b * block, min(C, (b + 1) * block))]
    assert idx[:len(exp)].tolist() == exp and np.all(idx[len(exp):K] == -1), "expansion of the block ids"
    diff = np.setxor1d(g, bid_o[:n])
    if diff.size:
        bs = oracle.block_scores(sc_o, block)
        kth = np.sort(bs)[::-1][n - 1]
        off = np.abs(bs[diff] - kth)
        assert np.all(off <= BAND), f"block selection differs outside the band: {off.max():.3e}"
    for p in needles:
        assert p // block in set(g.tolist()), f"needle {p} (block {p // block}) not picked"
    return int(diff.size // 2)


def run_block_parity(cfg, kb=16, block=64, rows=None, sparse=True, wl=None):
    _say(f"[blocks] {cfg.name} B={cfg.B} N={cfg.N} Tq={cfg.Tq} {cfg.q_dtype}/{cfg.kv_dtype} kb={kb} block={block}")
    import token_level_sparse_mqa_amd as hs2
    if wl is None:
        wl = make_workload(cfg)
    g = HipRun(wl)
    if cfg.bridge_D:
        g.bridge()
    o, bidx, idx = hs2.hs2_full_attn_select_blocks(g.q, g.k, g.v, g.q_pos, g.kv_len, k_scale=g.k_scale,
                                                   v_scale=g.v_scale, k_blocks=kb, block=block,
                                                   window=cfg.window, sm_scale=g.sm)
    torch.cuda.synchronize()
    o, bidx, idx = o.cpu().numpy(), bidx.cpu().numpy(), idx.cpu().numpy()
    O = OracleRun(wl)
    if rows is None:
        rows = [(b, i) for b in range(cfg.B) for i in range(cfg.Tq)]
    t0 = cfg.N - cfg.Tq
    needles = {}
    for (b, t, h, p) in wl.needles:
        needles.setdefault((b, t - t0), []).append(p)
    tol = tol_for(cfg.kv_dtype)
    idx_or = idx.copy()
    mism, oerr = 0, 0.0
    for (b, i) in rows:
        t = int(wl.q_pos[b, i])
        o_o, bid_o, id_o, sc_o = oracle.full_attn_select_blocks_row(O.q[b, i], O.k[b], O.v[b], t, O.sm, kb, block,
                                                                    cfg.window)
        mism += check_block_row(bidx[b, i], idx[b, i], bid_o, id_o, sc_o, t, kb, block, cfg.window,
                                needles.get((b, i), []))
        err = float(np.max(np.abs(o[b, i] - o_o)))
        oerr = max(oerr, err)
        assert err <= tol, f"row {(b, i)}: o error {err:.3e}"
        idx_or[b, i] = id_o
    if sparse:
        got = hs2.hs2_sparse_attn_layers(g.qs, g.k, g.v, to_dev(idx_or, "i32"), kv_len=g.kv_len, k_scale=g.k_scale,
                                         v_scale=g.v_scale, sm_scale=g.sm)
        for l in range(cfg.n_sparse):
            gl = got[l].cpu().numpy()
            for (b, i) in rows:
                ref = O.sparse_row(l, b, i, idx_or[b, i])
                err = float(np.max(np.abs(gl[b, i] - ref)))
                assert err <= tol, f"sparse layer {l} row {(b, i)}: {err:.3e}"
    _say(f"[blocks] {cfg.name} ok: rows={len(rows)} block-mismatches={mism} o_err={oerr:.2e}")


SMALL = [
    (small_config("blk_decode", 250, B=3, N=5000, Tq=2, n_sparse=2), 16, 64),
    (small_config("blk_fp8", 251, B=2, N=6001, Tq=1, kv_dtype="fp8", n_sparse=1), 16, 64),
    (small_config("blk_chunk", 252, B=2, N=3000, Tq=37, n_sparse=1), 16, 64),
    (small_config("blk_k4_b16", 253, B=2, N=1500, Tq=3, H=16, d=64, n_sparse=1), 4, 16),
    (small_config("blk_short", 254, B=2, N=700, Tq=9, n_sparse=1), 16, 64),     # fewer blocks than k_b
    (small_config("blk_f32", 255, B=1, N=3000, Tq=4, H=8, d=64, q_dtype="f32", kv_dtype="f32", n_sparse=1), 8, 32),
]


@pytest.mark.parametrize("cfg,kb,block", SMALL, ids=[c[0].name for c in SMALL])
def test_blocks_small(cfg, kb, block):
    run_block_parity(cfg, kb, block)


def test_blocks_tiny_needles():
    """The fp32 workload with 8 planted needles: every needle's whole block is selected."""
    run_block_parity(CONFIGS["tiny"], 16, 64)


@pytest.mark.parametrize("Tq", [1, 24])
def test_block_one_is_token_level(Tq):
    """block = 1, k_blocks = k reproduces hs2_full_attn_select (same scores, same selection)."""
    import token_level_sparse_mqa_amd as hs2
    cfg = small_config(f"blk_one_{Tq}", 256 + Tq, B=2, N=4000, Tq=Tq, n_sparse=1)
    g = HipRun(make_workload(cfg))
    _, idx_tok, _ = g.full()
    o, bidx, idx = hs2.hs2_full_attn_select_blocks(g.q, g.k, g.v, g.q_pos, g.kv_len, k_blocks=1024, block=1,
                                                   window=cfg.window, sm_scale=g.sm)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_tok)
    assert torch.equal(bidx, idx_tok[..., :1024])


def test_blocks_full_decode128k():
    run_block_parity(CONFIGS["decode128k"])


def test_blocks_full_decode1m_fp8():
    """16384 candidate blocks per row: the limit of the block-level selection."""
    run_block_parity(CONFIGS["decode1m_fp8"])


def test_blocks_full_prefill_chunk_sampled():
    cfg = CONFIGS["prefill_chunk"]
    t0 = cfg.N - cfg.Tq
    from workloads.gen import _needle_plan
    plan = _needle_plan(cfg)
    rows = sorted({(0, 0), (0, cfg.Tq - 1)} | {(0, plan[i][1] - t0) for i in (0, 21, 42, 63)} |
                  {(0, int(x)) for x in np.random.default_rng(1).choice(cfg.Tq, 4, replace=False)})
    run_block_parity(cfg, rows=rows)


def test_blocks_varlen_and_scattered():
    """Block selection on sequences of different lengths with NaN past each length, and on query
    positions in any order (see the token-level tests of the same names)."""
    from tests.test_parity_gpu import varlen_workload
    cfg = small_config("blk_varlen", 256, B=3, N=4000, Tq=2, n_sparse=1)
    run_block_parity(cfg, 16, 64, wl=varlen_workload(cfg, [4000, 2600, 1300]))
    cfg = small_config("blk_varlen_chunk", 257, B=2, N=3000, Tq=16, kv_dtype="fp8", n_sparse=1)
    run_block_parity(cfg, 16, 64, wl=varlen_workload(cfg, [3000, 1900]))
    cfg = small_config("blk_scattered_chunk", 258, B=1, N=3000, Tq=24, n_sparse=1)
    wl = make_workload(cfg)
    rng = np.random.default_rng(cfg.cfg_id)
    pos = rng.integers(0, cfg.N, size=(cfg.B, cfg.Tq)).astype(np.int32)
    pos[0, 0], pos[0, 1], pos[0, 2] = 0, cfg.N - 1, 700
    wl.q_pos = pos
    run_block_parity(cfg, 16, 64, wl=wl)
