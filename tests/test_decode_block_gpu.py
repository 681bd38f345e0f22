"""The decode hybrid block in one launch (hs2_decode_block) against the separate calls and the oracle.

The single launch runs the same device code as hs2_full_attn_select followed by
hs2_sparse_attn_layers (same plans, same splits), so its o, indices and sparse outputs must equal
theirs bit for bit; each case runs twice in a row on one workspace, the second time on other
inputs.  A small case is also checked against the oracle with the usual protocol.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.hs2_harness import HipRun, OracleRun, _say, check_indices, tol_for, to_dev
from workloads import CONFIGS, make_workload, small_config

pytestmark = pytest.mark.gpu


def _separate(g, cfg):
    import token_level_sparse_mqa_amd as hs2
    o, idx = hs2.hs2_full_attn_select(g.q, g.k, g.v, g.q_pos, g.kv_len, k_scale=g.k_scale, v_scale=g.v_scale,
                                      k_global=cfg.k_global, window=cfg.window, sm_scale=g.sm)
    ws = hs2.sparse_attn_layers_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.S, cfg.n_sparse, g.q.device)
    osp = hs2.hs2_sparse_attn_layers(g.qs, g.k, g.v, idx, kv_len=g.kv_len, k_scale=g.k_scale, v_scale=g.v_scale,
                                     sm_scale=g.sm, workspace=ws)
    return o, idx, osp


def _fused(g, cfg, ws):
    import token_level_sparse_mqa_amd as hs2
    return hs2.hs2_decode_block(g.q, g.qs, g.k, g.v, g.q_pos, g.kv_len, k_scale=g.k_scale, v_scale=g.v_scale,
                                k_global=cfg.k_global, window=cfg.window, sm_scale=g.sm, workspace=ws)


CASES = [
    small_config("db_decode", 270, B=3, N=5000, Tq=2, n_sparse=2),
    small_config("db_fp8", 271, B=2, N=6001, Tq=1, kv_dtype="fp8", n_sparse=3),
    small_config("db_d64", 272, B=4, N=3000, Tq=3, H=16, d=64, n_sparse=1),
    small_config("db_short", 273, B=2, N=700, Tq=4, n_sparse=2),          # fewer candidates than k
    small_config("db_k16", 274, B=2, N=2500, Tq=2, k_global=16, window=4, n_sparse=2),
]


@pytest.mark.parametrize("cfg", CASES + [CONFIGS["decode128k"], CONFIGS["decode1m_fp8"]], ids=lambda c: c.name)
def test_decode_block_equals_separate_calls(cfg):
    import token_level_sparse_mqa_amd as hs2
    _say(f"[decode_block] {cfg.name} B={cfg.B} N={cfg.N} Tq={cfg.Tq} {cfg.kv_dtype} L={cfg.n_sparse}")
    g1 = HipRun(make_workload(cfg))
    g2 = HipRun(make_workload(small_config(cfg.name + "_b", cfg.cfg_id + 1000, B=cfg.B, N=cfg.N, Tq=cfg.Tq,
                                           H=cfg.H, d=cfg.d, q_dtype=cfg.q_dtype, kv_dtype=cfg.kv_dtype,
                                           n_sparse=cfg.n_sparse, k_global=cfg.k_global, window=cfg.window)))
    ws = hs2.decode_block_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.N, cfg.k_global, cfg.window,
                                    hs2.dtype_code(g1.k), cfg.n_sparse, g1.q.device)
    for g in (g1, g2):
        ref = _separate(g, cfg)
        got = _fused(g, cfg, ws)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), "full-layer o differs"
        assert torch.equal(got[1], ref[1]), "indices differ"
        for l in range(cfg.n_sparse):
            assert torch.equal(got[2][l], ref[2][l]), f"sparse layer {l} differs"


def test_decode_block_oracle():
    """The single launch against the oracle directly (small decode case, every row)."""
    import token_level_sparse_mqa_amd as hs2
    cfg = CASES[0]
    wl = make_workload(cfg)
    g = HipRun(wl)
    o, idx, osp = _fused(g, cfg, None)
    torch.cuda.synchronize()
    o, idx = o.cpu().numpy(), idx.cpu().numpy()
    osp = [x.cpu().numpy() for x in osp]
    O = OracleRun(wl)
    tol = tol_for(cfg.kv_dtype)
    idx_oracle = idx.copy()
    for b in range(cfg.B):
        for i in range(cfg.Tq):
            o_o, idx_o, sc_o = O.full_row(b, i)
            check_indices(idx[b, i], idx_o, sc_o, int(wl.q_pos[b, i]), cfg.k_global, cfg.window)
            assert np.max(np.abs(o[b, i] - o_o)) <= tol
            idx_oracle[b, i] = idx_o
            # the block's sparse layers on its own indices against the oracle on the same indices
            for l in range(cfg.n_sparse):
                assert np.max(np.abs(osp[l][b, i] - O.sparse_row(l, b, i, idx[b, i]))) <= tol
    # and the sparse layers on the oracle's indices (rows whose selections differ inside the band
    # included), through the same device code as the block's sparse phase
    ws = hs2.sparse_attn_layers_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.S, cfg.n_sparse, g.q.device)
    o_ref = hs2.hs2_sparse_attn_layers(g.qs, g.k, g.v, to_dev(idx_oracle, "i32"), kv_len=g.kv_len,
                                       k_scale=g.k_scale, v_scale=g.v_scale, sm_scale=g.sm, workspace=ws)
    torch.cuda.synchronize()
    for l in range(cfg.n_sparse):
        got = o_ref[l].cpu().numpy()
        for b in range(cfg.B):
            for i in range(cfg.Tq):
                assert np.max(np.abs(got[b, i] - O.sparse_row(l, b, i, idx_oracle[b, i]))) <= tol


def test_decode_block_rejects():
    import token_level_sparse_mqa_amd as hs2
    cfg = CASES[0]
    g = HipRun(make_workload(cfg))
    with pytest.raises(hs2.HS2Error):          # query chunks take the separate calls
        q = torch.zeros((cfg.B, 8, cfg.H, cfg.d), dtype=torch.bfloat16, device="cuda")
        hs2.hs2_decode_block(q, [q], g.k, g.v, torch.zeros((cfg.B, 8), dtype=torch.int32, device="cuda"), g.kv_len)


def test_decode_block_varlen():
    """Sequences of different lengths with NaN past each length: the single launch equals the
    separate calls bit for bit, and its outputs are finite."""
    from tests.test_parity_gpu import varlen_workload
    import token_level_sparse_mqa_amd as hs2
    for cfg, lengths in ((small_config("db_varlen", 275, B=3, N=4000, Tq=2, n_sparse=2), [4000, 2600, 1300]),
                         (small_config("db_varlen_fp8", 276, B=2, N=5000, Tq=1, kv_dtype="fp8", n_sparse=2),
                          [3100, 5000])):
        _say(f"[decode_block] {cfg.name}")
        g = HipRun(varlen_workload(cfg, lengths))
        ws = hs2.decode_block_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.N, cfg.k_global, cfg.window,
                                        hs2.dtype_code(g.k), cfg.n_sparse, g.q.device)
        ref = _separate(g, cfg)
        got = _fused(g, cfg, ws)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.isfinite(got[0]).all()
        assert torch.equal(got[1], ref[1])
        for l in range(cfg.n_sparse):
            assert torch.equal(got[2][l], ref[2][l]) and torch.isfinite(got[2][l]).all()
