"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the same bytes.

Small cases span several key tiles, ragged tails and the method's degenerate cases; the five
workloads run at full size with every row (decode) or sampled rows (prefill chunks) checked.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from tests.hs2_harness import (HipRun, OracleRun, _say, bits_from_dev, check_bridge, check_indices,
                               to_dev, tol_for)
from workloads import CONFIGS, make_workload, small_config

pytestmark = pytest.mark.gpu




def run_parity(cfg, rows=None, check_scores=True, sparse_layers=None, score_tol=1e-7, wl=None):
    """The full layer, the selection and the sparse layers of one workload against the oracle on
    the given rows (default: every row).  The sparse layers are checked both ways (reading R12):
    the HIP path on the oracle's indices, and the HIP path on its own indices against the oracle
    on those same indices.  `wl` replaces the workload generated from cfg."""
    _say(f"[parity] {cfg.name} B={cfg.B} N={cfg.N} Tq={cfg.Tq} H={cfg.H} d={cfg.d} "
         f"{cfg.q_dtype}/{cfg.kv_dtype} k={cfg.k_global} W={cfg.window}")
    if wl is None:
        wl = make_workload(cfg)
    g = HipRun(wl)
    if cfg.bridge_D:
        g.bridge()
    o, idx, dbg = g.full(scores_dbg=check_scores)
    torch.cuda.synchronize()
    if rows is None:
        rows = [(b, i) for b in range(cfg.B) for i in range(cfg.Tq)]
    o_h, idx_h = o.cpu().numpy(), idx.cpu().numpy()
    dbg_rows = None
    if dbg is not None:       # only the checked rows come to the host (full chunks hold GBs of scores)
        sel = torch.tensor([b * cfg.Tq + i for (b, i) in rows], dtype=torch.int64, device=dbg.device)
        dbg_rows = dbg.view(cfg.B * cfg.Tq, cfg.N).index_select(0, sel).cpu().numpy()
        del dbg
    O = OracleRun(wl)
    if cfg.bridge_D:
        # the bridge stage first, against the oracle's float64 projection; the oracle's attention
        # then reads the validated HIP cache (reading R13)
        kb, vb = bits_from_dev(g.k[0]), bits_from_dev(g.v[0])
        check_bridge(wl.hidden, wl.wk, wl.wv, kb, vb, O.k_bits, O.v_bits)
        O.use_bridged_cache(kb, vb)
    t0 = cfg.N - cfg.Tq
    needles = {}
    for (b, t, h, p) in wl.needles:
        needles.setdefault((b, t - t0), []).append(p)
    tol = tol_for(cfg.kv_dtype)
    idx_oracle = idx_h.copy()         # rows not sampled keep the HIP path's own indices
    stats = {"mismatch": 0, "o_err": 0.0, "score_err": 0.0}
    for ri, (b, i) in enumerate(rows):
        o_o, idx_o, sc_o = O.full_row(b, i)
        t = int(wl.q_pos[b, i])
        st = check_indices(idx_h[b, i], idx_o, sc_o, t, cfg.k_global, cfg.window, needles.get((b, i), []))
        stats["mismatch"] += st["mismatch"]
        err = float(np.max(np.abs(o_h[b, i] - o_o)))
        stats["o_err"] = max(stats["o_err"], err)
        assert err <= tol, f"row {(b, i)}: full-layer o error {err:.3e} > {tol}"
        if dbg_rows is not None:
            C = sc_o.shape[0]
            if C:
                # fp32 logits carry a relative error: bound |d score| by score_tol + 1e-5 * score
                dsc = np.abs(dbg_rows[ri, :C] - sc_o)
                serr = float(np.max(dsc))
                stats["score_err"] = max(stats["score_err"], serr)
                assert np.all(dsc <= score_tol + 1e-5 * sc_o), f"row {(b, i)}: score error {serr:.3e}"
            assert np.all(dbg_rows[ri, C:] == -1.0)
        idx_oracle[b, i] = idx_o
    idx_dev = to_dev(idx_oracle, "i32")
    nl = cfg.n_sparse if sparse_layers is None else sparse_layers
    for layer in range(nl):
        for ws in (True, False):
            o_sp = g.sparse(layer, idx_dev, workspace=ws).cpu().numpy()
            for (b, i) in rows:
                ref = O.sparse_row(layer, b, i, idx_oracle[b, i])
                err = float(np.max(np.abs(o_sp[b, i] - ref)))
                assert err <= tol, f"sparse layer {layer} row {(b, i)} ws={ws}: error {err:.3e} > {tol}"
        # the other direction: the HIP path on its own indices, the oracle on the same indices
        o_own = g.sparse(layer, idx, workspace=True).cpu().numpy()
        for (b, i) in rows:
            ref = O.sparse_row(layer, b, i, idx_h[b, i])
            err = float(np.max(np.abs(o_own[b, i] - ref)))
            assert err <= tol, f"sparse layer {layer} row {(b, i)} on its own indices: error {err:.3e} > {tol}"
    _say(f"[parity] {cfg.name} ok: rows={len(rows)} band-mismatches={stats['mismatch']} "
         f"o_err={stats['o_err']:.2e} score_err={stats['score_err']:.2e}")
    return g, wl, idx, O


SMALL = [
    small_config("decode_ragged", 201, B=3, N=5000, Tq=2, n_sparse=2),
    small_config("fp8_ragged", 202, B=2, N=6001, Tq=1, kv_dtype="fp8", n_sparse=2),
    small_config("chunk_needles", 203, B=1, N=8192 + 128, Tq=128, n_sparse=1, needles="spread64"),
    small_config("h16_d64", 204, B=2, N=3000, Tq=3, H=16, d=64, n_sparse=1),
    small_config("h8_d128", 205, B=1, N=2500, Tq=5, H=8, d=128, n_sparse=1),
    small_config("f32_h16_d64", 206, B=1, N=4096, Tq=16, H=16, d=64, q_dtype="f32", kv_dtype="f32",
                 n_sparse=2, needles="seeded8"),
    small_config("f32_d128", 207, B=2, N=1500, Tq=2, H=32, d=128, q_dtype="f32", kv_dtype="f32", n_sparse=1),
    # every query before the window end: no candidates, window clamped at 0
    small_config("short_context", 208, B=1, N=100, Tq=100, n_sparse=1),
    # around C = k: positions 1148..1155 give C = 1021..1028
    small_config("k_boundary", 209, B=1, N=1156, Tq=8, n_sparse=1),
    # fewer candidates than k everywhere
    small_config("few_candidates", 210, B=2, N=700, Tq=4, n_sparse=1),
    # identical keys: every score ties; the k-th bucket overflows the LDS list -> exact fallback
    small_config("all_ties", 211, B=1, N=6000, Tq=2, n_sparse=1, ident_keys=True),
    small_config("all_ties_small", 212, B=1, N=2000, Tq=2, n_sparse=1, ident_keys=True),
    # small k and window
    small_config("k16_w4", 213, B=2, N=777, Tq=3, n_sparse=1, k_global=16, window=4),
    # query-chunk kernels: ragged workgroups, d=64, FP8, several sequences
    small_config("chunk_h16_d64", 215, B=2, N=2900, Tq=40, H=16, d=64, n_sparse=1),
    small_config("chunk_fp8", 216, B=1, N=3001, Tq=24, kv_dtype="fp8", n_sparse=1),
    small_config("chunk_ragged", 217, B=2, N=2000, Tq=13, n_sparse=1),
    small_config("chunk_k16_w4", 218, B=1, N=500, Tq=16, n_sparse=1, k_global=16, window=4),
    # 128 query rows (FP8 and d=64): the sparse layer plans two key splits per row and merges them
    small_config("rows128_fp8", 219, B=2, N=2000, Tq=64, kv_dtype="fp8", n_sparse=1),
    small_config("rows128_d64", 220, B=2, N=1500, Tq=64, H=16, d=64, n_sparse=1),
    # decode rows of many sequences (64 rows or more): the row kernels with key splits, each
    # row's top digit found once by its own launch before the gather and finish
    small_config("rows72_many_seqs", 221, B=24, N=2500, Tq=3, n_sparse=1),
    small_config("rows66_fp8", 222, B=66, N=1800, Tq=1, kv_dtype="fp8", n_sparse=1),
    # near-equal keys: distinct scores that all share the k-th's top radix digit, so the bucket
    # overflows the candidate list and the finish takes its streaming passes with the picks
    # spread over the whole row (decode rows and a query chunk)
    small_config("near_ties_rows", 223, B=2, N=9000, Tq=1, n_sparse=1, near_ties=0.02),
    small_config("near_ties_chunk", 224, B=1, N=7000, Tq=16, n_sparse=1, near_ties=0.02),
    # FP8 caches at d = 64 with 16 heads (the FP8 row, chunk, score and sparse kernels' d = 64 forms)
    small_config("fp8_h16_d64", 225, B=2, N=4000, Tq=2, H=16, d=64, kv_dtype="fp8", n_sparse=1),
    small_config("chunk_fp8_h16_d64", 226, B=1, N=3000, Tq=20, H=16, d=64, kv_dtype="fp8", n_sparse=1),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small(cfg):
    run_parity(cfg)


def test_deterministic_indices():
    cfg = SMALL[0]
    wl = make_workload(cfg)
    g = HipRun(wl)
    _, idx1, _ = g.full()
    _, idx2, _ = g.full()
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)


def test_sparse_workspace_reuse():
    """One sparse workspace reused by consecutive calls of different sizes gives the same bytes
    as a fresh workspace per call."""
    import token_level_sparse_mqa_amd as hs2
    big = small_config("ws_reuse_big", 230, B=4, N=3000, Tq=2, n_sparse=1)
    small = small_config("ws_reuse_small", 231, B=1, N=2000, Tq=1, n_sparse=1)
    runs = []
    for cfg in (big, small):
        g = HipRun(make_workload(cfg))
        _, idx, _ = g.full()
        runs.append((cfg, g, idx))
    cfg0, g0, _ = runs[0]
    shared = hs2.sparse_attn_workspace(cfg0.B, cfg0.Tq, cfg0.H, cfg0.d, cfg0.S, "cuda")
    for rep in range(2):
        for cfg, g, idx in runs:
            ref = g.sparse(0, idx, workspace=True)
            got = hs2.hs2_sparse_attn(g.qs[0], g.k, g.v, idx, kv_len=g.kv_len, sm_scale=g.sm, workspace=shared)
            torch.cuda.synchronize()
            assert torch.equal(ref, got), f"{cfg.name} pass {rep}: reused workspace changed the result"


@pytest.mark.parametrize("kv,B,Tq", [("bf16", 4, 2), ("fp8", 4, 2), ("bf16", 1, 16)])
def test_sparse_layers_match_per_layer(kv, B, Tq):
    """hs2_sparse_attn_layers gives every layer the same bytes as hs2_sparse_attn on that layer
    (same split plan and kernels, all layers in one launch), with and without a workspace."""
    import token_level_sparse_mqa_amd as hs2
    cfg = small_config(f"layers_{kv}_{B}x{Tq}", 232 + (kv == "fp8") + 2 * (Tq > 8), B=B, N=3000, Tq=Tq,
                       n_sparse=3, kv_dtype=kv)
    _say(f"[layers] {cfg.name}")
    g = HipRun(make_workload(cfg))
    _, idx, _ = g.full()
    for ws_on in (True, False):
        refs = [g.sparse(layer, idx, workspace=ws_on) for layer in range(3)]
        ws = hs2.sparse_attn_layers_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.S, 3, "cuda") if ws_on else None
        got = hs2.hs2_sparse_attn_layers(g.qs, g.k, g.v, idx, kv_len=g.kv_len, k_scale=g.k_scale,
                                         v_scale=g.v_scale, sm_scale=g.sm, workspace=ws)
        torch.cuda.synchronize()
        for layer in range(3):
            assert torch.equal(refs[layer], got[layer]), f"layer {layer} workspace={ws_on}"


def test_empty_batch_is_noop():
    import token_level_sparse_mqa_amd as hs2
    q = torch.empty((0, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((0, 1), dtype=torch.int32, device="cuda")
    kl = torch.empty((0,), dtype=torch.int32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    o, idx = hs2.hs2_full_attn_select(q, k, k, qp, kl, workspace=ws)
    assert o.shape == (0, 1, 32, 128) and idx.shape == (0, 1, 1152)


def test_invalid_positions_give_empty_rows():
    """A query position outside [0, kv_len) yields o = 0 and an all -1 index row (no fault)."""
    cfg = small_config("badpos", 214, B=2, N=1500, Tq=2, n_sparse=1)
    wl = make_workload(cfg)
    wl.q_pos[0, 0] = 1500       # == kv_len
    wl.q_pos[1, 1] = -5
    g = HipRun(wl)
    o, idx, _ = g.full()
    torch.cuda.synchronize()
    o, idx = o.cpu().numpy(), idx.cpu().numpy()
    assert np.all(idx[0, 0] == -1) and np.all(idx[1, 1] == -1)
    assert np.all(o[0, 0] == 0) and np.all(o[1, 1] == 0)
    assert np.all(idx[0, 1, 1024:] >= 0)


def test_bridge_small_exact():
    """Integer-valued operands: every fp32 partial sum is exact, so the bridge is bit-exact."""
    import token_level_sparse_mqa_amd as hs2
    import oracle
    rng = np.random.default_rng(5)
    T, D, d = 300, 256, 128
    h = rng.integers(-3, 4, size=(T, D)).astype(np.float32)
    wk = rng.integers(-3, 4, size=(D, d)).astype(np.float32)
    wv = rng.integers(-3, 4, size=(D, d)).astype(np.float32)
    from workloads.gen import f32_to_bf16_bits
    hb, wkb, wvb = f32_to_bf16_bits(h), f32_to_bf16_bits(wk), f32_to_bf16_bits(wv)
    k, v = hs2.hs2_kv_bridge(to_dev(hb, "bf16"), to_dev(wkb, "bf16"), to_dev(wvb, "bf16"))
    ko, vo = oracle.kv_bridge(hb, wkb, wvb)
    assert np.array_equal(bits_from_dev(k), ko) and np.array_equal(bits_from_dev(v), vo)


@pytest.mark.parametrize("T,D,d", [(1, 256, 128), (2, 256, 64), (3, 512, 128), (4, 256, 128), (5, 256, 64),
                                   (8, 2048, 128), (33, 256, 128), (64, 4096, 128), (65, 256, 128),
                                   (1, 4096, 64), (1, 4160, 128), (300, 512, 64), (513, 256, 128)])
def test_bridge_few_rows_exact(T, D, d):
    """Spans of a few rows (a decoded token's) on the vector-matrix kernel, and the sizes around its
    limits (T = 65 and D = 4160 take the MFMA tiles), plus MFMA spans with a ragged last 256-row tile
    at d = 64 and 128: integer operands, so bit-exact."""
    import token_level_sparse_mqa_amd as hs2
    import oracle
    from workloads.gen import f32_to_bf16_bits
    rng = np.random.default_rng(T * 7919 + D + d)
    hb = f32_to_bf16_bits(rng.integers(-3, 4, size=(T, D)).astype(np.float32))
    wkb = f32_to_bf16_bits(rng.integers(-3, 4, size=(D, d)).astype(np.float32))
    wvb = f32_to_bf16_bits(rng.integers(-3, 4, size=(D, d)).astype(np.float32))
    # rows written into the middle of a larger cache (row stride 2d), the rest left untouched
    cache = torch.full((T + 3, 2 * d), -5.0, dtype=torch.bfloat16, device="cuda")
    hs2.hs2_kv_bridge(to_dev(hb, "bf16"), to_dev(wkb, "bf16"), to_dev(wvb, "bf16"),
                      k_out=cache[2:2 + T, :d], v_out=cache[2:2 + T, d:], out_row_stride=2 * d)
    c = bits_from_dev(cache)
    ko, vo = oracle.kv_bridge(hb, wkb, wvb)
    assert np.array_equal(c[2:2 + T, :d], ko) and np.array_equal(c[2:2 + T, d:], vo)
    assert np.all(oracle.decode(c[:2], "bf16") == -5.0) and np.all(oracle.decode(c[2 + T:], "bf16") == -5.0)


@pytest.mark.parametrize("d", [64, 128])
def test_bridge_odd_stride_exact(d):
    """MFMA spans (ragged last tile) into rows whose stride is not a multiple of 4 elements and
    whose V part starts 2 bytes past an 8-byte boundary, so the kernel's 8-byte row writes are
    not allowed and it writes element by element: integer operands, bit-exact; the column
    between K and V and the rows around them stay untouched."""
    import token_level_sparse_mqa_amd as hs2
    import oracle
    from workloads.gen import f32_to_bf16_bits
    rng = np.random.default_rng(31 + d)
    T, D = 300, 256
    hb = f32_to_bf16_bits(rng.integers(-3, 4, size=(T, D)).astype(np.float32))
    wkb = f32_to_bf16_bits(rng.integers(-3, 4, size=(D, d)).astype(np.float32))
    wvb = f32_to_bf16_bits(rng.integers(-3, 4, size=(D, d)).astype(np.float32))
    cache = torch.full((T + 2, 2 * d + 1), -9.0, dtype=torch.bfloat16, device="cuda")
    hs2.hs2_kv_bridge(to_dev(hb, "bf16"), to_dev(wkb, "bf16"), to_dev(wvb, "bf16"),
                      k_out=cache[1:1 + T, :d], v_out=cache[1:1 + T, d + 1:], out_row_stride=2 * d + 1)
    c = bits_from_dev(cache)
    ko, vo = oracle.kv_bridge(hb, wkb, wvb)
    assert np.array_equal(c[1:1 + T, :d], ko) and np.array_equal(c[1:1 + T, d + 1:], vo)
    dec = oracle.decode(c, "bf16")
    assert np.all(dec[1:1 + T, d] == -9.0) and np.all(dec[0] == -9.0) and np.all(dec[1 + T] == -9.0)


def test_bridge_one_row_random():
    """One decoded token at the workload's width: random operands within the fp32 summation bound."""
    import token_level_sparse_mqa_amd as hs2
    import oracle
    from workloads.gen import f32_to_bf16_bits
    rng = np.random.default_rng(8)
    for T in (1, 7):
        D, d = 2048, 128
        hb = f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
        wkb = f32_to_bf16_bits((rng.standard_normal((D, d)) * 0.02).astype(np.float32))
        wvb = f32_to_bf16_bits((rng.standard_normal((D, d)) * 0.02).astype(np.float32))
        k, v = hs2.hs2_kv_bridge(to_dev(hb, "bf16"), to_dev(wkb, "bf16"), to_dev(wvb, "bf16"))
        ko, vo = oracle.kv_bridge(hb, wkb, wvb)
        check_bridge(hb, wkb, wvb, bits_from_dev(k), bits_from_dev(v), ko, vo, rate_check=False)


def test_bridge_strided_rows():
    import token_level_sparse_mqa_amd as hs2
    import oracle
    from workloads.gen import f32_to_bf16_bits
    rng = np.random.default_rng(6)
    T, D, d = 130, 128, 64
    hb = f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wkb = f32_to_bf16_bits((rng.standard_normal((D, d)) * 0.05).astype(np.float32))
    wvb = f32_to_bf16_bits((rng.standard_normal((D, d)) * 0.05).astype(np.float32))
    cache = torch.full((T, 3 * d), -7.0, dtype=torch.bfloat16, device="cuda")
    hs2.hs2_kv_bridge(to_dev(hb, "bf16"), to_dev(wkb, "bf16"), to_dev(wvb, "bf16"),
                      k_out=cache[:, d:2 * d], v_out=cache[:, 2 * d:], out_row_stride=3 * d)
    c = bits_from_dev(cache)
    ko, vo = oracle.kv_bridge(hb, wkb, wvb)
    assert np.all(oracle.decode(c[:, :d], "bf16") == -7.0)
    check_bridge(hb, wkb, wvb, np.ascontiguousarray(c[:, d:2 * d]), np.ascontiguousarray(c[:, 2 * d:]), ko, vo)


# ---------------------------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------------------------
def test_full_tiny():
    run_parity(CONFIGS["tiny"])


def test_full_decode128k():
    run_parity(CONFIGS["decode128k"])


def test_full_decode1m_fp8():
    run_parity(CONFIGS["decode1m_fp8"], score_tol=1e-7)


def _chunk_rows(cfg, extra_rows, n_groups, n_random, seed):
    """Rows of a full-size query chunk to check: the first and last row of n_groups of the chunk
    kernel's 8-query workgroups spread over the chunk (including the first and the last
    workgroup), the given rows, and n_random seeded rows."""
    rng = np.random.default_rng(seed)
    ngrp = cfg.Tq // 8
    rows = set()
    for gi in np.linspace(0, ngrp - 1, n_groups).round().astype(int):
        rows.update({(0, 8 * int(gi)), (0, 8 * int(gi) + 7)})
    rows.update(extra_rows)
    rows.update((0, int(i)) for i in rng.choice(cfg.Tq, size=n_random, replace=False))
    return sorted(rows)


def test_full_prefill_chunk_sampled():
    """prefill_chunk: every needle row (all 64), the first and last row of 12 workgroups and 8 seeded
    rows, with scores."""
    cfg = CONFIGS["prefill_chunk"]
    t0 = cfg.N - cfg.Tq
    from workloads.gen import _needle_plan
    needle_rows = [(0, t - t0) for (_, t, _, _) in _needle_plan(cfg)]
    rows = _chunk_rows(cfg, needle_rows, n_groups=12, n_random=8, seed=0)
    assert len(rows) >= 64
    run_parity(cfg, rows=rows, check_scores=True)


def test_full_prefill_exit256k_sampled():
    """prefill_exit256k: the bridge against the float64 projection, then the first and last row of
    24 workgroups and 20 seeded rows of the chunk, with scores."""
    cfg = CONFIGS["prefill_exit256k"]
    rows = _chunk_rows(cfg, [], n_groups=24, n_random=20, seed=1)
    assert len(rows) >= 64
    run_parity(cfg, rows=rows, check_scores=True)


def varlen_workload(cfg, lengths):
    """cfg's workload with sequences of different lengths: sequence b holds lengths[b] valid cache
    rows, its queries are the last Tq positions of those, and every cache row past its length is
    NaN (K and V; for FP8 the codes and the row scales), so a kernel that read past kv_len, or let
    a masked row's data into a product, would put NaN into the outputs."""
    wl = make_workload(cfg)
    L = np.asarray(lengths, dtype=np.int32)
    assert L.shape == (cfg.B,) and np.all(L <= cfg.N) and np.all(L >= cfg.Tq)
    wl.kv_len = L.copy()
    wl.q_pos = (L[:, None] - cfg.Tq + np.arange(cfg.Tq, dtype=np.int32)[None, :]).astype(np.int32)
    for b, n in enumerate(L):
        if cfg.kv_dtype == "bf16":
            wl.k[b, n:] = 0x7FC0
            wl.v[b, n:] = 0x7FC0
        elif cfg.kv_dtype == "fp8":
            wl.k[b, n:] = 0x7F
            wl.v[b, n:] = 0x7F
            wl.k_scale[b, n:] = np.nan
            wl.v_scale[b, n:] = np.nan
        else:
            wl.k[b, n:] = np.nan
            wl.v[b, n:] = np.nan
    return wl


VARLEN = [
    # decode rows: one full-length sequence, one mid-length, one just above k + W candidates
    (small_config("varlen_rows", 240, B=3, N=4000, Tq=2, n_sparse=1), [4000, 2600, 1300]),
    (small_config("varlen_fp8", 241, B=2, N=5000, Tq=1, kv_dtype="fp8", n_sparse=1), [3100, 5000]),
    (small_config("varlen_f32", 242, B=2, N=1500, Tq=2, H=16, d=64, q_dtype="f32", kv_dtype="f32",
                  n_sparse=1), [1500, 1200]),
    # query chunks: the 8-query workgroups stop at their own sequence's last row
    (small_config("varlen_chunk", 243, B=2, N=3000, Tq=24, n_sparse=1), [3000, 1900]),
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: c[0].name)
def test_varlen_poisoned_tail(case):
    cfg, lengths = case
    g, wl, idx, O = run_parity(cfg, wl=varlen_workload(cfg, lengths))
    # every index lies below its own sequence's length
    idx_h = idx.cpu().numpy()
    for b, n in enumerate(lengths):
        assert np.all(idx_h[b] < n)


SPARSE_LISTS = [("bf16", 300), ("bf16", 1152), ("fp8", 777)]


@pytest.mark.parametrize("kv, S", SPARSE_LISTS, ids=lambda x: str(x))
def test_sparse_list_semantics(kv, S):
    """hs2_sparse_attn on lists the selection never produces, against its documented semantics:
    entries outside [0, min(kv_len, Nmax)) are skipped like -1 (including rows inside Nmax but past
    the sequence's length), repeated entries count once per occurrence, and a row with no valid
    entry gets o = 0.  The expected value filters the list by that rule and hands the rest to the
    oracle's sparse attention; the split and the one-workgroup forms are both checked."""
    cfg = small_config(f"sparse_lists_{kv}_{S}", 250 + S % 97 + (kv == "fp8"), B=2, N=3000, Tq=3,
                       kv_dtype=kv, n_sparse=1)
    _say(f"[sparse-lists] {cfg.name}")
    wl = make_workload(cfg)
    L = np.array([3000, 2200], dtype=np.int32)
    wl.kv_len = L
    rng = np.random.default_rng(cfg.cfg_id)
    idx = np.empty((cfg.B, cfg.Tq, S), dtype=np.int32)
    for b in range(cfg.B):
        for i in range(cfg.Tq):
            if (b, i) == (1, 2):
                # nothing valid: -1, past this sequence's length but inside Nmax, past Nmax
                row = rng.choice(np.array([-1, -7, int(L[1]), int(L[1]) + 5, cfg.N - 1, cfg.N, cfg.N + 7, 2 ** 30]),
                                 size=S)
            else:
                row = rng.choice(cfg.N, size=S, replace=False).astype(np.int64)
                u = rng.random(S)
                row[u < 0.10] = -1                                     # holes
                past = (u >= 0.10) & (u < 0.14)
                row[past] = cfg.N + rng.integers(0, 1000, size=int(past.sum()))      # past Nmax
                rep = (u >= 0.14) & (u < 0.19)                         # repeats of earlier entries
                src = rng.integers(0, S, size=int(rep.sum()))
                row[rep] = row[src]
            idx[b, i] = row.astype(np.int32)
    g = HipRun(wl)
    O = OracleRun(wl)
    tol = tol_for(cfg.kv_dtype)
    idx_dev = to_dev(idx, "i32")
    for ws in (True, False):
        o = g.sparse(0, idx_dev, workspace=ws).cpu().numpy()
        for b in range(cfg.B):
            for i in range(cfg.Tq):
                row = idx[b, i].astype(np.int64)
                keep = row[(row >= 0) & (row < min(int(L[b]), cfg.N))]
                ref = O.sparse_row(0, b, i, keep)
                err = float(np.max(np.abs(o[b, i] - ref)))
                assert err <= tol, f"ws={ws} row {(b, i)}: error {err:.3e} > {tol}"
                if keep.shape[0] == 0:
                    assert np.all(o[b, i] == 0.0)
    # kv_len omitted (NULL): every entry below Nmax counts, also those past the sequence's length
    import token_level_sparse_mqa_amd as hs2
    o = hs2.hs2_sparse_attn(g.qs[0], g.k, g.v, idx_dev, kv_len=None, k_scale=g.k_scale, v_scale=g.v_scale,
                            sm_scale=g.sm).cpu().numpy()
    for b in range(cfg.B):
        for i in range(cfg.Tq):
            row = idx[b, i].astype(np.int64)
            ref = O.sparse_row(0, b, i, row[(row >= 0) & (row < cfg.N)])
            err = float(np.max(np.abs(o[b, i] - ref)))
            assert err <= tol, f"kv_len=None row {(b, i)}: error {err:.3e} > {tol}"
    _say(f"[sparse-lists] {cfg.name} ok")


SCATTERED = [
    small_config("scattered_rows", 244, B=2, N=3000, Tq=5, n_sparse=1),
    small_config("scattered_chunk", 245, B=1, N=3000, Tq=24, n_sparse=1),
    small_config("scattered_chunk_fp8", 246, B=2, N=2500, Tq=16, kv_dtype="fp8", n_sparse=1),
]


@pytest.mark.parametrize("cfg", SCATTERED, ids=lambda c: c.name)
def test_scattered_positions(cfg):
    """Query positions in any order, not the last Tq of the sequence: unsorted, spread over the
    whole sequence (some with fewer than k + W visible keys, one at position 0) and repeated, so
    the 8-query workgroups of the chunk kernels span very different key ranges."""
    wl = make_workload(cfg)
    rng = np.random.default_rng(cfg.cfg_id)
    pos = rng.integers(0, cfg.N, size=(cfg.B, cfg.Tq)).astype(np.int32)
    pos[0, 0] = 0
    pos[0, 1] = cfg.N - 1
    pos[-1, -1] = pos[-1, 0]                    # a repeated position
    pos[0, 2] = 700                             # fewer candidates than k
    wl.q_pos = pos
    run_parity(cfg, wl=wl)


def test_two_streams_concurrently():
    """A decode workload and a query chunk (full layer, selection and a sparse layer, each call with
    its own workspace) on two streams at once equal the same calls run one after another: the
    entry points share no state between calls."""
    import token_level_sparse_mqa_amd as hs2
    cfgs = [small_config("streams_decode", 280, B=2, N=6000, Tq=1, n_sparse=1),
            small_config("streams_chunk", 281, B=1, N=9000, Tq=16, n_sparse=1)]
    runs = [HipRun(make_workload(c)) for c in cfgs]

    def step(g, cfg):
        o, idx = hs2.hs2_full_attn_select(g.q, g.k, g.v, g.q_pos, g.kv_len, k_global=cfg.k_global,
                                          window=cfg.window, sm_scale=g.sm)
        return o, idx, g.sparse(0, idx)

    ref = [step(g, c) for g, c in zip(runs, cfgs)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        outs = []
        for g, c, s in zip(runs, cfgs, streams):
            with torch.cuda.stream(s):
                outs.append(step(g, c))
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            for x, y in zip(got, want):
                assert torch.equal(x, y), f"repeat {rep}: a concurrent call differs from the sequential one"
