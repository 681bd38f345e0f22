"""The agentic multi-turn loop on the GPU against the oracle.

One trace grows through rounds of decoded action tokens and prefilled observation chunks.  Every
appended span goes through the KV bridge (rows written in place into a cache of fixed capacity),
the full-attention layer with selection, and the sparse layers on the loop's own indices.  The
cache past the current length holds NaN, so a read of a row that is not yet written shows up in
the outputs.

Checks, per query row (position t):
  * the full layer's o and indices against the oracle on the oracle's own bridge of the same
    hidden states (the parity protocol of the other workloads: exact window, selection equal
    outside the near-tie band, o within 2e-3);
  * the sparse layers: where the loop's indices equal the oracle's, the loop's own outputs against
    the oracle's; elsewhere the span's sparse layers are run again on the oracle's indices;
  * after the loop: the cache against the oracle's bridge (per-element fp32 summation bound), and
    the rows past the final length still NaN.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from tests.hs2_harness import _say, bits_from_dev, check_bridge, check_indices, to_dev, tol_for
from workloads import AgenticConfig, make_agentic

pytestmark = pytest.mark.gpu

SMALL = [
    # a 2,048-token trace, 2 rounds of 3 action tokens and a 200-token observation (ragged tiles)
    AgenticConfig("agentic_small", 240, N0=2048, turns=2, act=3, obs=200, H=8, d=128, D=512, n_sparse=2),
    # the context crosses k + W = 1152 during the loop: rows with fewer candidates than k first
    AgenticConfig("agentic_grow", 241, N0=600, turns=3, act=2, obs=300, H=16, d=64, D=256, n_sparse=1),
]
SLACK = 40          # cache rows past the final length, left NaN


def run_loop(cfg: AgenticConfig):
    import token_level_sparse_mqa_amd as hs2
    from token_level_sparse_mqa_amd.agentic import AgenticSession
    inp = make_agentic(cfg)
    hid = to_dev(inp.hidden, "bf16")
    qf = to_dev(inp.q_full, "bf16")
    qs = [to_dev(x, "bf16") for x in inp.q_sparse]
    sess = AgenticSession(to_dev(inp.wk, "bf16"), to_dev(inp.wv, "bf16"), capacity=cfg.N_final + SLACK,
                          H=cfg.H, n_sparse=cfg.n_sparse, max_span=cfg.obs, k_global=cfg.k_global,
                          window=cfg.window, fill=float("nan"))
    sess.bridge_prefix(hid[:cfg.N0])
    out = []
    for (kind, p, T) in cfg.phases():
        j = p - cfg.N0
        o, idx, o_sp = sess.append(hid[p:p + T], qf[j:j + T], [x[j:j + T] for x in qs])
        out.append((kind, p, T, o[0].cpu().numpy(), idx[0].cpu().numpy(), [x[0].cpu().numpy() for x in o_sp]))
    torch.cuda.synchronize()
    assert sess.length == cfg.N_final
    return inp, sess, out, hs2


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_agentic_loop(cfg):
    _say(f"[agentic] {cfg.name} N0={cfg.N0} turns={cfg.turns} act={cfg.act} obs={cfg.obs} H={cfg.H} "
         f"d={cfg.d} D={cfg.D} L={cfg.n_sparse}")
    inp, sess, out, hs2 = run_loop(cfg)
    kb_gpu, vb_gpu = bits_from_dev(sess.k[0]), bits_from_dev(sess.v[0])
    # rows past the final length were never written
    tail_k = oracle.decode(kb_gpu[cfg.N_final:], "bf16")
    tail_v = oracle.decode(vb_gpu[cfg.N_final:], "bf16")
    assert np.all(np.isnan(tail_k)) and np.all(np.isnan(tail_v))
    kb, vb = oracle.kv_bridge(inp.hidden, inp.wk, inp.wv)
    check_bridge(inp.hidden, inp.wk, inp.wv, kb_gpu[:cfg.N_final], vb_gpu[:cfg.N_final], kb, vb)
    K, V = oracle.decode(kb, "bf16"), oracle.decode(vb, "bf16")
    sm = 1.0 / math.sqrt(cfg.d)
    tol = tol_for("bf16")
    qf = oracle.decode(inp.q_full, "bf16")
    qs = [oracle.decode(x, "bf16") for x in inp.q_sparse]
    mismatch_rows, o_err, sp_err, reruns = 0, 0.0, 0.0, 0
    for (kind, p, T, o, idx, o_sp) in out:
        j0 = p - cfg.N0
        idx_or = np.empty_like(idx)
        rerun = []
        for i in range(T):
            t = p + i
            o_o, idx_o, sc_o = oracle.full_attn_select_row(qf[j0 + i], K, V, t, sm, cfg.k_global, cfg.window)
            check_indices(idx[i], idx_o, sc_o, t, cfg.k_global, cfg.window)
            err = float(np.max(np.abs(o[i] - o_o)))
            o_err = max(o_err, err)
            assert err <= tol, f"{kind} span at {p}, row {i}: full-layer o error {err:.3e}"
            idx_or[i] = idx_o
            same = np.array_equal(idx[i], idx_o)
            if not same:
                mismatch_rows += 1
                rerun.append(i)
            for l in range(cfg.n_sparse):
                ref = oracle.sparse_attention_row(qs[l][j0 + i], K, V, idx_o, sm)
                if same:
                    e = float(np.max(np.abs(o_sp[l][i] - ref)))
                    sp_err = max(sp_err, e)
                    assert e <= tol, f"{kind} span at {p}, row {i}, sparse layer {l}: error {e:.3e}"
        if rerun:
            # the loop's indices differ from the oracle's only inside the near-tie band: run this
            # span's sparse layers again on the oracle's indices (same cache, same kv_len)
            reruns += 1
            qd = [to_dev(x[j0:j0 + T], "bf16").view(1, T, cfg.H, cfg.d) for x in inp.q_sparse]
            kv_len = torch.tensor([p + T], dtype=torch.int32, device="cuda")
            got = hs2.hs2_sparse_attn_layers(qd, sess.k, sess.v, to_dev(idx_or[None], "i32"), kv_len=kv_len,
                                             sm_scale=sm)
            for l in range(cfg.n_sparse):
                g = got[l][0].cpu().numpy()
                for i in rerun:
                    ref = oracle.sparse_attention_row(qs[l][j0 + i], K, V, idx_or[i], sm)
                    e = float(np.max(np.abs(g[i] - ref)))
                    sp_err = max(sp_err, e)
                    assert e <= tol, f"{kind} span at {p}, row {i}, sparse layer {l} (oracle idx): {e:.3e}"
    _say(f"[agentic] {cfg.name} ok: spans={len(out)} rows={cfg.n_new} band-mismatch rows={mismatch_rows} "
         f"o_err={o_err:.2e} sparse_err={sp_err:.2e} reruns={reruns}")


def test_agentic_session_errors():
    """Spans past the capacity or max_span, and a wrong number of sparse queries, are rejected."""
    from token_level_sparse_mqa_amd.agentic import AgenticSession
    cfg = SMALL[0]
    dev = "cuda"
    w = torch.zeros((cfg.D, cfg.d), dtype=torch.bfloat16, device=dev)
    sess = AgenticSession(w, w, capacity=16, H=cfg.H, n_sparse=1, max_span=8)
    h = torch.zeros((9, cfg.D), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((9, cfg.H, cfg.d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        sess.append(h, q, [q])                      # 9 > max_span
    with pytest.raises(ValueError):
        sess.append(h[:2], q[:2], [])               # one sparse query expected
    sess.bridge_prefix(h[:9])
    with pytest.raises(ValueError):
        sess.append(h[:8], q[:8], [q[:8]])          # 9 + 8 > capacity
    o, idx, o_sp = sess.append(h[:7], q[:7], [q[:7]])
    torch.cuda.synchronize()
    assert sess.length == 16
    # zero queries over zero keys: uniform weights, window indices only
    assert torch.all(idx[0, :, :cfg.k_global] == -1)


def test_agentic_graph_replay():
    """The whole multi-turn step captured in one HIP graph: every replay (with eager work and
    synchronisations between them) reproduces the eager step's outputs and cache bit for bit."""
    from token_level_sparse_mqa_amd.agentic import AgenticSession
    cfg = SMALL[0]
    inp = make_agentic(cfg)
    hid, qf = to_dev(inp.hidden, "bf16"), to_dev(inp.q_full, "bf16")
    qs = [to_dev(x, "bf16") for x in inp.q_sparse]
    sess = AgenticSession(to_dev(inp.wk, "bf16"), to_dev(inp.wv, "bf16"), capacity=cfg.N_final, H=cfg.H,
                          n_sparse=cfg.n_sparse, max_span=cfg.obs)
    sess.bridge_prefix(hid[:cfg.N0])
    spans = [(hid[p:p + T], qf[p - cfg.N0:p - cfg.N0 + T], [x[p - cfg.N0:p - cfg.N0 + T] for x in qs])
             for (_, p, T) in cfg.phases()]
    res = [(torch.empty((T, cfg.H, cfg.d), dtype=torch.float32, device="cuda"),
            torch.empty((T, cfg.S), dtype=torch.int32, device="cuda"),
            torch.empty((cfg.n_sparse, T, cfg.H, cfg.d), dtype=torch.float32, device="cuda"))
           for (_, _, T) in cfg.phases()]

    def step():
        sess.reset(cfg.N0)
        for (h, q, q_sp), (ro, ri, rs) in zip(spans, res):
            o, idx, o_sp = sess.append(h, q, q_sp)
            ro.copy_(o[0])
            ri.copy_(idx[0])
            for l in range(cfg.n_sparse):
                rs[l].copy_(o_sp[l][0])

    step()
    torch.cuda.synchronize()
    ref = [tuple(x.clone() for x in r) for r in res]
    kref, vref = sess.k.clone(), sess.v.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for r in res:
            for x in r:
                x.zero_()
        sess.k[0, cfg.N0:].zero_()
        sess.v[0, cfg.N0:].zero_()
        a = torch.randn((512, 512), device="cuda")
        (a @ a).sum().item()                                   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for s, (r, rr) in enumerate(zip(res, ref)):
            for x, y in zip(r, rr):
                assert torch.equal(x, y), f"replay {rep}, span {s} differs from the eager step"
        assert torch.equal(sess.k, kref) and torch.equal(sess.v, vref), f"replay {rep}: cache differs"
