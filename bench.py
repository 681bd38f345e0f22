"""Throughput of the hybrid-block hot path on one MI355X.

A step is one pass of the whole hot path over one batch: the full-attention MQA layer with
token-level selection (hs2_full_attn_select) followed by the index-reusing sparse layers
(hs2_sparse_attn_layers), plus the KV bridge for the prefill-exit workload.  Inputs are resident in
HBM before the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode128k]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query tokens/s for select+sparse attn at 128K & 1M ctx; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BLOCK = 64                      # block-level selection: positions per block
BF16_PEAK_TFLOPS = 2500.0
SLEEP_CYCLES = 200000           # ~0.1 ms of GPU sleep queued ahead of a timed region


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def upload(wl, dev):
    import torch

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    cfg = wl.cfg
    t = {"q": up(wl.q_full, cfg.q_dtype), "qs": [up(x, cfg.q_dtype) for x in wl.q_sparse],
         "q_pos": up(wl.q_pos, "i32"), "kv_len": up(wl.kv_len, "i32"), "k_scale": None, "v_scale": None}
    if cfg.bridge_D:
        t["hidden"], t["wk"], t["wv"] = up(wl.hidden, "bf16"), up(wl.wk, "bf16"), up(wl.wv, "bf16")
        t["k"] = torch.empty((1, cfg.N, cfg.d), dtype=torch.bfloat16, device=dev)
        t["v"] = torch.empty((1, cfg.N, cfg.d), dtype=torch.bfloat16, device=dev)
    else:
        t["k"], t["v"] = up(wl.k, cfg.kv_dtype), up(wl.v, cfg.kv_dtype)
        if cfg.kv_dtype == "fp8":
            t["k_scale"], t["v_scale"] = up(wl.k_scale, "f32"), up(wl.v_scale, "f32")
    return t


def kv_bytes_per_row(cfg):
    b = {"bf16": 2, "f32": 4, "fp8": 1}[cfg.kv_dtype]
    return cfg.d * b + (4 if cfg.kv_dtype == "fp8" else 0)


def algorithmic(cfg):
    """Algorithmic bytes / flops per launch of each kernel, and per step (what the method must
    move or compute; the second K pass of the score and split bookkeeping are excluded)."""
    rows = cfg.B * cfg.Tq
    kvb = kv_bytes_per_row(cfg)
    qb = {"bf16": 2, "f32": 4}[cfg.q_dtype] * cfg.H * cfg.d
    # visible (query, key) pairs and unique cache rows touched
    pairs = sum(cfg.N - cfg.Tq + i + 1 for i in range(cfg.Tq)) * cfg.B
    full_bytes = cfg.B * cfg.N * 2 * kvb + rows * (qb + cfg.H * cfg.d * 4 + cfg.S * 4)
    full_flops = 4.0 * cfg.H * cfg.d * pairs
    sparse_bytes = rows * (cfg.S * 2 * kvb + cfg.S * 4 + qb + cfg.H * cfg.d * 4)
    sparse_flops = 4.0 * cfg.H * cfg.d * cfg.S * rows
    out = {
        "full_attn": {"bytes": cfg.B * cfg.N * 2 * kvb, "flops": full_flops},
        "sparse_attn": {"bytes": sparse_bytes, "flops": sparse_flops},
        # all sparse layers in one launch: each layer still gathers its rows
        "sparse_layers": {"bytes": cfg.n_sparse * sparse_bytes, "flops": cfg.n_sparse * sparse_flops},
        "step": {"bytes": full_bytes + cfg.n_sparse * sparse_bytes,
                 "flops": full_flops + cfg.n_sparse * sparse_flops},
    }
    if cfg.bridge_D:
        out["bridge"] = {"bytes": cfg.N * (cfg.bridge_D * 2 + 4 * cfg.d) + 4 * cfg.bridge_D * cfg.d,
                         "flops": 2.0 * cfg.N * cfg.bridge_D * 2 * cfg.d}
        out["step"]["bytes"] += out["bridge"]["bytes"]
        out["step"]["flops"] += out["bridge"]["flops"]
    return out


# kernel name -> (algorithmic unit key, bound)
KERNEL_UNITS = {
    "full_attn_generic": ("full_attn", "hbm"),
    "full_attn_mfma": ("full_attn", "hbm"),
    "full_attn_prefill": ("full_attn", "mfma"),
    "sparse_attn_generic": ("sparse_attn", "hbm"),
    "sparse_attn_mfma": ("sparse_attn", "hbm"),
    "sparse_attn_layers_mfma": ("sparse_layers", "hbm"),
    "bridge_mfma": ("bridge", "hbm"),
    "bridge_rows": ("bridge", "hbm"),
    "bridge_fp8": ("bridge_fp8", "mfma"),
    "decode_block": ("step", "hbm"),
}
KERNEL_SOURCES = {
    "full_attn_mfma": ["attn_rows.hip", "attn_rows_dev.h", "mfma_tiles.h"],
    "score_rows_mfma": ["score_rows.hip", "score_rows_dev.h", "mfma_tiles.h"],
    "score_prefill": ["attn_prefill.hip", "mfma_tiles.h"],
    "full_attn_prefill": ["attn_prefill.hip", "mfma_tiles.h"],
    "sparse_attn_mfma": ["attn_rows.hip", "attn_rows_dev.h", "mfma_tiles.h"],
    "sparse_attn_layers_mfma": ["attn_rows.hip", "attn_rows_dev.h", "mfma_tiles.h"],
    "bridge_mfma": ["bridge_mfma.hip", "mfma_tiles.h"],
    "bridge_rows": ["bridge_rows.hip"],
    "bridge_fp8": ["bridge_fp8.hip"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(ROOT, "token_level_sparse_mqa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a copy kernel
    of known size), or None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("src_sha") != kernel_source_hash(kernel):
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def timed_steps(step, nsteps):
    """K steps back to back on the current stream, an event before each and one after the last:
    (median ms per step, mean ms per step, wall seconds of the region).  A short GPU sleep queued
    ahead of the first event keeps the host's launch latency out of the first step."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    torch.cuda._sleep(SLEEP_CYCLES)
    for i in range(nsteps):
        ev[i].record(stream)
        step()
    ev[nsteps].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(nsteps))
    return per[len(per) // 2], ev[0].elapsed_time(ev[nsteps]) / nsteps, wall


def cold_steps(step, nsteps, flush):
    """Median ms of one step with the L2 and memory-side cache flushed before it (a 512 MiB buffer
    written between steps, outside the events)."""
    import torch
    per = []
    for r in range(nsteps):
        flush.fill_(r & 0xFF)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(SLEEP_CYCLES)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1))
    per.sort()
    return per[len(per) // 2]


def stored_counters(workload, kernel):
    """Compute-unit counters of the kernel from the committed rocprofv3 summary
    (profiles/<kernel>_<workload>_counters.json: MFMA busy, VALU busy), or None when there is none
    or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("src_sha") != kernel_source_hash(kernel):
        return None
    return {k: rec[k] for k in ("mfma_busy", "valu_busy", "mfma_flops_frac") if k in rec}


def run_gpu(cfg, steps, warmup, profile=True, select="token", decode_block=False, layers="sequential",
            supplements=True):
    """One hybrid block per step.  layers="sequential": the sparse layers as one hs2_sparse_attn
    call each, in order, as a decoder runs them (layer l+1's queries come from layer l's output);
    layers="fused": all sparse layers in one hs2_sparse_attn_layers call (their queries given
    up front).  Supplements: the other layer mode and a cold-cache step time."""
    import torch

    import token_level_sparse_mqa_amd as hs2
    from workloads import make_workload

    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name}")
    wl = make_workload(cfg)
    t = upload(wl, dev)
    sm = 1.0 / math.sqrt(cfg.d)
    R = cfg.B * cfg.Tq
    kvd = hs2.dtype_code(t["k"])
    blocks = select == "blocks"
    kb = cfg.k_global // BLOCK
    if blocks:
        nws = hs2.hs2_full_attn_select_blocks_workspace_size(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.N, kb, BLOCK,
                                                             cfg.window, kvd)
    else:
        nws = hs2.hs2_full_attn_select_workspace_size(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.N, cfg.k_global, cfg.window,
                                                      kvd)
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    bidx = torch.empty((cfg.B, cfg.Tq, kb), dtype=torch.int32, device=dev)
    sws = hs2.sparse_attn_layers_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.S, cfg.n_sparse, dev)
    sws1 = hs2.sparse_attn_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.S, dev)
    o = torch.empty((cfg.B, cfg.Tq, cfg.H, cfg.d), dtype=torch.float32, device=dev)
    idx = torch.empty((cfg.B, cfg.Tq, cfg.S), dtype=torch.int32, device=dev)
    o_sp = [torch.empty_like(o) for _ in range(cfg.n_sparse)]

    if decode_block:
        dbws = hs2.decode_block_workspace(cfg.B, cfg.Tq, cfg.H, cfg.d, cfg.N, cfg.k_global, cfg.window, kvd,
                                          cfg.n_sparse, dev)

    def full():
        if cfg.bridge_D:
            hs2.hs2_kv_bridge(t["hidden"], t["wk"], t["wv"], k_out=t["k"][0], v_out=t["v"][0])
        if blocks:
            hs2.hs2_full_attn_select_blocks(t["q"], t["k"], t["v"], t["q_pos"], t["kv_len"], k_scale=t["k_scale"],
                                            v_scale=t["v_scale"], k_blocks=kb, block=BLOCK, window=cfg.window,
                                            sm_scale=sm, o=o, block_idx=bidx, idx=idx, workspace=ws)
        else:
            hs2.hs2_full_attn_select(t["q"], t["k"], t["v"], t["q_pos"], t["kv_len"], k_scale=t["k_scale"],
                                     v_scale=t["v_scale"], k_global=cfg.k_global, window=cfg.window, sm_scale=sm,
                                     o=o, idx=idx, workspace=ws)

    def step_sequential():
        full()
        for layer in range(cfg.n_sparse):
            hs2.hs2_sparse_attn(t["qs"][layer], t["k"], t["v"], idx, kv_len=t["kv_len"], k_scale=t["k_scale"],
                                v_scale=t["v_scale"], sm_scale=sm, o=o_sp[layer], workspace=sws1)

    def step_fused():
        full()
        hs2.hs2_sparse_attn_layers(t["qs"], t["k"], t["v"], idx, kv_len=t["kv_len"], k_scale=t["k_scale"],
                                   v_scale=t["v_scale"], sm_scale=sm, os=o_sp, workspace=sws)

    def step_block():
        # the whole block (full layer, selection, sparse layers) in one launch
        hs2.hs2_decode_block(t["q"], t["qs"], t["k"], t["v"], t["q_pos"], t["kv_len"], k_scale=t["k_scale"],
                             v_scale=t["v_scale"], k_global=cfg.k_global, window=cfg.window, sm_scale=sm,
                             o=o, idx=idx, os=o_sp, workspace=dbws)

    step = step_block if decode_block else (step_sequential if layers == "sequential" else step_fused)
    log(f"[bench] warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {steps} steps")
    ms, ms_mean, wall = timed_steps(step, steps)
    res = {"ms_per_step": ms, "ms_mean": ms_mean, "wall_s": wall, "rows": R, "wl": wl, "layers": layers}
    if supplements and not decode_block:
        other = step_fused if layers == "sequential" else step_sequential
        for _ in range(2):
            other()
        res["ms_other_layers"], _, _ = timed_steps(other, steps)
        log(f"[bench] cold-cache steps")
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        res["ms_cold"] = cold_steps(step, steps, flush)
        del flush
    kernels = {}
    if profile:
        # per-kernel durations from a second region of the same length (an event record between
        # two kernels of a step serialises them, so the step time above has none)
        log(f"[bench] per-kernel event timing, {steps} steps")
        hs2.profile_enable(True)
        timed_steps(step, steps)
        kernels = hs2.profile_read()
        hs2.profile_enable(False)
    res["kernels"] = kernels
    return res


def agentic_units(cfg):
    """Algorithmic bytes / flops of one agentic step (every span of every round), per kernel family:
    the prefill attention over the observation chunks, the decode attention of the action tokens, the
    sparse layers of all spans, and the bridge of all new rows."""
    kvb = 2 * cfg.d                       # one bf16 K or V row
    qb = 2 * cfg.H * cfg.d
    units = {"full_attn_prefill": {"bytes": 0.0, "flops": 0.0}, "full_attn_mfma": {"bytes": 0.0, "flops": 0.0},
             "sparse_layers": {"bytes": 0.0, "flops": 0.0}, "bridge": {"bytes": 0.0, "flops": 0.0},
             "prefill_launches": 0, "decode_launches": 0}
    for (kind, p, T) in cfg.phases():
        pairs = sum(p + i + 1 for i in range(T))
        key = "full_attn_prefill" if kind == "obs" else "full_attn_mfma"
        units[key]["bytes"] += (p + T) * 2 * kvb
        units[key]["flops"] += 4.0 * cfg.H * cfg.d * pairs
        units["prefill_launches" if kind == "obs" else "decode_launches"] += 1
        units["sparse_layers"]["bytes"] += cfg.n_sparse * T * (cfg.S * 2 * kvb + cfg.S * 4 + qb + cfg.H * cfg.d * 4)
        units["sparse_layers"]["flops"] += cfg.n_sparse * 4.0 * cfg.H * cfg.d * cfg.S * T
        units["bridge"]["bytes"] += T * (cfg.D * 2 + 4 * cfg.d) + 4 * cfg.D * cfg.d
        units["bridge"]["flops"] += 2.0 * T * cfg.D * 2 * cfg.d
    return units


def run_agentic(cfg, steps, warmup, profile=True):
    """The multi-turn loop: a step rewinds the session to the initial trace and runs every round
    (act decoded tokens, then one observation chunk), bridging each new token into the cache.  It is
    timed twice: launched from Python, and replayed from one HIP graph captured from the same calls."""
    import torch

    import token_level_sparse_mqa_amd as hs2
    from token_level_sparse_mqa_amd.agentic import AgenticSession
    from workloads import make_agentic

    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name}")
    inp = make_agentic(cfg)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    hid, qf, qs = up(inp.hidden), up(inp.q_full), [up(x) for x in inp.q_sparse]
    sess = AgenticSession(up(inp.wk), up(inp.wv), capacity=cfg.N_final, H=cfg.H, n_sparse=cfg.n_sparse,
                          max_span=cfg.obs, k_global=cfg.k_global, window=cfg.window)
    sess.bridge_prefix(hid[:cfg.N0])
    spans = [(hid[p:p + T], qf[p - cfg.N0:p - cfg.N0 + T], [x[p - cfg.N0:p - cfg.N0 + T] for x in qs])
             for (_, p, T) in cfg.phases()]

    def step():
        sess.reset(cfg.N0)
        for (h, q, q_sp) in spans:
            sess.append(h, q, q_sp)

    log(f"[bench] warmup {warmup}")
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()

    def timed(fn, nsteps):
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(nsteps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / nsteps, time.perf_counter() - w0

    log(f"[bench] timing {steps} eager steps")
    ms_eager, _ = timed(step, steps)
    log("[bench] capturing the step in a HIP graph")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()                      # one more warm pass on the capture stream (no allocation left)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {steps} graph replays")
    ms_graph, wall = timed(graph.replay, steps)
    kernels = {}
    if profile:
        log(f"[bench] per-kernel event timing, {steps} eager steps")
        hs2.profile_enable(True)
        timed(step, steps)
        kernels = hs2.profile_read()
        hs2.profile_enable(False)
    return {"ms_per_step": ms_graph, "ms_eager": ms_eager, "wall_s": wall, "rows": cfg.n_new,
            "kernels": kernels, "inp": inp, "steps": steps}


def agentic_cpu_baseline(cfg, inp, budget_s=20.0):
    """The oracle on a bounded sample of the agentic step: the trace's K/V are bridged first
    (untimed, as on the GPU), then spans in loop order, each bridging its rows and running every
    row's full layer, selection and sparse layers, until the budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    sm = 1.0 / math.sqrt(cfg.d)
    kb, vb = oracle.kv_bridge(inp.hidden[:cfg.N0], inp.wk, inp.wv)
    K = np.empty((cfg.N_final, cfg.d))
    V = np.empty((cfg.N_final, cfg.d))
    K[:cfg.N0], V[:cfg.N0] = oracle.decode(kb, "bf16"), oracle.decode(vb, "bf16")
    t0 = time.perf_counter()
    done = 0
    for (kind, p, T) in cfg.phases():
        kb, vb = oracle.kv_bridge(inp.hidden[p:p + T], inp.wk, inp.wv)
        K[p:p + T], V[p:p + T] = oracle.decode(kb, "bf16"), oracle.decode(vb, "bf16")
        for i in range(T):
            j = p - cfg.N0 + i
            _, idx, _ = oracle.full_attn_select_row(oracle.decode(inp.q_full[j], "bf16"), K, V, p + i, sm,
                                                    cfg.k_global, cfg.window)
            for l in range(cfg.n_sparse):
                oracle.sparse_attention_row(oracle.decode(inp.q_sparse[l][j], "bf16"), K, V, idx, sm)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {done} new tokens of one {cfg.name} step in loop order (bridge of their rows, "
                      f"full layer + selection + {cfg.n_sparse} sparse layers per token; the initial "
                      f"{cfg.N0}-row trace bridged beforehand, untimed), {el:.1f} s"}


def agentic_main(cfg, args):
    res = run_agentic(cfg, args.steps, args.warmup, profile=not args.no_profile)
    ms = res["ms_per_step"]
    units = agentic_units(cfg)
    kernels = {}
    for name, (tot, n) in res["kernels"].items():
        kernels[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
    roof = None
    if "full_attn_prefill" in kernels:
        k = kernels["full_attn_prefill"]
        per_step_s = k["avg_us"] * k["launches"] / res["steps"] / 1e6
        ach = units["full_attn_prefill"]["flops"] / per_step_s / 1e12
        roof = {"bound": "mfma", "kernel": "full_attn_prefill", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": stored_traffic(cfg.name, "full_attn_prefill"),
                "per": f"sum over the step's {units['prefill_launches']} observation chunks"}
    n_act = cfg.turns * cfg.act
    out = {
        "metric": "agentic loop: new tokens/s (action decode + observation prefill over a growing context)",
        "value": cfg.n_new / (ms / 1e3), "unit": "new tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": 1, "initial_context": cfg.N0, "final_context": cfg.N_final,
                   "turns": cfg.turns, "action_tokens": cfg.act, "observation_tokens": cfg.obs, "H": cfg.H,
                   "d": cfg.d, "bridge_D": cfg.D, "kv_dtype": "bf16", "k_global": cfg.k_global,
                   "window": cfg.window, "sparse_layers": cfg.n_sparse, "launch": "hip graph replay"},
        "ms_per_step_eager": res["ms_eager"],
        "roofline": roof, "kernels": kernels,
    }
    out["config"]["action_tokens_per_step"] = n_act
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = agentic_cpu_baseline(cfg, res["inp"])
    print(json.dumps(out), flush=True)


def bridge_fp8_main(cfg, args):
    """Multi-target FP8 bridge: a step is one hs2_kv_bridge_fp8 call, all targets' K/V caches of
    cfg.T tokens projected from the same hidden states (resident in HBM) and quantised."""
    import torch

    import token_level_sparse_mqa_amd as hs2
    from workloads import make_bridge_fp8_inputs

    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name}")
    inp = make_bridge_fp8_inputs(cfg)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    hid = up(inp.hidden)
    wks, wvs = [up(w) for w in inp.wk_t], [up(w) for w in inp.wv_t]
    kc = [torch.empty((cfg.T, cfg.d), dtype=torch.uint8, device=dev) for _ in range(cfg.L)]
    vc = [torch.empty((cfg.T, cfg.d), dtype=torch.uint8, device=dev) for _ in range(cfg.L)]
    ks = [torch.empty((cfg.T,), dtype=torch.float32, device=dev) for _ in range(cfg.L)]
    vs = [torch.empty((cfg.T,), dtype=torch.float32, device=dev) for _ in range(cfg.L)]

    def step():
        hs2.hs2_kv_bridge_fp8(hid, wks, wvs, k_outs=kc, v_outs=vc, k_scales=ks, v_scales=vs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(args.steps)
    kernels = {}
    if not args.no_profile:
        hs2.profile_enable(True)
        timed(args.steps)
        for name, (tot, n) in hs2.profile_read().items():
            kernels[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
        hs2.profile_enable(False)
    roof = None
    if "bridge_fp8" in kernels:
        ach = cfg.flops / (kernels["bridge_fp8"]["avg_us"] / 1e6) / 1e12
        roof = {"bound": "mfma", "kernel": "bridge_fp8", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": stored_traffic(cfg.name, "bridge_fp8")}
    hbm_bytes = cfg.T * cfg.D * 2 + cfg.L * 2 * (cfg.d * cfg.D * 2 + cfg.T * (cfg.d + 4))
    out = {
        "metric": "multi-target FP8 KV bridge: tokens/s projected into every target's FP8 cache",
        "value": cfg.T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.D, "d": cfg.d, "targets": cfg.L,
                   "output": "fp8 e4m3fn + fp32 row scale"},
        "roofline": roof, "step_hbm_frac": hbm_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] cpu baseline (oracle)")
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < 10.0 and done < cfg.T:
            oracle.kv_bridge_fp8(inp.hidden[done:done + 4096], inp.wk_t, inp.wv_t)
            done += 4096
        el = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": done / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "sample": f"the first {done} tokens of {cfg.name} (all {cfg.L} targets), {el:.1f} s"}
    print(json.dumps(out), flush=True)


def gather_cold_sweep(reps=5):
    """Supplementary, labelled measurement of the sparse-layer kernel on decode-shaped gathers
    large enough to be bandwidth-dominated: B sequences x 1 query x S = 1152 selected rows (a
    random sorted set per query) out of a 1 GiB bf16 K+V cache, with the L2 and the memory-side
    cache flushed (a 512 MiB buffer written) before every repetition.  Median over reps."""
    import torch

    import token_level_sparse_mqa_amd as hs2
    dev = torch.device("cuda:0")
    H, d, S = 32, 128, 1152
    gen = torch.Generator(device=dev)
    gen.manual_seed(1152)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = []
    for B, N in ((16, 131072), (64, 32768), (256, 8192)):      # B * N * 512 B = 1 GiB of K+V
        k = torch.randn((B, N, d), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((B, N, d), generator=gen, device=dev).to(torch.bfloat16)
        q = torch.randn((B, 1, H, d), generator=gen, device=dev).to(torch.bfloat16)
        idx = torch.rand((B, N), generator=gen, device=dev).argsort(dim=1)[:, :S].sort(dim=1).values
        idx = idx.to(torch.int32).reshape(B, 1, S).contiguous()
        ws = hs2.sparse_attn_workspace(B, 1, H, d, S, dev)
        o = torch.empty((B, 1, H, d), dtype=torch.float32, device=dev)
        for _ in range(2):
            hs2.hs2_sparse_attn(q, k, v, idx, o=o, workspace=ws)
        times = []
        for r in range(reps):
            flush.fill_(r & 0xFF)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # a short GPU sleep ahead of the start event keeps the device busy while the host
            # enqueues the call, so the events bracket the kernels and not the host's launch latency
            torch.cuda._sleep(SLEEP_CYCLES)
            e0.record()
            hs2.hs2_sparse_attn(q, k, v, idx, o=o, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        us = sorted(times)[len(times) // 2]
        nbytes = B * (S * 2 * d * 2 + S * 4 + H * d * 2 + H * d * 4)
        out.append({"B": B, "cache_rows_per_seq": N, "S": S, "bytes": nbytes, "us": us,
                    "GB/s": nbytes / us / 1e3, "frac": nbytes / us / 1e3 / HBM_PEAK_GBS})
        del k, v, q, idx, ws, o
    del flush
    return {"label": "supplementary: sparse-layer kernel, cold cache, decode-shaped gathers from a "
                     "1 GiB bf16 K+V cache (not the timed step)", "points": out}


def host_info():
    """CPU model (from /proc/cpuinfo) and numpy's BLAS library (threadpoolctl)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info() if p.get("user_api") == "blas"]
        blas = ", ".join(libs) or None
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas}


def cpu_baseline(cfg, wl, budget_s=30.0, min_s=10.0, select="token"):
    """The float64 oracle, as it stands, on a bounded sample of the same workload: whole query
    rows, each with the full layer, the selection and every sparse layer, including decoding
    the cache bytes.  Small workloads are repeated until min_s of work; large ones stop after
    budget_s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    sm = 1.0 / math.sqrt(cfg.d)
    rows = [(b, i) for b in range(cfg.B) for i in range(cfg.Tq)]
    t0 = time.perf_counter()
    done, passes = 0, 0
    while True:
        decoded = {}
        passes += 1
        for (b, i) in rows:
            if b not in decoded:
                if cfg.bridge_D:
                    kb, vb = oracle.kv_bridge(wl.hidden, wl.wk, wl.wv)
                    decoded[b] = (oracle.decode(kb, "bf16"), oracle.decode(vb, "bf16"))
                else:
                    ks = wl.k_scale[b] if wl.k_scale is not None else None
                    vs = wl.v_scale[b] if wl.v_scale is not None else None
                    decoded[b] = (oracle.decode(wl.k[b], cfg.kv_dtype, ks), oracle.decode(wl.v[b], cfg.kv_dtype, vs))
            k, v = decoded[b]
            q = oracle.decode(wl.q_full[b, i], cfg.q_dtype)
            t = int(wl.q_pos[b, i])
            if select == "blocks":
                _, _, idx, _ = oracle.full_attn_select_blocks_row(q, k, v, t, sm, cfg.k_global // BLOCK, BLOCK,
                                                                  cfg.window)
            else:
                _, idx, _ = oracle.full_attn_select_row(q, k, v, t, sm, cfg.k_global, cfg.window)
            for l in range(cfg.n_sparse):
                oracle.sparse_attention_row(oracle.decode(wl.q_sparse[l][b, i], cfg.q_dtype), k, v, idx, sm)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        el = time.perf_counter() - t0
        if el > budget_s or el >= min_s:
            break
    return {"value": done / el, "unit": "query tokens/s", "cores": cores, "kind": "oracle", **host_info(),
            "sample": f"{done} query rows of {cfg.name} ({passes} pass(es) over its {len(rows)} rows; each "
                      f"row: full layer + {'block' if select == 'blocks' else 'token'}-level selection + {cfg.n_sparse} sparse layers, incl. decoding the "
                      f"cache), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode128k")
    ap.add_argument("--select", choices=("token", "blocks"), default="token",
                    help="token-level selection (the method) or the 64-token block-level variant")
    ap.add_argument("--decode-block", action="store_true",
                    help="decode workloads: run the hybrid block as one launch (hs2_decode_block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--no-gather-sweep", action="store_true",
                    help="skip the cold-cache gather sweep reported with the decode workloads")
    ap.add_argument("--fused-layers", action="store_true",
                    help="time the step with all sparse layers in one hs2_sparse_attn_layers call (their "
                         "queries given up front) instead of one call per layer")
    ap.add_argument("--no-supplements", action="store_true",
                    help="time only the step (no other layer mode, no cold-cache steps): profiling runs")
    ap.add_argument("--gather-sweep-only", action="store_true",
                    help="run only the cold-cache gather sweep and print it (profiling of the sparse kernel)")
    ap.add_argument("--no-1m", action="store_true",
                    help="decode128k: skip the nested decode1m_fp8 record")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration runs)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the hot path is measured on one GPU's share "
              f"(sharding is described in DESIGN.md); got --gpus {args.gpus}, WORLD_SIZE {world}",
              file=sys.stderr)
        sys.exit(2)

    if args.calib_copy_mib:
        import torch
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.gather_sweep_only:
        print(json.dumps({"gather_cold_sweep": gather_cold_sweep()}), flush=True)
        return
    from workloads import AGENTIC, BRIDGE_FP8, CONFIGS
    if args.workload in AGENTIC:
        agentic_main(AGENTIC[args.workload], args)
        return
    if args.workload in BRIDGE_FP8:
        bridge_fp8_main(BRIDGE_FP8[args.workload], args)
        return
    cfg = CONFIGS[args.workload]
    layers = "fused" if args.fused_layers else "sequential"
    res = run_gpu(cfg, args.steps, args.warmup, profile=not args.no_profile, select=args.select,
                  decode_block=args.decode_block, layers=layers, supplements=not args.no_supplements)
    out = workload_record(cfg, res, args)
    out = {"metric": METRIC, **out}
    if cfg.name == "decode128k" and not args.no_1m and not args.decode_block and args.select == "token":
        # the metric is quoted at 128K and 1M context: the 1M FP8 decode block in the same run
        res1m = run_gpu(CONFIGS["decode1m_fp8"], args.steps, args.warmup, profile=not args.no_profile,
                        layers=layers, supplements=not args.no_supplements)
        rec = workload_record(CONFIGS["decode1m_fp8"], res1m, args)
        out["decode1m_fp8"] = {k: rec[k] for k in ("value", "unit", "ms_per_step", "ms_per_step_mean",
                                                   "ms_per_step_fused_layers", "ms_per_step_sequential_layers",
                                                   "ms_per_step_cold", "dtype", "config", "roofline",
                                                   "full_select_frac", "step_roofline_frac", "kernels") if k in rec}
    if cfg.Tq == 1 and not args.no_gather_sweep and not args.no_profile:
        log("[bench] cold-cache gather sweep")
        out["gather_cold_sweep"] = gather_cold_sweep()
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(cfg, res["wl"], select=args.select)
    print(json.dumps(out), flush=True)


# kernels of the full layer with its selection (the step minus the sparse layers and the bridge)
FULL_SELECT_KERNELS = ("full_attn_mfma", "full_attn_combine", "full_attn_prefill", "full_attn_generic",
                       "score_rows_mfma", "score_prefill", "score_generic", "select_digit", "select_gather",
                       "select_finish", "select_block_max", "select_blocks")


def workload_record(cfg, res, args):
    """The bench fields of one workload's run: value, step times, roofline of the dominant kernel,
    the full layer's HBM fraction and per-kernel times."""
    ms = res["ms_per_step"]
    value = res["rows"] / (ms / 1e3)
    alg = algorithmic(cfg)
    kernels = {}
    for name, (tot, n) in res["kernels"].items():
        kernels[name] = {"avg_us": 1e3 * tot / max(n, 1), "launches": n}
    roof = None
    cand = [(v["avg_us"] * v["launches"], k) for k, v in kernels.items() if k in KERNEL_UNITS]
    if cand:
        _, kname = max(cand)
        unit, bound = KERNEL_UNITS[kname]
        avg_s = kernels[kname]["avg_us"] / 1e6
        traffic = stored_traffic(cfg.name, kname)
        if bound == "hbm":
            ach = alg[unit]["bytes"] / avg_s / 1e9          # every unit is per launch
            roof = {"bound": "hbm", "kernel": kname, "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ach / HBM_PEAK_GBS, "traffic": traffic}
        else:
            ach = alg[unit]["flops"] / avg_s / 1e12
            roof = {"bound": "mfma", "kernel": kname, "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS, "traffic": traffic}
        cnt = stored_counters(cfg.name, kname)
        if cnt is not None:
            roof["counters"] = cnt
    step_frac = {"hbm": alg["step"]["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "mfma": alg["step"]["flops"] / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS}
    out = {
        "value": value, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"f32": "f32", "bf16": "bf16"}[cfg.q_dtype] +
        ("+fp8kv" if cfg.kv_dtype == "fp8" else ""), "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "context": cfg.N, "Tq": cfg.Tq, "H": cfg.H, "d": cfg.d,
                   "kv_dtype": cfg.kv_dtype, "k_global": cfg.k_global, "window": cfg.window,
                   "sparse_layers": cfg.n_sparse, "bridge_D": cfg.bridge_D,
                   "selection": "token" if args.select == "token" else f"blocks of {BLOCK}",
                   "launch": "one launch (hs2_decode_block)" if args.decode_block else
                   ("one launch per kernel; the sparse layers one call each, in order" if res["layers"] == "sequential"
                    else "one launch per kernel; all sparse layers in one call")},
        "ms_per_step_mean": res["ms_mean"],
        "roofline": roof, "step_roofline_frac": step_frac, "kernels": kernels,
    }
    if "ms_other_layers" in res:
        other = "ms_per_step_fused_layers" if res["layers"] == "sequential" else "ms_per_step_sequential_layers"
        out[other] = res["ms_other_layers"]
        out["ms_per_step_" + res["layers"] + "_layers"] = ms
    if "ms_cold" in res:
        out["ms_per_step_cold"] = res["ms_cold"]
    # the full layer with its selection against its algorithmic bytes (K and V read once)
    fs = [kernels[k]["avg_us"] * kernels[k]["launches"] for k in FULL_SELECT_KERNELS if k in kernels]
    if fs and "full_attn_mfma" in kernels:
        per_step_s = sum(fs) / kernels["full_attn_mfma"]["launches"] / 1e6
        out["full_select_frac"] = {"hbm": alg["full_attn"]["bytes"] / per_step_s / 1e9 / HBM_PEAK_GBS,
                                   "us": per_step_s * 1e6, "kernels": [k for k in FULL_SELECT_KERNELS if k in kernels]}
    return out


if __name__ == "__main__":
    main()
