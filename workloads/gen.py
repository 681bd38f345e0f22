"""Seeded input generation (no arithmetic of the method lives here).

Recipe, identical for every consumer:

* every tensor is drawn in float64 from
  ``Generator(PCG64(SeedSequence([cfg_id, tensor_id, layer_id])))``;
  tensor ids: Q_full=0, K=1, V=2, Q_sparse=10+l, hidden=20, Wk=21, Wv=22, needle draws=30;
  large tensors are drawn in row blocks from the one stream, in row-major order;
* fp32 tensors are the float64 draws rounded to binary32 (numpy, round to nearest even);
  bf16 tensors are those binary32 values rounded again to bfloat16 (torch, round to
  nearest even) and kept as uint16 bit patterns;
* FP8 caches: per cache row (one token's d-vector) the scale is ``max|x| / 448`` stored
  as fp32, the code is ``x / scale`` clamped to [-448, 448] and rounded to OCP E4M3FN
  by torch; codes are kept as uint8.  The decoded value of a row is ``code * scale``;
* planted needles overwrite a key row with four times one head of one query's full-layer
  query vector (the multiplication by four is exact in fp32 and bf16).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

from .configs import Config

T_QFULL, T_K, T_V, T_QSPARSE, T_HIDDEN, T_WK, T_WV, T_NEEDLE = 0, 1, 2, 10, 20, 21, 22, 30
FP8_MAX = 448.0
_BLOCK_ELEMS = 1 << 24


def rng_for(cfg_id: int, tensor_id: int, layer_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tensor_id, layer_id])))


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """float64 N(0, std^2) drawn in row blocks from one stream, returned as float32."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    pos = 0
    while pos < n:
        m = min(_BLOCK_ELEMS, n - pos)
        x = rng.standard_normal(m)
        if std != 1.0:
            x = x * std
        out[pos:pos + m] = x.astype(np.float32)
        pos += m
    return out.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float32).numpy()


def quantize_fp8_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row scale = amax/448 (fp32); codes = E4M3FN(x/scale) via torch.  x: [..., d] fp32."""
    amax = np.abs(x).max(axis=-1).astype(np.float32)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1, x.shape[-1])
    flat_s = scale.reshape(-1)
    flat_o = out.reshape(-1, x.shape[-1])
    rows_per = max(1, _BLOCK_ELEMS // x.shape[-1])
    for r0 in range(0, flat_x.shape[0], rows_per):
        r1 = min(flat_x.shape[0], r0 + rows_per)
        y = torch.from_numpy(flat_x[r0:r1] / flat_s[r0:r1, None]).clamp_(-FP8_MAX, FP8_MAX)
        flat_o[r0:r1] = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out, scale


def _store(x32: np.ndarray, dtype: str):
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _times4(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return (bits * np.float32(4.0)).astype(np.float32)
    return f32_to_bf16_bits(bf16_bits_to_f32(bits) * np.float32(4.0))


@dataclass
class Workload:
    cfg: Config
    q_full: np.ndarray                       # [B,Tq,H,d] f32 or bf16 bits
    q_sparse: List[np.ndarray]               # n_sparse x [B,Tq,H,d]
    k: Optional[np.ndarray]                  # [B,N,d] f32 / bf16 bits / fp8 codes (None: from bridge)
    v: Optional[np.ndarray]
    k_scale: Optional[np.ndarray] = None     # [B,N] fp32 (fp8 only)
    v_scale: Optional[np.ndarray] = None
    q_pos: np.ndarray = None                 # [B,Tq] int32
    kv_len: np.ndarray = None                # [B] int32
    hidden: Optional[np.ndarray] = None      # [N,D] bf16 bits (bridge configs)
    wk: Optional[np.ndarray] = None          # [D,d] bf16 bits
    wv: Optional[np.ndarray] = None
    needles: List[Tuple[int, int, int, int]] = field(default_factory=list)  # (b, t, h, p)


def _needle_plan(cfg: Config) -> List[Tuple[int, int, int, int]]:
    t0 = cfg.N - cfg.Tq
    plan = []
    if cfg.needles == "seeded8":
        # 8 needles: positions drawn without replacement from [0, t0 - W], heads drawn
        # uniformly; needle i belongs to the query at position t0 + 2i.
        assert cfg.Tq >= 16 and t0 - cfg.window >= 8
        rng = rng_for(cfg.cfg_id, T_NEEDLE)
        ps = rng.choice(t0 - cfg.window + 1, size=8, replace=False)
        hs = rng.integers(0, cfg.H, size=8)
        for i in range(8):
            plan.append((0, t0 + 2 * i, int(hs[i]), int(ps[i])))
    elif cfg.needles == "spread64":
        # 64 needles spread evenly over the cached prefix and over the query chunk.
        assert cfg.Tq % 64 == 0 and t0 % 64 == 0
        sp, sq = t0 // 64, cfg.Tq // 64
        for i in range(64):
            plan.append((0, t0 + sq * i + sq - 1, i % cfg.H, sp * i + sp // 2))
    for (_, t, _, p) in plan:
        assert p <= t - cfg.window, "a needle must be a global candidate of its query"
    return plan


def make_workload(cfg: Config) -> Workload:
    B, N, Tq, H, d = cfg.B, cfg.N, cfg.Tq, cfg.H, cfg.d
    q_full = _store(_normal(rng_for(cfg.cfg_id, T_QFULL), (B, Tq, H, d)), cfg.q_dtype)
    q_sparse = [_store(_normal(rng_for(cfg.cfg_id, T_QSPARSE + l), (B, Tq, H, d)), cfg.q_dtype)
                for l in range(cfg.n_sparse)]
    q_pos = np.tile(np.arange(N - Tq, N, dtype=np.int32), (B, 1))
    kv_len = np.full((B,), N, dtype=np.int32)
    wl = Workload(cfg, q_full, q_sparse, None, None, q_pos=q_pos, kv_len=kv_len)
    if cfg.bridge_D:
        assert B == 1
        D = cfg.bridge_D
        wl.hidden = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_HIDDEN), (N, D)))
        wl.wk = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WK), (D, d), std=0.02))
        wl.wv = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WV), (D, d), std=0.02))
        return wl
    k32 = _normal(rng_for(cfg.cfg_id, T_K), (B, N, d))
    v32 = _normal(rng_for(cfg.cfg_id, T_V), (B, N, d))
    if cfg.ident_keys:
        k32[:] = k32[:, :1, :]
    elif cfg.near_ties > 0:
        k32 = (k32[:, :1, :] + np.float32(cfg.near_ties) * k32).astype(np.float32)
    if cfg.kv_dtype == "fp8":
        wl.k, wl.k_scale = quantize_fp8_rows(k32)
        wl.v, wl.v_scale = quantize_fp8_rows(v32)
    else:
        wl.k = _store(k32, cfg.kv_dtype)
        wl.v = _store(v32, cfg.kv_dtype)
    plan = _needle_plan(cfg)
    if plan:
        assert cfg.kv_dtype in ("f32", "bf16") and cfg.q_dtype == cfg.kv_dtype
    t0 = N - Tq
    for (b, t, h, p) in plan:
        wl.k[b, p, :] = _times4(q_full[b, t - t0, h, :], cfg.kv_dtype)
    wl.needles = plan
    return wl
