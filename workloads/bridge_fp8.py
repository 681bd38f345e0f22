"""Seeded inputs of the multi-target FP8 bridge (no arithmetic of the method lives here).

Every cross-decoder full-attention layer projects the self-decoder's hidden states with its own
Wk, Wv (lynxflow blog, "Two-Level KV Sharing").  The pages' model has 49 layers of which the first
25 form the self-decoder (kucoin news flash); with hybrid blocks of one full layer and three sparse
layers the 24 cross-decoder layers hold 6 full layers, hence 6 targets.  Weights are kept in a
linear layer's layout, [d, D] per projection.

Recipe (the streams of ``workloads.gen``): hidden [T, D] from tensor id 20; target l's Wk from
(21, layer l) and Wv from (22, layer l), N(0, 0.02^2); float64 draws rounded to fp32 then bf16.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

from .gen import T_HIDDEN, T_WK, T_WV, _normal, f32_to_bf16_bits, rng_for


@dataclass(frozen=True)
class BridgeFp8Config:
    name: str
    cfg_id: int
    T: int          # hidden-state rows (tokens)
    D: int          # hidden width
    d: int          # head dim of the K/V caches
    L: int          # target layers

    @property
    def flops(self) -> float:
        return 2.0 * self.T * self.D * self.L * 2 * self.d


BRIDGE_FP8 = {
    # the 262,144-token prefill exit of the bridge workload, into 6 targets' FP8 caches
    "bridge_fp8_256k": BridgeFp8Config("bridge_fp8_256k", 7, T=262144, D=2048, d=128, L=6),
}


@dataclass
class BridgeFp8Inputs:
    cfg: BridgeFp8Config
    hidden: np.ndarray          # [T, D] bf16 bits
    wk_t: List[np.ndarray]      # L x [d, D] bf16 bits
    wv_t: List[np.ndarray]


def make_bridge_fp8_inputs(cfg: BridgeFp8Config) -> BridgeFp8Inputs:
    hidden = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_HIDDEN), (cfg.T, cfg.D)))
    wk = [f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WK, l), (cfg.d, cfg.D), std=0.02)) for l in range(cfg.L)]
    wv = [f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WV, l), (cfg.d, cfg.D), std=0.02)) for l in range(cfg.L)]
    return BridgeFp8Inputs(cfg, hidden, wk, wv)
