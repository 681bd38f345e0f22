"""Seeded inputs of the agentic multi-turn workload (no arithmetic of the method lives here).

The pages build the hybrid block around agentic inference: in every round a few decoded action
tokens are followed by a long observation to prefill, on top of a context that only gets longer
(agentik-os article, "How HySparse2 shrinks agent KV and prefill": section 1 "Agentic inference as
the driving workload", and the same article's "How it fits into an agentic stack": the agent's
single context grows by each observation in turn).  The pages give no lengths; the configs below pick a short action of a few dozen tokens and an
observation of one 4,096-token chunk, starting from a context that already holds a long trace.

One sequence (one agent trace).  Positions 0 .. N0-1 are the trace already in the cache; then
``turns`` rounds of ``act`` action tokens (decoded one at a time) followed by ``obs`` observation
tokens (one prefill chunk).  Every token has a self-decoder hidden state (the input of the KV
bridge, D wide); every new token has a full-layer query and one query per sparse layer.  The
hidden states and queries are independent draws: the model that would produce them is not part
of the hot path.

Recipe: the streams of ``workloads.gen`` (``rng_for(cfg_id, tensor_id)``), tensor ids
hidden = 20 ([N_final, D]), Wk = 21, Wv = 22 ([D, d], std 0.02), Q_full = 0 and
Q_sparse = 10 + l ([N_new, H, d] for the N_new = N_final - N0 new tokens in position order);
float64 draws rounded to fp32 then bf16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .gen import T_HIDDEN, T_QFULL, T_QSPARSE, T_WK, T_WV, _normal, f32_to_bf16_bits, rng_for


@dataclass(frozen=True)
class AgenticConfig:
    name: str
    cfg_id: int
    N0: int            # context already in the cache when the loop starts
    turns: int         # rounds of (action, observation)
    act: int           # action tokens per round, decoded one at a time
    obs: int           # observation tokens per round, prefilled as one chunk
    H: int = 32
    d: int = 128
    D: int = 2048      # self-decoder hidden width (KV-bridge input)
    n_sparse: int = 3
    k_global: int = 1024
    window: int = 128

    @property
    def S(self) -> int:
        return self.k_global + self.window

    @property
    def n_new(self) -> int:
        return self.turns * (self.act + self.obs)

    @property
    def N_final(self) -> int:
        return self.N0 + self.n_new

    def phases(self) -> List[Tuple[str, int, int]]:
        """(kind, first position, tokens) in order: kind "act" is one decoded token, "obs" one chunk."""
        out, p = [], self.N0
        for _ in range(self.turns):
            for _ in range(self.act):
                out.append(("act", p, 1))
                p += 1
            out.append(("obs", p, self.obs))
            p += self.obs
        return out


AGENTIC = {
    # 112K-token trace, four rounds of a 32-token action and a 4,096-token observation (to 131,200)
    "agentic": AgenticConfig("agentic", 6, N0=114688, turns=4, act=32, obs=4096),
}


@dataclass
class AgenticInputs:
    cfg: AgenticConfig
    hidden: np.ndarray            # [N_final, D] bf16 bits
    wk: np.ndarray                # [D, d] bf16 bits
    wv: np.ndarray
    q_full: np.ndarray            # [N_new, H, d] bf16 bits, new tokens in position order
    q_sparse: List[np.ndarray]    # n_sparse x [N_new, H, d]


def make_agentic(cfg: AgenticConfig) -> AgenticInputs:
    n, H, d, D = cfg.n_new, cfg.H, cfg.d, cfg.D
    hidden = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_HIDDEN), (cfg.N_final, D)))
    wk = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WK), (D, d), std=0.02))
    wv = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_WV), (D, d), std=0.02))
    q_full = f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_QFULL), (n, H, d)))
    q_sparse = [f32_to_bf16_bits(_normal(rng_for(cfg.cfg_id, T_QSPARSE + l), (n, H, d)))
                for l in range(cfg.n_sparse)]
    return AgenticInputs(cfg, hidden, wk, wv, q_full, q_sparse)
