"""The five synthetic workloads of the hot path, plus a builder for small ones.

Shapes follow the hybrid-block description on the pages: 1,024 token-level
global picks plus a forced window of the 128 most recent tokens (kucoin news
flash, body paragraph; lynxflow blog, "Token-Level Sparse Selection"), one
shared KV head (MQA; ainews page, experimental-setup paragraph), FP8 caches
(same paragraph), and the million-token context of the pages' cost analysis.

Every query token is one of the last ``Tq`` positions of its sequence:
position ``t = N - Tq + i``, and the cache holds ``N`` rows including the
query's own row.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int            # seed namespace
    B: int                 # sequences
    N: int                 # cache rows per sequence (Nmax == kv_len)
    Tq: int                # query tokens per sequence (the last Tq positions)
    H: int                 # query heads (one shared KV head)
    d: int                 # head dim
    q_dtype: str           # "f32" | "bf16"
    kv_dtype: str          # "f32" | "bf16" | "fp8"
    n_sparse: int          # index-reusing sparse layers after the full layer
    k_global: int = 1024
    window: int = 128
    needles: str = "none"  # "none" | "seeded8" | "spread64"
    bridge_D: int = 0      # >0: K/V come from a KV-Bridge projection of hidden states [N, D]
    ident_keys: bool = False  # every K row equal (tie / closed-form edge case)
    near_ties: float = 0.0    # >0: every K row = one shared row + near_ties * its own N(0, 1) row

    @property
    def S(self) -> int:
        return self.k_global + self.window

    @property
    def rows(self) -> int:
        return self.B * self.Tq

    def q_positions(self):
        return [self.N - self.Tq + i for i in range(self.Tq)]


CONFIGS = {
    # 1 sequence, 4096 keys, last 16 positions, H16 d64, fp32, 8 needles, 2 sparse layers
    "tiny": Config("tiny", 1, B=1, N=4096, Tq=16, H=16, d=64, q_dtype="f32", kv_dtype="f32",
                   n_sparse=2, needles="seeded8"),
    # batch-8 decode at 128K context, H32 d128 bf16, 3 sparse layers
    "decode128k": Config("decode128k", 2, B=8, N=131072, Tq=1, H=32, d=128, q_dtype="bf16",
                         kv_dtype="bf16", n_sparse=3),
    # 65536 cached + 4096-token causal chunk, 64 needles spread uniformly, 3 sparse layers
    "prefill_chunk": Config("prefill_chunk", 3, B=1, N=69632, Tq=4096, H=32, d=128,
                            q_dtype="bf16", kv_dtype="bf16", n_sparse=3, needles="spread64"),
    # 1M-token decode with FP8 E4M3 KV + per-row fp32 scale, bf16 Q, 3 sparse layers
    "decode1m_fp8": Config("decode1m_fp8", 4, B=1, N=1048576, Tq=1, H=32, d=128,
                           q_dtype="bf16", kv_dtype="fp8", n_sparse=3),
    # KV-Bridge of hidden states [262144 x 2048] then a 4096-token chunk, 3 sparse layers
    "prefill_exit256k": Config("prefill_exit256k", 5, B=1, N=262144, Tq=4096, H=32, d=128,
                               q_dtype="bf16", kv_dtype="bf16", n_sparse=3, bridge_D=2048),
}

ORDER = ["tiny", "decode128k", "prefill_chunk", "decode1m_fp8", "prefill_exit256k"]


def get_config(name: str) -> Config:
    return CONFIGS[name]


def small_config(name: str, cfg_id: int, *, B: int, N: int, Tq: int, H: int = 32, d: int = 128,
                 q_dtype: str = "bf16", kv_dtype: str = "bf16", n_sparse: int = 1,
                 k_global: int = 1024, window: int = 128, needles: str = "none",
                 bridge_D: int = 0, ident_keys: bool = False, near_ties: float = 0.0,
                 base: Optional[Config] = None) -> Config:
    """A reduced workload for parity tests (sizes the oracle finishes in seconds)."""
    if base is not None:
        return replace(base, name=name, cfg_id=cfg_id, B=B, N=N, Tq=Tq)
    return Config(name, cfg_id, B=B, N=N, Tq=Tq, H=H, d=d, q_dtype=q_dtype, kv_dtype=kv_dtype,
                  n_sparse=n_sparse, k_global=k_global, window=window, needles=needles,
                  bridge_D=bridge_D, ident_keys=ident_keys, near_ties=near_ties)
