"""One agent trace over a growing KV cache: the multi-turn loop of the hybrid block.

The pages' agentic loop alternates a short decoded action with a long observation that is
prefilled, and the context only grows (agentik-os article, "How HySparse2 shrinks agent KV and
prefill": section 1 "Agentic inference as the driving workload" and its "How it fits into an agentic
stack": observations are appended to one long context buffer, and
the cross-decoder K/V come from the self-decoder through the KV bridge).  A session holds one
sequence's bf16 K/V cache at a fixed capacity and appends spans of tokens to it.  Appending T
tokens at positions p .. p+T-1 is three calls of the C ABI, in stream order:

  1. hs2_kv_bridge writes K/V rows p .. p+T-1 from the span's hidden states, in place;
  2. hs2_full_attn_select attends the span's queries (causal, kv_len = p+T) and selects;
  3. hs2_sparse_attn_layers runs every sparse layer on those indices.

A decoded action token is a span of one; an observation is one span (a prefill chunk).  Rows at
and past the current length are never read.  Positions and lengths are views of one device table,
and every buffer is allocated up front or grown on first use, so a warm session launches kernels
only.  Single sequence (B = 1); every call is ordered on the given stream.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import torch

from . import (hs2_full_attn_select, hs2_full_attn_select_workspace_size, hs2_kv_bridge,
               hs2_sparse_attn_layers, hs2_sparse_attn_layers_workspace_size, HS2_BF16)


class AgenticSession:
    def __init__(self, w_k: torch.Tensor, w_v: torch.Tensor, capacity: int, H: int, n_sparse: int,
                 max_span: int, k_global: int = 1024, window: int = 128, sm_scale: Optional[float] = None,
                 device=None, fill: Optional[float] = None):
        """w_k, w_v: [D, d] bf16 bridge projections of the cross-decoder full layer.
        capacity: cache rows; max_span: the longest span appended in one call.
        fill: optional value written to every cache row first (a test can plant NaN there to check
        that rows past the length are never read)."""
        D, d = w_k.shape
        dev = w_k.device if device is None else torch.device(device)
        self.w_k, self.w_v = w_k, w_v
        self.D, self.d, self.H, self.L = D, d, H, n_sparse
        self.capacity, self.max_span = capacity, max_span
        self.k_global, self.window, self.S = k_global, window, k_global + window
        self.sm = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
        self.k = torch.empty((1, capacity, d), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty((1, capacity, d), dtype=torch.bfloat16, device=dev)
        if fill is not None:
            self.k.fill_(fill)
            self.v.fill_(fill)
        # pos[i] = i: a span's query positions are pos[p : p+T], its kv_len is pos[p+T]
        self.pos = torch.arange(capacity + 1, dtype=torch.int32, device=dev)
        self.o = torch.empty((1, max_span, H, d), dtype=torch.float32, device=dev)
        self.idx = torch.empty((1, max_span, self.S), dtype=torch.int32, device=dev)
        self.o_sp = [torch.empty((1, max_span, H, d), dtype=torch.float32, device=dev) for _ in range(n_sparse)]
        self._ws_full = torch.empty((0,), dtype=torch.uint8, device=dev)
        self._ws_sparse = torch.empty((0,), dtype=torch.uint8, device=dev)
        self.length = 0

    def _workspace(self, T: int) -> Tuple[torch.Tensor, torch.Tensor]:
        nf = hs2_full_attn_select_workspace_size(1, T, self.H, self.d, self.capacity, self.k_global,
                                                 self.window, HS2_BF16)
        ns = hs2_sparse_attn_layers_workspace_size(1, T, self.H, self.d, self.S, self.L)
        if nf > self._ws_full.numel():
            self._ws_full = torch.empty((nf,), dtype=torch.uint8, device=self.k.device)
        if ns > self._ws_sparse.numel():
            self._ws_sparse = torch.empty((ns,), dtype=torch.uint8, device=self.k.device)
        return self._ws_full, self._ws_sparse

    def bridge_prefix(self, hidden: torch.Tensor, stream=None):
        """K/V rows 0 .. n-1 of a trace already in context (no queries): hidden [n, D] bf16."""
        n = hidden.shape[0]
        if self.length != 0 or n > self.capacity:
            raise ValueError("bridge_prefix starts an empty session and must fit the capacity")
        if n:
            hs2_kv_bridge(hidden, self.w_k, self.w_v, k_out=self.k[0, :n], v_out=self.v[0, :n], stream=stream)
        self.length = n

    def reset(self, length: int):
        """Rewind to a shorter length (rows past it are overwritten by later appends)."""
        if not 0 <= length <= self.length:
            raise ValueError("reset only rewinds")
        self.length = length

    def append(self, hidden: torch.Tensor, q: torch.Tensor, q_sparse: Sequence[torch.Tensor], stream=None
               ) -> Tuple[torch.Tensor, torch.Tensor, List[torch.Tensor]]:
        """Append T tokens and attend them.  hidden [T, D] bf16; q and each of q_sparse [T, H, d]
        bf16 (the full layer's and the sparse layers' queries of the span).  Returns views
        (o [1,T,H,d] fp32, idx [1,T,k+W] int32, [o of each sparse layer]) that the next call
        overwrites."""
        T = hidden.shape[0]
        p = self.length
        if T < 1 or T > self.max_span or p + T > self.capacity:
            raise ValueError(f"span of {T} tokens at {p}: max_span {self.max_span}, capacity {self.capacity}")
        if len(q_sparse) != self.L:
            raise ValueError(f"expected {self.L} sparse-layer queries")
        hs2_kv_bridge(hidden, self.w_k, self.w_v, k_out=self.k[0, p:p + T], v_out=self.v[0, p:p + T],
                      stream=stream)
        ws_full, ws_sparse = self._workspace(T)
        q_pos = self.pos[p:p + T].view(1, T)
        kv_len = self.pos[p + T:p + T + 1]
        o, idx = self.o[:, :T], self.idx[:, :T]
        hs2_full_attn_select(q.view(1, T, self.H, self.d), self.k, self.v, q_pos, kv_len,
                             k_global=self.k_global, window=self.window, sm_scale=self.sm, o=o, idx=idx,
                             workspace=ws_full, stream=stream)
        o_sp = [x[:, :T] for x in self.o_sp]
        if self.L:
            hs2_sparse_attn_layers([x.view(1, T, self.H, self.d) for x in q_sparse], self.k, self.v, idx,
                                   kv_len=kv_len, sm_scale=self.sm, os=o_sp, workspace=ws_sparse, stream=stream)
        self.length = p + T
        return o, idx, o_sp
