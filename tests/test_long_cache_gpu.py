"""Query chunks over caches longer than 2^31 bytes per sequence, against closed forms.

Eight query tokens over MARK + 4096 keys of d = 128, where MARK is the first row whose byte
offset in K or V reaches 2^31 (2^23 rows of bf16, 2^24 rows of FP8 codes; 2.15 GB per tensor):
past the range the chunk kernels address with 32-bit offsets, so the call runs on the row
kernels.  Every key is zero, so each head's softmax is uniform over [0, t] (the pinned special
case of identical keys: p = 1/(t+1), O = the mean of the V rows, every candidate's score
H/(t+1), and the picks are the k lowest candidates by the tie rule).  V is zero except in the
rows at or past MARK, where row j holds 2^18 in column j mod 128 (FP8, twice as many rows: 2^19
as code 448 with row scale 2^19/448); a row read from a wrapped offset would bring zeros, so O
would fall towards 0.

Expected values, in float64 on the host (val = the decoded planted value):
  O_full[i, h, c]   = val * #{j in [MARK, t_i] : j mod 128 = c} / (t_i + 1)
  idx[i]            = 0..1023, then t_i-127..t_i
  O_sparse[i, h, c] = val * #{j in window(t_i) : j mod 128 = c} / 1152
                    (the 1024 picks are zero rows; the window's 128 consecutive rows, all past
                    MARK, hold every residue once)
The weights are exactly 1 and the sums of the P.V products stay exact in fp32, so the outputs
sit far inside the tolerances (2e-3 bf16, 2e-2 FP8).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests.hs2_harness import _say

pytestmark = pytest.mark.gpu

TQ, H, D, KG, W = 8, 32, 128, 1024, 128
E4M3_448 = 0x7E                      # OCP E4M3FN: exponent field 15, mantissa 6 -> 1.75 * 2^8


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_long_cache_chunk_closed_form(kv):
    import token_level_sparse_mqa_amd as hs2
    mark = (1 << 31) // (D * (2 if kv == "bf16" else 1))
    N = mark + 4096
    tol = 2e-3 if kv == "bf16" else 2e-2
    plant = float(1 << 18) if kv == "bf16" else float(1 << 19)     # O near 1 either way
    _say(f"[long_cache] {kv} B=1 Tq={TQ} N={N} d={D}")
    dev = torch.device("cuda")
    rows = torch.arange(mark, N, device=dev)
    ks = vs = None
    if kv == "bf16":
        k = torch.zeros((1, N, D), dtype=torch.bfloat16, device=dev)
        v = torch.zeros((1, N, D), dtype=torch.bfloat16, device=dev)
        v[0, rows, rows % D] = plant
        val = plant
    else:
        k = torch.zeros((1, N, D), dtype=torch.uint8, device=dev)
        v = torch.zeros((1, N, D), dtype=torch.uint8, device=dev)
        v[0, rows, rows % D] = E4M3_448
        ks = torch.ones((1, N), dtype=torch.float32, device=dev)
        vs = torch.ones((1, N), dtype=torch.float32, device=dev)
        scale = np.float32(plant / 448.0)
        vs[0, mark:] = float(scale)
        val = 448.0 * float(scale)
    gen = torch.Generator().manual_seed(5)
    q = torch.randn((1, TQ, H, D), generator=gen).to(torch.bfloat16).to(dev)
    qs = torch.randn((1, TQ, H, D), generator=gen).to(torch.bfloat16).to(dev)
    q_pos = torch.arange(N - TQ, N, dtype=torch.int32, device=dev).reshape(1, TQ)
    kv_len = torch.tensor([N], dtype=torch.int32, device=dev)
    o, idx = hs2.hs2_full_attn_select(q, k, v, q_pos, kv_len, k_scale=ks, v_scale=vs, k_global=KG, window=W)
    sws = hs2.sparse_attn_layers_workspace(1, TQ, H, D, KG + W, 1, dev)
    (osp,) = hs2.hs2_sparse_attn_layers([qs], k, v, idx, kv_len=kv_len, k_scale=ks, v_scale=vs, workspace=sws)
    torch.cuda.synchronize()
    o, idx, osp = o.cpu().numpy(), idx.cpu().numpy(), osp.cpu().numpy()
    for i in range(TQ):
        t = N - TQ + i
        cnt = np.bincount(np.arange(mark, t + 1) % D, minlength=D).astype(np.float64)
        want = val * cnt / (t + 1)
        assert want.min() > 0.9, "the planted rows must carry a visible weight"
        err = np.max(np.abs(o[0, i] - want[None, :]))
        assert err <= tol, f"row {i}: full-layer O off by {err}"
        exp_idx = np.concatenate([np.arange(KG), np.arange(t - W + 1, t + 1)]).astype(np.int32)
        assert np.array_equal(idx[0, i], exp_idx), f"row {i}: indices differ"
        win = np.arange(t - W + 1, t + 1)
        assert win.min() >= mark
        want_sp = val * np.bincount(win % D, minlength=D) / (KG + W)
        err = np.max(np.abs(osp[0, i] - want_sp[None, :]))
        assert err <= tol, f"row {i}: sparse O off by {err}"
