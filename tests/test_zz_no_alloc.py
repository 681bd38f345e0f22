"""GPU: hs2_full_attn_select_noalloc (static per-GPU scratch, no allocation) against
hs2_full_attn_select with its own workspace, through the C ABI, on consecutive calls of
decreasing size that reuse the same scratch: indices bit-identical, o identical (same kernels)."""
import pytest
import torch

from tests.hs2_harness import HipRun, _say
from workloads import make_workload, small_config

pytestmark = pytest.mark.gpu

CASES = [
    # decode rows of several sequences (row kernels with key splits), then a smaller call
    small_config("noalloc_big", 240, B=6, N=70000, Tq=2, n_sparse=0),
    small_config("noalloc_small", 241, B=2, N=5000, Tq=1, n_sparse=0),
    # a query chunk (chunk kernels) and an FP8 cache after them, smaller again
    small_config("noalloc_chunk", 242, B=1, N=3000, Tq=24, n_sparse=0),
    small_config("noalloc_fp8", 243, B=1, N=2200, Tq=1, kv_dtype="fp8", n_sparse=0),
]


def test_noalloc_matches_workspace_call():
    import token_level_sparse_mqa_amd as hs2
    for cfg in CASES:
        _say(f"[noalloc] {cfg.name} B={cfg.B} N={cfg.N} Tq={cfg.Tq} kv={cfg.kv_dtype}")
        g = HipRun(make_workload(cfg))
        ref_o, ref_idx, _ = g.full()
        o = torch.full_like(ref_o, float("nan"))
        idx = torch.full_like(ref_idx, -7)
        hs2.hs2_full_attn_select_noalloc(g.q, g.k, g.v, g.q_pos, g.kv_len, o=o, idx=idx, k_scale=g.k_scale,
                                         v_scale=g.v_scale, k_global=cfg.k_global, window=cfg.window,
                                         sm_scale=g.sm)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"{cfg.name}: indices differ"
        assert torch.equal(o, ref_o), f"{cfg.name}: o differs (max {float((o - ref_o).abs().max()):.3e})"
