"""CPU: the Python binding checks the shape, dtype and device of every caller-supplied tensor
against the call's sizes before it reaches the C ABI (which sees only pointers).  The library
is replaced by a stub that fails the test if any call gets through."""
import pytest
import torch

import token_level_sparse_mqa_amd as hs2

B, TQ, H, D, N, KG, W = 2, 3, 4, 64, 500, 16, 4


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def _stub():
        raise AssertionError("the C ABI was reached with invalid tensors")
    monkeypatch.setattr(hs2, "lib", _stub)


def _full(**over):
    a = dict(q=torch.zeros(B, TQ, H, D, dtype=torch.bfloat16), k=torch.zeros(B, N, D, dtype=torch.bfloat16),
             v=torch.zeros(B, N, D, dtype=torch.bfloat16), q_pos=torch.zeros(B, TQ, dtype=torch.int32),
             kv_len=torch.zeros(B, dtype=torch.int32), k_global=KG, window=W,
             o=torch.zeros(B, TQ, H, D), idx=torch.zeros(B, TQ, KG + W, dtype=torch.int32),
             workspace=torch.zeros(16, dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("over", [
    dict(o=torch.zeros(B, TQ, H, D - 1)),                                  # undersized o
    dict(o=torch.zeros(B, TQ, H, D, dtype=torch.float16)),                 # wrong o dtype
    dict(idx=torch.zeros(B, TQ, KG + W - 1, dtype=torch.int32)),           # idx shorter than k + W
    dict(idx=torch.zeros(B, TQ, KG + W, dtype=torch.int64)),
    dict(scores_dbg=torch.zeros(B, TQ, N - 1)),                            # scores_dbg [B, Tq, Nmax]
    dict(v=torch.zeros(B, N - 1, D, dtype=torch.bfloat16)),                # v shorter than k
    dict(v=torch.zeros(B, N, D, dtype=torch.float32)),                     # v dtype differs from k
    dict(k=torch.zeros(B, N, D // 2, dtype=torch.bfloat16)),               # k row width differs from q
    dict(q_pos=torch.zeros(B, TQ + 1, dtype=torch.int32)),
    dict(q_pos=torch.zeros(B, TQ, dtype=torch.int64)),
    dict(kv_len=torch.zeros(B + 1, dtype=torch.int32)),
    dict(k_scale=torch.zeros(B, N - 1)),
    dict(q=torch.zeros(B, TQ, H, D)[..., :D].to(torch.float64)),           # q dtype
    dict(o=torch.zeros(B, TQ, H, D, device="meta")),                       # another device
])
def test_full_attn_select_rejects_tensors(over):
    with pytest.raises(ValueError):
        hs2.hs2_full_attn_select(**_full(**over))


@pytest.mark.parametrize("over", [
    dict(block_idx=torch.zeros(B, TQ, 1, dtype=torch.int32)),              # fewer than k_blocks
    dict(idx=torch.zeros(B, TQ, 2 * 8 + W - 1, dtype=torch.int32)),
    dict(o=torch.zeros(B, TQ, H, D + 1)),
])
def test_blocks_rejects_tensors(over):
    a = _full(idx=torch.zeros(B, TQ, 2 * 8 + W, dtype=torch.int32))
    a.pop("k_global")
    a.update(k_blocks=2, block=8, block_idx=torch.zeros(B, TQ, 2, dtype=torch.int32))
    a.update(over)
    with pytest.raises(ValueError):
        hs2.hs2_full_attn_select_blocks(**a)


def _sparse(**over):
    a = dict(q=torch.zeros(B, TQ, H, D, dtype=torch.bfloat16), k=torch.zeros(B, N, D, dtype=torch.bfloat16),
             v=torch.zeros(B, N, D, dtype=torch.bfloat16), idx=torch.zeros(B, TQ, KG + W, dtype=torch.int32),
             o=torch.zeros(B, TQ, H, D))
    a.update(over)
    return a


@pytest.mark.parametrize("over", [
    dict(o=torch.zeros(B, TQ, H, D // 2)),
    dict(idx=torch.zeros(B, TQ + 1, KG + W, dtype=torch.int32)),           # idx rows != query rows
    dict(idx=torch.zeros(B, TQ, KG + W, dtype=torch.int16)),
    dict(v=torch.zeros(B, N - 7, D, dtype=torch.bfloat16)),
    dict(kv_len=torch.zeros(B, 1, dtype=torch.int32)),
    dict(k=torch.zeros(B + 1, N, D, dtype=torch.bfloat16), v=torch.zeros(B + 1, N, D, dtype=torch.bfloat16)),
])
def test_sparse_rejects_tensors(over):
    with pytest.raises(ValueError):
        hs2.hs2_sparse_attn(**_sparse(**over))


def test_sparse_layers_rejects_tensors():
    a = _sparse()
    qs = [a["q"], a["q"].clone()]
    with pytest.raises(ValueError):     # one output short
        hs2.hs2_sparse_attn_layers(qs, a["k"], a["v"], a["idx"], os=[a["o"]])
    with pytest.raises(ValueError):     # an undersized output
        hs2.hs2_sparse_attn_layers(qs, a["k"], a["v"], a["idx"], os=[a["o"], torch.zeros(B, TQ, H, D - 1)])
    with pytest.raises(ValueError):     # idx of another batch size
        hs2.hs2_sparse_attn_layers(qs, a["k"], a["v"], torch.zeros(B + 1, TQ, 8, dtype=torch.int32))


def test_decode_block_rejects_tensors():
    a = _full()
    qs = [a["q"].clone()]
    base = dict(k_global=KG, window=W, o=a["o"], idx=a["idx"], workspace=a["workspace"])
    with pytest.raises(ValueError):
        hs2.hs2_decode_block(a["q"], qs, a["k"], a["v"], a["q_pos"], a["kv_len"],
                             os=[torch.zeros(B, TQ, H, D - 1)], **base)
    with pytest.raises(ValueError):
        hs2.hs2_decode_block(a["q"], qs, a["k"], a["v"], a["q_pos"], a["kv_len"], os=[a["o"].clone()],
                             **dict(base, idx=torch.zeros(B, TQ, KG, dtype=torch.int32)))
