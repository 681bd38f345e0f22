"""Python binding of libhs2 (HySparse2 hybrid-block attention hot path, MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of libhs2.so,
called through its C ABI (include/hs2.h) with ctypes.  torch provides device memory and
the current stream.  The functions carry the C names:

    hs2_kv_bridge, hs2_kv_bridge_fp8, hs2_full_attn_select, hs2_full_attn_select_workspace_size,
    hs2_full_attn_select_noalloc,
    hs2_full_attn_select_blocks, hs2_full_attn_select_blocks_workspace_size,
    hs2_sparse_attn, hs2_sparse_attn_workspace_size, hs2_sparse_attn_layers,
    hs2_sparse_attn_layers_workspace_size, hs2_decode_block, hs2_decode_block_workspace_size,
    hs2_last_error, hs2_version

There is no fallback: if the built library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

HS2_F32, HS2_BF16, HS2_FP8_E4M3 = 0, 1, 2
HS2_OK, HS2_ERR_INVALID_ARG, HS2_ERR_UNSUPPORTED, HS2_ERR_WORKSPACE, HS2_ERR_HIP = 0, -1, -2, -3, -4
HS2_MAX_SELECT_NMAX = 65535 * 4096      # cache rows per sequence of the calls that select (hs2.h)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libhs2.so")
_LIB: Optional[ctypes.CDLL] = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "hs2_kv_bridge": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _i64, _vp]),
    "hs2_kv_bridge_fp8": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp]),
    "hs2_full_attn_select_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i64, _i32, _i32, ctypes.c_int]),
    "hs2_full_attn_select": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                            _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32,
                                            _vp, _vp, _vp, _vp, _sz, _vp]),
    "hs2_full_attn_select_noalloc": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                                    _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32,
                                                    _vp, _vp, _vp, _vp]),
    "hs2_full_attn_select_blocks_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                                         ctypes.c_int]),
    "hs2_full_attn_select_blocks": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                                   _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _f32,
                                                   _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "hs2_sparse_attn": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32, _vp,
                                       _i32, _i32, _i32, _i32, _i64, _f32, _vp, _vp, _sz, _vp]),
    "hs2_sparse_attn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "hs2_sparse_attn_layers": (ctypes.c_int, [_vp, _i32, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp,
                                              _i32, _vp, _i32, _i32, _i32, _i32, _i64, _f32, _vp, _vp, _sz,
                                              _vp]),
    "hs2_sparse_attn_layers_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "hs2_decode_block_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i64, _i32, _i32, ctypes.c_int, _i32]),
    "hs2_decode_block": (ctypes.c_int, [_vp, _vp, _i32, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                        _i32, _i32, _i32, _i32, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz,
                                        _vp]),
    "hs2_last_error": (ctypes.c_char_p, []),
    "hs2_version": (ctypes.c_char_p, []),
    "hs2_profile_enable": (None, [ctypes.c_int]),
    "hs2_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
}


class HS2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hs2 status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libhs2.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m token_level_sparse_mqa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def hs2_last_error() -> str:
    return lib().hs2_last_error().decode()


def hs2_version() -> str:
    return lib().hs2_version().decode()


def _check(status: int):
    if status != HS2_OK:
        raise HS2Error(status, hs2_last_error())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HS2_F32
    if t.dtype == torch.bfloat16:
        return HS2_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return HS2_FP8_E4M3
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to hs2 must be contiguous")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], name: str, shape, dtypes, device, optional: bool = False):
    """The C ABI sees only pointers, so buffer sizes are checked here: shape, dtype and device of a
    caller-supplied tensor must be what the call reads or writes."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


_KV_DTYPES = (torch.float32, torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


def _check_select_inputs(q, k, v, q_pos, kv_len, k_scale, v_scale):
    """Shapes shared by the calls of the full layer: q [B,Tq,H,d], k/v [B,Nmax,d], q_pos [B,Tq],
    kv_len [B], scales [B,Nmax] (FP8 caches only)."""
    if q.dim() != 4 or k.dim() != 3:
        raise ValueError("q must be [B, Tq, H, d] and k, v [B, Nmax, d]")
    B, Tq, H, d = q.shape
    dev = q.device
    _expect(q, "q", (B, Tq, H, d), (torch.float32, torch.bfloat16), dev)
    _expect(k, "k", (B, k.shape[1], d), _KV_DTYPES, dev)
    _expect(v, "v", tuple(k.shape), (k.dtype,), dev)
    _expect(q_pos, "q_pos", (B, Tq), (torch.int32,), dev)
    _expect(kv_len, "kv_len", (B,), (torch.int32,), dev)
    _expect(k_scale, "k_scale", (B, k.shape[1]), (torch.float32,), dev, optional=True)
    _expect(v_scale, "v_scale", (B, k.shape[1]), (torch.float32,), dev, optional=True)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def hs2_kv_bridge(hidden: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor,
                  k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                  out_row_stride: Optional[int] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """K = bf16(hidden @ w_k), V = bf16(hidden @ w_v).  hidden [T, D] bf16; w_k, w_v [D, d] bf16."""
    T, D = hidden.shape
    d = w_k.shape[1]
    if k_out is None:
        k_out = torch.empty((T, d), dtype=torch.bfloat16, device=hidden.device)
    if v_out is None:
        v_out = torch.empty((T, d), dtype=torch.bfloat16, device=hidden.device)
    stride = d if out_row_stride is None else out_row_stride
    for t in (k_out, v_out):   # rows may sit inside a wider cache: check the row stride instead
        if t.dim() != 2 or t.shape != (T, d) or t.stride(1) != 1 or (T > 1 and t.stride(0) != stride):
            raise ValueError("k_out/v_out must be [T, d] views with unit column stride and row stride "
                             "out_row_stride")
    _check(lib().hs2_kv_bridge(_ptr(hidden), T, D, _ptr(w_k), _ptr(w_v), d, k_out.data_ptr(),
                               v_out.data_ptr(), stride, _stream(stream)))
    return k_out, v_out


def _ptr_array(ts):
    return ctypes.cast((ctypes.c_void_p * len(ts))(*[_ptr(t) for t in ts]), ctypes.c_void_p)


def hs2_kv_bridge_fp8(hidden: torch.Tensor, w_ks, w_vs, k_outs=None, v_outs=None, k_scales=None, v_scales=None,
                      out_row_stride: Optional[int] = None, stream=None):
    """Multi-target bridge into FP8 caches.  hidden [T, D] bf16; w_ks, w_vs: one [d, D] bf16 weight
    (linear layout) per target.  Returns (k_codes, k_scales, v_codes, v_scales), lists of u8 [T, d]
    and fp32 [T] tensors (or the given ones, which may be row views of wider caches)."""
    T, D = hidden.shape
    L = len(w_ks)
    d = w_ks[0].shape[0]
    dev = hidden.device
    if len(w_vs) != L:
        raise ValueError("one w_v per w_k")
    for w in list(w_ks) + list(w_vs):
        if w.shape != (d, D) or w.dtype != torch.bfloat16:
            raise ValueError("weights must be bf16 [d, D]")
    if k_outs is None:
        k_outs = [torch.empty((T, d), dtype=torch.uint8, device=dev) for _ in range(L)]
    if v_outs is None:
        v_outs = [torch.empty((T, d), dtype=torch.uint8, device=dev) for _ in range(L)]
    if k_scales is None:
        k_scales = [torch.empty((T,), dtype=torch.float32, device=dev) for _ in range(L)]
    if v_scales is None:
        v_scales = [torch.empty((T,), dtype=torch.float32, device=dev) for _ in range(L)]
    stride = d if out_row_stride is None else out_row_stride
    for t in list(k_outs) + list(v_outs):
        if t.dim() != 2 or t.shape != (T, d) or t.stride(1) != 1 or (T > 1 and t.stride(0) != stride):
            raise ValueError("code outputs must be [T, d] u8 views with unit column stride and row stride "
                             "out_row_stride")
    _check(lib().hs2_kv_bridge_fp8(_ptr(hidden), T, D, _ptr_array(w_ks), _ptr_array(w_vs), L, d,
                                   ctypes.cast((ctypes.c_void_p * L)(*[t.data_ptr() for t in k_outs]), ctypes.c_void_p),
                                   ctypes.cast((ctypes.c_void_p * L)(*[t.data_ptr() for t in v_outs]), ctypes.c_void_p),
                                   _ptr_array(k_scales), _ptr_array(v_scales), stride, _stream(stream)))
    return k_outs, k_scales, v_outs, v_scales


def hs2_full_attn_select_workspace_size(B: int, Tq: int, H: int, d: int, Nmax: int, k_global: int,
                                        window: int, kv_dtype: int) -> int:
    return int(lib().hs2_full_attn_select_workspace_size(B, Tq, H, d, Nmax, k_global, window, kv_dtype))


def hs2_sparse_attn_workspace_size(B: int, Tq: int, H: int, d: int, S: int) -> int:
    return int(lib().hs2_sparse_attn_workspace_size(B, Tq, H, d, S))


def sparse_attn_workspace(B: int, Tq: int, H: int, d: int, S: int, device) -> torch.Tensor:
    """A workspace for hs2_sparse_attn (reusable across calls ordered on one stream)."""
    n = hs2_sparse_attn_workspace_size(B, Tq, H, d, S)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=device)


def hs2_full_attn_select(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                         kv_len: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                         v_scale: Optional[torch.Tensor] = None, k_global: int = 1024, window: int = 128,
                         sm_scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                         idx: Optional[torch.Tensor] = None, scores_dbg: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Full-attention MQA layer + token-level selection.  Returns (o fp32 [B,Tq,H,d], idx int32 [B,Tq,k+W])."""
    _check_select_inputs(q, k, v, q_pos, kv_len, k_scale, v_scale)
    B, Tq, H, d = q.shape
    Nmax = k.shape[1]
    kvd = dtype_code(k)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Tq, k_global + window), dtype=torch.int32, device=q.device)
    _expect(o, "o", (B, Tq, H, d), (torch.float32,), q.device)
    _expect(idx, "idx", (B, Tq, k_global + window), (torch.int32,), q.device)
    _expect(scores_dbg, "scores_dbg", (B, Tq, Nmax), (torch.float32,), q.device, optional=True)
    if workspace is not None and workspace.device != q.device:
        raise ValueError("workspace must be on the device of q")
    if workspace is None:
        n = hs2_full_attn_select_workspace_size(B, Tq, H, d, Nmax, k_global, window, kvd)
        workspace = torch.empty((max(n, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().hs2_full_attn_select(
        _ptr(q), dtype_code(q), _ptr(k), _ptr(v), kvd, _ptr(k_scale), _ptr(v_scale), _ptr(q_pos), _ptr(kv_len),
        B, Tq, H, d, Nmax, k_global, window, float(sm_scale), _ptr(o), _ptr(idx), _ptr(scores_dbg),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, idx


HS2_NOALLOC_SCRATCH_BYTES = 64 << 20      # static per-GPU scratch of hs2_full_attn_select_noalloc (hs2.h)


def hs2_full_attn_select_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                                 kv_len: torch.Tensor, o: torch.Tensor, idx: torch.Tensor,
                                 k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                                 k_global: int = 1024, window: int = 128, sm_scale: Optional[float] = None,
                                 scores_dbg: Optional[torch.Tensor] = None, stream=None):
    """hs2_full_attn_select working in the library's static per-GPU scratch instead of a workspace:
    nothing is allocated, so the caller passes the outputs o fp32 [B,Tq,H,d] and idx int32 [B,Tq,k+W].
    Calls that may overlap on one GPU share that scratch and race.  Returns (o, idx)."""
    _check_select_inputs(q, k, v, q_pos, kv_len, k_scale, v_scale)
    B, Tq, H, d = q.shape
    Nmax = k.shape[1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _expect(o, "o", (B, Tq, H, d), (torch.float32,), q.device)
    _expect(idx, "idx", (B, Tq, k_global + window), (torch.int32,), q.device)
    _expect(scores_dbg, "scores_dbg", (B, Tq, Nmax), (torch.float32,), q.device, optional=True)
    _check(lib().hs2_full_attn_select_noalloc(
        _ptr(q), dtype_code(q), _ptr(k), _ptr(v), dtype_code(k), _ptr(k_scale), _ptr(v_scale), _ptr(q_pos),
        _ptr(kv_len), B, Tq, H, d, Nmax, k_global, window, float(sm_scale), _ptr(o), _ptr(idx), _ptr(scores_dbg),
        _stream(stream)))
    return o, idx


def hs2_full_attn_select_blocks_workspace_size(B: int, Tq: int, H: int, d: int, Nmax: int, k_blocks: int,
                                               block: int, window: int, kv_dtype: int) -> int:
    return int(lib().hs2_full_attn_select_blocks_workspace_size(B, Tq, H, d, Nmax, k_blocks, block, window,
                                                                kv_dtype))


def hs2_full_attn_select_blocks(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                                kv_len: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                                v_scale: Optional[torch.Tensor] = None, k_blocks: int = 16, block: int = 64,
                                window: int = 128, sm_scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                                block_idx: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                                scores_dbg: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                stream=None):
    """Full-attention MQA layer + block-level selection.  Returns (o fp32 [B,Tq,H,d],
    block_idx int32 [B,Tq,k_blocks], idx int32 [B,Tq,k_blocks*block+window])."""
    _check_select_inputs(q, k, v, q_pos, kv_len, k_scale, v_scale)
    B, Tq, H, d = q.shape
    Nmax = k.shape[1]
    kvd = dtype_code(k)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device)
    if block_idx is None:
        block_idx = torch.empty((B, Tq, k_blocks), dtype=torch.int32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Tq, k_blocks * block + window), dtype=torch.int32, device=q.device)
    _expect(o, "o", (B, Tq, H, d), (torch.float32,), q.device)
    _expect(block_idx, "block_idx", (B, Tq, k_blocks), (torch.int32,), q.device)
    _expect(idx, "idx", (B, Tq, k_blocks * block + window), (torch.int32,), q.device)
    _expect(scores_dbg, "scores_dbg", (B, Tq, Nmax), (torch.float32,), q.device, optional=True)
    if workspace is not None and workspace.device != q.device:
        raise ValueError("workspace must be on the device of q")
    if workspace is None:
        n = hs2_full_attn_select_blocks_workspace_size(B, Tq, H, d, Nmax, k_blocks, block, window, kvd)
        workspace = torch.empty((max(n, 1),), dtype=torch.uint8, device=q.device)
    _check(lib().hs2_full_attn_select_blocks(
        _ptr(q), dtype_code(q), _ptr(k), _ptr(v), kvd, _ptr(k_scale), _ptr(v_scale), _ptr(q_pos), _ptr(kv_len),
        B, Tq, H, d, Nmax, k_blocks, block, window, float(sm_scale), _ptr(o), _ptr(block_idx), _ptr(idx),
        _ptr(scores_dbg), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, block_idx, idx


def _check_sparse_inputs(qs, k, v, idx, kv_len, k_scale, v_scale, workspace):
    """q [B,Tq,H,d] per layer, k/v [B,Nmax,d], idx [B,Tq,S], kv_len [B] (optional), scales [B,Nmax]."""
    q = qs[0]
    if q.dim() != 4 or k.dim() != 3 or idx.dim() != 3:
        raise ValueError("q must be [B, Tq, H, d], k and v [B, Nmax, d], idx [B, Tq, S]")
    B, Tq, H, d = q.shape
    dev = q.device
    for x in qs:
        _expect(x, "q", (B, Tq, H, d), (torch.float32, torch.bfloat16), dev)
    _expect(k, "k", (B, k.shape[1], d), _KV_DTYPES, dev)
    _expect(v, "v", tuple(k.shape), (k.dtype,), dev)
    _expect(idx, "idx", (B, Tq, idx.shape[-1]), (torch.int32,), dev)
    _expect(kv_len, "kv_len", (B,), (torch.int32,), dev, optional=True)
    _expect(k_scale, "k_scale", (B, k.shape[1]), (torch.float32,), dev, optional=True)
    _expect(v_scale, "v_scale", (B, k.shape[1]), (torch.float32,), dev, optional=True)
    if workspace is not None and workspace.device != dev:
        raise ValueError("workspace must be on the device of q")


def hs2_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                    kv_len: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                    v_scale: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                    o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Sparse layer reusing the full layer's KV and indices.  Returns o fp32 [B,Tq,H,d]."""
    _check_sparse_inputs([q], k, v, idx, kv_len, k_scale, v_scale, workspace)
    B, Tq, H, d = q.shape
    Nmax = k.shape[1]
    S = idx.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device)
    _expect(o, "o", (B, Tq, H, d), (torch.float32,), q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hs2_sparse_attn(
        _ptr(q), dtype_code(q), _ptr(k), _ptr(v), dtype_code(k), _ptr(k_scale), _ptr(v_scale), _ptr(idx), S,
        _ptr(kv_len), B, Tq, H, d, Nmax, float(sm_scale), _ptr(o), _ptr(workspace), wsb, _stream(stream)))
    return o


def hs2_sparse_attn_layers_workspace_size(B: int, Tq: int, H: int, d: int, S: int, L: int) -> int:
    return int(lib().hs2_sparse_attn_layers_workspace_size(B, Tq, H, d, S, L))


def sparse_attn_layers_workspace(B: int, Tq: int, H: int, d: int, S: int, L: int, device) -> torch.Tensor:
    """A workspace for hs2_sparse_attn_layers with L layers (reusable across ordered calls)."""
    n = hs2_sparse_attn_layers_workspace_size(B, Tq, H, d, S, L)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=device)


def hs2_sparse_attn_layers(qs, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                           kv_len: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                           v_scale: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                           os=None, workspace: Optional[torch.Tensor] = None, stream=None):
    """L sparse layers (one query tensor each) over the same KV and indices in one call.
    Returns the list of o tensors (fp32 [B,Tq,H,d])."""
    L = len(qs)
    B, Tq, H, d = qs[0].shape
    for q in qs:
        if q.shape != qs[0].shape or q.dtype != qs[0].dtype:
            raise ValueError("all layers' queries must have the same shape and dtype")
    _check_sparse_inputs(qs, k, v, idx, kv_len, k_scale, v_scale, workspace)
    Nmax = k.shape[1]
    S = idx.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if os is None:
        os = [torch.empty((B, Tq, H, d), dtype=torch.float32, device=qs[0].device) for _ in range(L)]
    if len(os) != L:
        raise ValueError("one output per layer")
    for o in os:
        _expect(o, "o", (B, Tq, H, d), (torch.float32,), qs[0].device)
    qa = (ctypes.c_void_p * L)(*[_ptr(q) for q in qs])
    oa = (ctypes.c_void_p * L)(*[_ptr(o) for o in os])
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hs2_sparse_attn_layers(
        ctypes.cast(qa, ctypes.c_void_p), L, dtype_code(qs[0]), _ptr(k), _ptr(v), dtype_code(k), _ptr(k_scale),
        _ptr(v_scale), _ptr(idx), S, _ptr(kv_len), B, Tq, H, d, Nmax, float(sm_scale),
        ctypes.cast(oa, ctypes.c_void_p), _ptr(workspace), wsb, _stream(stream)))
    return os


def hs2_decode_block_workspace_size(B: int, Tq: int, H: int, d: int, Nmax: int, k_global: int, window: int,
                                    kv_dtype: int, L: int) -> int:
    return int(lib().hs2_decode_block_workspace_size(B, Tq, H, d, Nmax, k_global, window, kv_dtype, L))


def decode_block_workspace(B: int, Tq: int, H: int, d: int, Nmax: int, k_global: int, window: int, kv_dtype: int,
                           L: int, device) -> torch.Tensor:
    n = hs2_decode_block_workspace_size(B, Tq, H, d, Nmax, k_global, window, kv_dtype, L)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=device)


def hs2_decode_block(q: torch.Tensor, qs, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                     kv_len: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                     v_scale: Optional[torch.Tensor] = None, k_global: int = 1024, window: int = 128,
                     sm_scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                     idx: Optional[torch.Tensor] = None, os=None, workspace: Optional[torch.Tensor] = None,
                     stream=None):
    """The decode hybrid block (full layer + selection + every sparse layer) in one launch.
    Returns (o fp32 [B,Tq,H,d], idx int32 [B,Tq,k+W], [o of each sparse layer])."""
    _check_select_inputs(q, k, v, q_pos, kv_len, k_scale, v_scale)
    B, Tq, H, d = q.shape
    L = len(qs)
    Nmax = k.shape[1]
    kvd = dtype_code(k)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((B, Tq, k_global + window), dtype=torch.int32, device=q.device)
    if os is None:
        os = [torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device) for _ in range(L)]
    if workspace is None:
        workspace = decode_block_workspace(B, Tq, H, d, Nmax, k_global, window, kvd, L, q.device)
    for x in qs:
        if x.shape != q.shape or x.dtype != q.dtype:
            raise ValueError("every sparse layer's queries must have the full layer's shape and dtype")
    if len(os) != L:
        raise ValueError("one output per sparse layer")
    _expect(o, "o", (B, Tq, H, d), (torch.float32,), q.device)
    _expect(idx, "idx", (B, Tq, k_global + window), (torch.int32,), q.device)
    for x in list(os):
        _expect(x, "o_sparse", (B, Tq, H, d), (torch.float32,), q.device)
    for x in qs:
        _expect(x, "q_sparse", (B, Tq, H, d), (q.dtype,), q.device)
    if workspace.device != q.device:
        raise ValueError("workspace must be on the device of q")
    qa = (ctypes.c_void_p * L)(*[_ptr(x) for x in qs])
    oa = (ctypes.c_void_p * L)(*[_ptr(x) for x in os])
    _check(lib().hs2_decode_block(
        _ptr(q), ctypes.cast(qa, ctypes.c_void_p), L, dtype_code(q), _ptr(k), _ptr(v), kvd, _ptr(k_scale),
        _ptr(v_scale), _ptr(q_pos), _ptr(kv_len), B, Tq, H, d, Nmax, k_global, window, float(sm_scale), _ptr(o),
        _ptr(idx), ctypes.cast(oa, ctypes.c_void_p), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return o, idx, os


def profile_enable(enable: bool = True):
    lib().hs2_profile_enable(1 if enable else 0)


def profile_read() -> dict:
    """{kernel name: (total ms, launches)} accumulated since profile_enable(True)."""
    out = {}
    i = 0
    name = ctypes.c_char_p()
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    while lib().hs2_profile_read(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)) == 0:
        out[name.value.decode()] = (ms.value, n.value)
        i += 1
    return out
