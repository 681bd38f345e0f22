"""Float64 CPU oracle of the HySparse2 hybrid-block attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (``token_level_sparse_mqa_amd``) and never imports it.

What the hot path computes, written as plain definitions (numpy, float64):

* KV Bridging: the cross-decoder full-attention layer builds its K/V by projecting
  self-decoder hidden states, one projection pair per target layer (lynxflow blog,
  "Two-Level KV Sharing"; agentik-os article, section 2 "Two levels of KV sharing";
  ainews page, mechanism paragraph).  Read here as K = H.Wk, V = H.Wv with no bias,
  no positional rotation and no norm, rounded to bf16 (round to nearest even).
* Full-attention MQA layer: softmax attention of H query heads over one shared KV
  head (ainews page, GQA to MQA in the experimental-setup paragraph), causal, with
  scale 1/sqrt(d).  It outputs O and, "upon completion", the selection indices
  (lynxflow blog, "Two-Level KV Sharing", KV Reuse).
* Selection score (the pages leave it open; agentik-os "What is not documented"):
  per key, the sum over heads of the full layer's softmax probabilities, the softmax
  being over every visible key, window included.
* Token-level selection: the 1,024 best-scoring positions chosen one by one, ties
  to the lower index, plus a forced window of the 128 most recent positions
  (kucoin news flash; lynxflow "Token-Level Sparse Selection"; agentik-os section 3).
  Candidates for the global picks are the positions before the window, j <= t - W;
  the window is [t - W + 1, t], clamped at 0.  Fewer than k candidates: take all.
  Index layout per query: [global picks ascending, -1 padding up to k]
  followed by [window ascending, -1 padding up to W].
* Sparse layers (KV Reuse): each layer's own Q attends with softmax over exactly the
  selected rows of the full layer's cache (lynxflow "Two-Level KV Sharing";
  agentik-os section 2; ainews mechanism paragraph).
* FP8 caches (ainews experimental-setup paragraph): OCP E4M3FN codes times a per-row
  fp32 scale.
* Multi-target FP8 bridge: every cross-decoder full layer projects the same hidden states
  with its own Wk, Wv (lynxflow "Two-Level KV Sharing") into an FP8 cache (ainews
  experimental-setup paragraph): per row, scale = amax/448 in fp32, codes = E4M3FN of x/scale.
* Block-level selection, the first-generation scheme the pages compare against (kucoin
  news flash; lynxflow "Token-Level Sparse Selection"): candidates in groups of 64, a
  group kept whole when any member is important.  Read here with the same score and the
  same budget: block score = max of its members' scores, the 1024/64 = 16 best blocks.

Every function is pinned by tests under tests/test_oracle_*.py against closed forms,
library routines, brute force and invariants.
"""
from __future__ import annotations

import numpy as np

K_GLOBAL = 1024
WINDOW = 128


# ----------------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------------
def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen the bits, then reinterpret."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bfloat16, ties to even (finite inputs).

    A bf16 value is m * 2^(e-7) with an 8-bit significand m in [128, 255] (normal) or a
    multiple of 2^-133 (subnormal).  The spacing at x is found from its exponent and
    x / spacing is rounded with numpy's round-half-to-even, so the result is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = x != 0
    ax = np.abs(x[nz])
    e = np.floor(np.log2(ax))
    # guard the floor(log2) against rounding at exact powers of two
    e = np.where(2.0 ** e > ax, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= ax, e + 1, e)
    e = np.maximum(e, -126.0)                 # subnormal range shares the 2^-133 spacing
    spacing = 2.0 ** (e - 7)
    out[nz] = np.sign(x[nz]) * np.round(ax / spacing) * spacing
    f32 = out.astype(np.float32)              # exact: every bf16 value is a binary32 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return bits


def e4m3fn_bits_to_f64(u8: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 ("FN": no infinities).

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent field 0 holds the
    subnormals m * 2^-9; S.1111.111 is NaN; every other code is (1 + m/8) * 2^(e-7).
    """
    c = np.asarray(u8, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = s * val
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def decode(arr: np.ndarray, dtype: str, scale: np.ndarray | None = None) -> np.ndarray:
    """Stored bytes -> float64 values.  fp8 rows are multiplied by their fp32 scale."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        return e4m3fn_bits_to_f64(arr) * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# KV Bridging
# ----------------------------------------------------------------------------------------------
def kv_bridge(hidden_bf16: np.ndarray, wk_bf16: np.ndarray, wv_bf16: np.ndarray,
              row_block: int = 8192):
    """K = bf16(H.Wk), V = bf16(H.Wv) with float64 products and sums.

    hidden [T, D], wk/wv [D, d] as bf16 bit patterns -> (k, v) [T, d] bf16 bit patterns.
    """
    wk = bf16_bits_to_f64(wk_bf16)
    wv = bf16_bits_to_f64(wv_bf16)
    T = hidden_bf16.shape[0]
    k = np.empty((T, wk.shape[1]), dtype=np.uint16)
    v = np.empty((T, wv.shape[1]), dtype=np.uint16)
    for r0 in range(0, T, row_block):
        h = bf16_bits_to_f64(hidden_bf16[r0:r0 + row_block])
        k[r0:r0 + row_block] = f64_to_bf16_bits_rne(h @ wk)
        v[r0:r0 + row_block] = f64_to_bf16_bits_rne(h @ wv)
    return k, v


FP8_MAX = 448.0


def e4m3fn_encode_rne(y: np.ndarray) -> np.ndarray:
    """Values -> OCP E4M3FN codes: the nearest finite code (ties to the even code, i.e. even
    mantissa), saturating at +-448; the sign bit follows the value's sign (-0 -> 0x80).  Written
    as a search over the 127 non-negative finite code values."""
    table = e4m3fn_bits_to_f64(np.arange(0x7F, dtype=np.uint8))        # ascending: 0 .. 448
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), FP8_MAX)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))


def kv_bridge_fp8(hidden_bf16: np.ndarray, wk_t_bf16, wv_t_bf16, row_block: int = 8192):
    """Multi-target KV bridge into FP8 caches.  Every target layer has its own projections
    (lynxflow "Two-Level KV Sharing"); here all targets project the same hidden states.
    hidden [T, D] bf16 bits; wk_t_bf16 / wv_t_bf16: one [d, D] bf16 matrix per target (a linear
    layer's weight: output rows).  Per target and row: x = H.W^T with float64 products and sums,
    taken to fp32 (the precision the quantisation decides in); scale = fp32(amax|x| / 448) (1 when
    the row is all zero); codes = E4M3FN(fp32(x / scale)).
    Returns a list of (k_codes [T, d] u8, k_scale [T] f32, v_codes, v_scale), one per target."""
    T = hidden_bf16.shape[0]
    out = []
    for wk_b, wv_b in zip(wk_t_bf16, wv_t_bf16):
        res = []
        for w_b in (wk_b, wv_b):
            w = bf16_bits_to_f64(w_b)
            d = w.shape[0]
            codes = np.empty((T, d), dtype=np.uint8)
            scale = np.empty((T,), dtype=np.float32)
            for r0 in range(0, T, row_block):
                h = bf16_bits_to_f64(hidden_bf16[r0:r0 + row_block])
                x = (h @ w.T).astype(np.float32)
                amax = np.abs(x).max(axis=1)
                sc = (amax / np.float32(FP8_MAX)).astype(np.float32)
                sc = np.where(amax > 0, sc, np.float32(1.0)).astype(np.float32)
                y = (x / sc[:, None]).astype(np.float32)
                codes[r0:r0 + row_block] = e4m3fn_encode_rne(y.astype(np.float64))
                scale[r0:r0 + row_block] = sc
            res += [codes, scale]
        out.append(tuple(res))
    return out


# ----------------------------------------------------------------------------------------------
# Full-attention layer, score, selection
# ----------------------------------------------------------------------------------------------
def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, t: int, sm: float):
    """One query token at position t.  q [H, d]; k, v [N, d] (one shared KV head).

    s[h, j] = sm * q[h].k[j] for 0 <= j <= t; p = softmax_j(s); o[h] = sum_j p[h, j] v[j].
    Returns (o [H, d], p [H, t+1]).
    """
    kk = k[: t + 1]
    s = sm * (q @ kk.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v[: t + 1], p


def selection_scores(p: np.ndarray, t: int, window: int) -> np.ndarray:
    """score[j] = sum_h p[h, j] for the global candidates j in [0, t - window]."""
    C = max(0, t - window + 1)
    return p[:, :C].sum(axis=0)


def select_global(score: np.ndarray, k_global: int) -> np.ndarray:
    """The min(k, C) best candidates by (score descending, index ascending), ascending."""
    order = np.argsort(-score, kind="stable")
    return np.sort(order[: min(k_global, score.shape[0])])


def assemble_indices(global_sel: np.ndarray, t: int, k_global: int, window: int) -> np.ndarray:
    """[global picks, -1 pad to k] ++ [window max(0,t-W+1)..t, -1 pad to W]."""
    idx = np.full(k_global + window, -1, dtype=np.int32)
    idx[: global_sel.shape[0]] = global_sel
    win = np.arange(max(0, t - window + 1), t + 1)
    idx[k_global: k_global + win.shape[0]] = win
    return idx


def full_attn_select_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, t: int, sm: float,
                         k_global: int = K_GLOBAL, window: int = WINDOW):
    """One query token of the full-attention layer: (o [H,d], idx [k+W], score [C])."""
    o, p = dense_attention(q, k, v, t, sm)
    score = selection_scores(p, t, window)
    g = select_global(score, k_global)
    return o, assemble_indices(g, t, k_global, window), score


# ----------------------------------------------------------------------------------------------
# Block-level selection (the first-generation variant the token-level one replaces)
# ----------------------------------------------------------------------------------------------
BLOCK = 64


def block_scores(score: np.ndarray, block: int) -> np.ndarray:
    """Candidates grouped in consecutive blocks of `block` positions (the last block may be
    shorter); a block's score is the largest score of its members, so a block ranks as high as
    its most important token (kucoin news flash: groups of 64 kept whole when any member is
    important).  score [C] -> [ceil(C / block)]."""
    C = score.shape[0]
    nb = -(-C // block)
    return np.array([score[b * block: min(C, (b + 1) * block)].max() for b in range(nb)], dtype=np.float64)


def select_blocks(score: np.ndarray, k_blocks: int, block: int) -> np.ndarray:
    """The min(k_blocks, #blocks) best blocks by (block score descending, block id ascending),
    as ascending block ids: the token rule applied to blocks, with the same budget of
    k_blocks * block positions."""
    return select_global(block_scores(score, block), k_blocks)


def expand_blocks(blocks: np.ndarray, C: int, block: int) -> np.ndarray:
    """Every candidate position of the chosen blocks, ascending (a block past C is cut at C)."""
    parts = [np.arange(b * block, min(C, (b + 1) * block)) for b in np.asarray(blocks, dtype=np.int64)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def full_attn_select_blocks_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, t: int, sm: float,
                                k_blocks: int = K_GLOBAL // BLOCK, block: int = BLOCK,
                                window: int = WINDOW):
    """One query token with block-level selection: (o [H,d], block ids [k_blocks] ascending with
    -1 padding, idx [k_blocks * block + W] in the token layout, score [C])."""
    o, p = dense_attention(q, k, v, t, sm)
    score = selection_scores(p, t, window)
    blocks = select_blocks(score, k_blocks, block)
    bid = np.full(k_blocks, -1, dtype=np.int32)
    bid[: blocks.shape[0]] = blocks
    idx = assemble_indices(expand_blocks(blocks, score.shape[0], block), t, k_blocks * block, window)
    return o, bid, idx, score


# ----------------------------------------------------------------------------------------------
# Sparse (index-reusing) layer
# ----------------------------------------------------------------------------------------------
def sparse_attention_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                         sm: float) -> np.ndarray:
    """Softmax attention of q [H,d] over the rows k[idx], v[idx] (entries -1 skipped)."""
    sel = np.asarray(idx)[np.asarray(idx) >= 0]
    if sel.shape[0] == 0:
        return np.zeros_like(q)
    s = sm * (q @ k[sel].T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v[sel]
