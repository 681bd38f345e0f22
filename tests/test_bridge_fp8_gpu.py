"""GPU parity of the multi-target FP8 bridge (hs2_kv_bridge_fp8) against the oracle.

The quantisation is decided in fp32 on both sides: the oracle rounds its float64 product to fp32,
the kernel accumulates in fp32.  With integer operands every fp32 sum is exact, so codes and
scales must be bit-identical.  With real-valued operands the two fp32 values differ by at most the
summation bound D * 2^-24 * sum|h w|, so a code may differ only by one step, only where the
oracle's quotient lies within that bound (scaled) of the rounding boundary between the two codes,
and the scales agree to the same relative bound.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.hs2_harness import _say, to_dev
from workloads.gen import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _run(hb, wks, wvs, stride=None, T_view=None):
    import token_level_sparse_mqa_amd as hs2
    T, D = hb.shape
    d = wks[0].shape[0]
    L = len(wks)
    if stride is None:
        return hs2.hs2_kv_bridge_fp8(to_dev(hb, "bf16"), [to_dev(w, "bf16") for w in wks],
                                     [to_dev(w, "bf16") for w in wvs])
    # codes into the middle of wider rows, the bytes around them untouched
    kc = [torch.full((T, stride), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(L)]
    vc = [torch.full((T, stride), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(L)]
    off = (stride - d) // 2
    res = hs2.hs2_kv_bridge_fp8(to_dev(hb, "bf16"), [to_dev(w, "bf16") for w in wks], [to_dev(w, "bf16") for w in wvs],
                                k_outs=[c[:, off:off + d] for c in kc], v_outs=[c[:, off:off + d] for c in vc],
                                out_row_stride=stride)
    for c in kc + vc:
        h = c.cpu().numpy()
        assert np.all(h[:, :off] == 0x5A) and np.all(h[:, off + d:] == 0x5A), "bytes outside the code rows written"
    return res


def _host(res):
    kc, ks, vc, vs = res
    return [(kc[l].cpu().numpy(), ks[l].cpu().numpy(), vc[l].cpu().numpy(), vs[l].cpu().numpy()) for l in range(len(kc))]


@pytest.mark.parametrize("T,D,L,d,stride", [(300, 256, 3, 128, None), (1, 64, 1, 64, None), (257, 128, 8, 64, 96),
                                            (1000, 512, 2, 128, 160)])
def test_bridge_fp8_integer_exact(T, D, L, d, stride):
    """Integer operands: exact fp32 sums, so codes and scales are bit-identical to the oracle's."""
    rng = np.random.default_rng(T + 31 * L + d)
    hb = f32_to_bf16_bits(rng.integers(-3, 4, size=(T, D)).astype(np.float32))
    hb[T // 2] = 0                                  # a zero row: scale 1, codes 0
    wks = [f32_to_bf16_bits(rng.integers(-3, 4, size=(d, D)).astype(np.float32)) for _ in range(L)]
    wvs = [f32_to_bf16_bits(rng.integers(-3, 4, size=(d, D)).astype(np.float32)) for _ in range(L)]
    got = _host(_run(hb, wks, wvs, stride=stride))
    ref = oracle.kv_bridge_fp8(hb, wks, wvs)
    for l in range(L):
        for a, b, what in zip(got[l], ref[l], ("k codes", "k scale", "v codes", "v scale")):
            assert np.array_equal(a, b), f"target {l}: {what} differ"
    assert np.all(got[0][1][T // 2] == 1.0) and np.all(got[0][0][T // 2] == 0)


def check_fp8_close(hb, wks, wvs, got, ref, sample_rows=None):
    """Real-valued operands: the bound described in the module docstring."""
    D = hb.shape[1]
    rows = np.arange(hb.shape[0]) if sample_rows is None else sample_rows
    h = oracle.decode(hb[rows], "bf16")
    mism, total = 0, 0
    for l in range(len(wks)):
        for (codes, scale, w_bits), (rc, rs) in (((got[l][0], got[l][1], wks[l]), (ref[l][0], ref[l][1])),
                                                 ((got[l][2], got[l][3], wvs[l]), (ref[l][2], ref[l][3]))):
            w = oracle.decode(w_bits, "bf16")
            exact = h @ w.T
            bound = D * 2.0 ** -24 * (np.abs(h) @ np.abs(w).T)            # |fp32 sum - exact|
            amax = np.abs(exact).max(axis=1)
            gs, rsc = scale[rows].astype(np.float64), rs[rows].astype(np.float64)
            # scales: amax / 448 each, the maxima within the summation bound (+ fp32 roundings)
            assert np.all(np.abs(gs - rsc) <= (bound.max(axis=1) / 448.0 + 4 * 2.0 ** -24 * amax / 448.0) + 1e-30)
            gc, oc = codes[rows], rc[rows]
            diff = gc != oc
            mism += int(diff.sum())
            total += gc.size
            if diff.any():
                gv = oracle.e4m3fn_bits_to_f64(gc)
                ov = oracle.e4m3fn_bits_to_f64(oc)
                # adjacent codes only, same sign
                assert np.all(np.abs(gc[diff].astype(int) - oc[diff].astype(int)) == 1), "codes differ by more than one step"
                # the exact quotient sits within the summation bound of the boundary between them
                mid = (gv[diff] + ov[diff]) / 2
                q = (exact / rsc[:, None])[diff]
                rel = (bound.max(axis=1) / np.maximum(amax, 1e-30))[:, None] * np.ones_like(exact)
                tol = (bound / rsc[:, None])[diff] + np.abs(q) * (rel[diff] + 1e-5) + 1e-9
                assert np.all(np.abs(np.abs(q) - np.abs(mid)) <= tol), "a code differs away from a rounding boundary"
    frac = mism / max(total, 1)
    _say(f"[bridge_fp8] code mismatch fraction {frac:.2e} over {total} codes")
    assert frac < 1e-3
    return frac


@pytest.mark.parametrize("T,D,L,d", [(777, 2048, 3, 128), (300, 1024, 2, 64)])
def test_bridge_fp8_random(T, D, L, d):
    rng = np.random.default_rng(T * 3 + L)
    hb = f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wks = [f32_to_bf16_bits((rng.standard_normal((d, D)) * 0.02).astype(np.float32)) for _ in range(L)]
    wvs = [f32_to_bf16_bits((rng.standard_normal((d, D)) * 0.02).astype(np.float32)) for _ in range(L)]
    got = _host(_run(hb, wks, wvs))
    ref = oracle.kv_bridge_fp8(hb, wks, wvs)
    check_fp8_close(hb, wks, wvs, got, ref)


def test_bridge_fp8_targets_independent():
    """A target whose Wk is another target's Wv reproduces that target's V bit for bit."""
    rng = np.random.default_rng(77)
    T, D, d = 513, 512, 128
    hb = f32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wv0 = f32_to_bf16_bits((rng.standard_normal((d, D)) * 0.02).astype(np.float32))
    wks = [f32_to_bf16_bits((rng.standard_normal((d, D)) * 0.02).astype(np.float32)), wv0.copy()]
    wvs = [wv0, f32_to_bf16_bits((rng.standard_normal((d, D)) * 0.02).astype(np.float32))]
    got = _host(_run(hb, wks, wvs))
    assert np.array_equal(got[1][0], got[0][2]) and np.array_equal(got[1][1], got[0][3])


def test_bridge_fp8_full_size_sampled():
    """The bench shape: 262,144 hidden states of width 2048 into 6 targets' FP8 caches, rows sampled."""
    from workloads import BRIDGE_FP8, make_bridge_fp8_inputs
    cfg = BRIDGE_FP8["bridge_fp8_256k"]
    inp = make_bridge_fp8_inputs(cfg)
    got = _host(_run(inp.hidden, inp.wk_t, inp.wv_t))
    rows = np.sort(np.random.default_rng(5).choice(cfg.T, size=512, replace=False))
    sub = inp.hidden[rows]
    ref = oracle.kv_bridge_fp8(sub, inp.wk_t, inp.wv_t)
    # compare the sampled rows: the oracle ran on those rows only
    got_rows = [(g[0][rows], g[1][rows], g[2][rows], g[3][rows]) for g in got]
    check_fp8_close(sub, inp.wk_t, inp.wv_t, got_rows, ref)


def test_bridge_fp8_encoder_exact():
    """The conversion to E4M3FN on its own: one-hot hidden rows pick a weight column per row, and a
    448 in column 0 makes every row's scale exactly 1, so each code is the encoding of a chosen bf16
    value: every midpoint between neighbouring codes (ties to even), every code value, random values
    in range, both signs; bit-identical to the oracle's encoder."""
    T, D, d = 64, 64, 128
    vals = oracle.e4m3fn_bits_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(21)
    pool = np.concatenate([vals, mids, -vals, -mids, rng.uniform(-448, 448, 4096)])
    pool = oracle.bf16_bits_to_f64(f32_to_bf16_bits(pool.astype(np.float32)))    # bf16 values (mids exact)
    need = T * (d - 1)
    pool = np.resize(rng.permutation(pool), need)
    w = np.zeros((d, D), dtype=np.float32)
    w[0, :] = 448.0
    w[1:, :T] = pool.reshape(d - 1, T)
    wb = f32_to_bf16_bits(w)
    hb = f32_to_bf16_bits(np.eye(T, D, dtype=np.float32))
    got = _host(_run(hb, [wb], [wb[::-1].copy()]))
    ref = oracle.kv_bridge_fp8(hb, [wb], [wb[::-1].copy()])
    assert np.all(got[0][1] == 1.0)
    for a, b, what in zip(got[0], ref[0], ("k codes", "k scale", "v codes", "v scale")):
        assert np.array_equal(a, b), what
