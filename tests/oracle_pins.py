"""Pins of the float64 oracle: checks against facts fixed outside the oracle itself.

Each ``check_*`` takes the oracle module (so a deliberately broken copy can be passed
in by the mutation tests) and raises AssertionError when a pin fails.  Sources of
truth: closed forms, library routines (torch CPU float64 scaled_dot_product_attention,
torch's bf16 / float8_e4m3fn conversions), brute force on tiny inputs, invariants.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch


def _sdpa_causal_row(q, k, v, t, sm):
    """Library reference: torch SDPA (float64, CPU) with an explicit causal mask row."""
    H, d = q.shape
    qt = torch.from_numpy(q).reshape(1, H, 1, d)
    kt = torch.from_numpy(np.ascontiguousarray(k)).reshape(1, 1, -1, d).expand(1, H, -1, d)
    vt = torch.from_numpy(np.ascontiguousarray(v)).reshape(1, 1, -1, d).expand(1, H, -1, d)
    mask = torch.zeros(1, 1, 1, k.shape[0], dtype=torch.bool)
    mask[..., : t + 1] = True
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm)
    return o.reshape(H, d).numpy()


def check_dense_vs_sdpa(O, seed=0):
    rng = np.random.default_rng(seed)
    for (H, d, N, t) in [(4, 16, 37, 36), (4, 16, 37, 0), (3, 8, 50, 21), (16, 64, 300, 299)]:
        q = rng.standard_normal((H, d))
        k = rng.standard_normal((N, d)) * 1.3
        v = rng.standard_normal((N, d))
        sm = 1.0 / math.sqrt(d)
        o, p = O.dense_attention(q, k, v, t, sm)
        ref = _sdpa_causal_row(q, k, v, t, sm)
        assert p.shape == (H, t + 1)
        assert np.max(np.abs(o - ref)) <= 1e-12, "dense attention differs from SDPA"


def check_identical_keys(O):
    """Identical keys: uniform p = 1/(t+1), O = mean of visible V rows, score = H/(t+1),
    ties resolve to the lowest indices."""
    rng = np.random.default_rng(1)
    H, d, N, t, W, kg = 5, 8, 400, 330, 16, 100
    q = rng.standard_normal((H, d))
    k = np.tile(rng.standard_normal((1, d)), (N, 1))
    v = rng.standard_normal((N, d))
    o, p = O.dense_attention(q, k, v, t, 1.0 / math.sqrt(d))
    assert np.allclose(p, 1.0 / (t + 1), rtol=0, atol=1e-15)
    assert np.allclose(o, v[: t + 1].mean(axis=0)[None, :], rtol=0, atol=1e-13)
    sc = O.selection_scores(p, t, W)
    assert sc.shape == (t - W + 1,)
    assert np.allclose(sc, H / (t + 1), rtol=0, atol=1e-14)
    g = O.select_global(np.full(sc.shape, H / (t + 1)), kg)
    assert np.array_equal(g, np.arange(kg))


def check_score_mass(O):
    """Each head's probabilities sum to one, so candidate scores plus the window's
    mass over all heads equals H."""
    rng = np.random.default_rng(2)
    H, d, N, W = 6, 16, 260, 32
    q = rng.standard_normal((H, d)) * 2
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    for t in (259, 100, W - 1, W, 5):
        _, p = O.dense_attention(q, k, v, t, 0.25)
        sc = O.selection_scores(p, t, W)
        C = max(0, t - W + 1)
        assert sc.shape == (C,)
        win_mass = p[:, C: t + 1].sum()
        assert abs(sc.sum() + win_mass - H) <= 1e-12
        # window mass is exactly the probability of the last min(W, t+1) positions
        assert abs(win_mass - p[:, max(0, t - W + 1):].sum()) <= 1e-12


def check_onehot_keys(O):
    """Orthogonal one-hot keys: q = e_a gives logit sm*c on key a and 0 elsewhere."""
    H, d, t, c = 2, 8, 7, 3.0
    k = np.zeros((t + 1, d))
    for j in range(t + 1):
        k[j, j] = c
    q = np.zeros((H, d))
    q[0, 2] = 1.0
    q[1, 5] = 1.0
    v = np.arange((t + 1) * d, dtype=np.float64).reshape(t + 1, d)
    sm = 0.5
    _, p = O.dense_attention(q, k, v, t, sm)
    z = math.exp(sm * c) + t
    for h, a in ((0, 2), (1, 5)):
        assert abs(p[h, a] - math.exp(sm * c) / z) <= 1e-15
        others = np.delete(p[h], a)
        assert np.allclose(others, 1.0 / z, rtol=0, atol=1e-15)


def _rank_count_select(scores, k):
    """Brute force from the definition: j is picked iff fewer than k candidates beat it,
    where i beats j when s_i > s_j, or s_i == s_j and i < j."""
    n = len(scores)
    sel = []
    for j in range(n):
        beat = sum(1 for i in range(n) if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if beat < k:
            sel.append(j)
    return np.array(sel, dtype=np.int64)


def check_selection_bruteforce(O, trials=300):
    rng = np.random.default_rng(3)
    for _ in range(trials):
        n = int(rng.integers(1, 13))
        s = rng.integers(0, 4, size=n).astype(np.float64)  # many exact ties
        for k in range(0, n + 2):
            got = O.select_global(s, k)
            exp = _rank_count_select(list(s), k)
            assert np.array_equal(got, exp), (s, k, got, exp)


def check_selection_exhaustive(O):
    """For n <= 8, among all k-subsets the picked one has the largest score multiset and,
    among equal multisets, the lexicographically smallest index list."""
    rng = np.random.default_rng(4)
    for _ in range(60):
        n = int(rng.integers(1, 9))
        s = rng.integers(0, 3, size=n).astype(np.float64)
        for k in range(1, n + 1):
            best = None
            for sub in itertools.combinations(range(n), k):
                key = (tuple(sorted((-s[i] for i in sub))), sub)
                if best is None or key < best:
                    best = key
            assert tuple(O.select_global(s, k)) == best[1]


def check_window_enumeration(O, k=1024, W=128, t_max=1300):
    """Exact index lists for every position 0..t_max on identical scores."""
    for t in range(t_max + 1):
        C = max(0, t - W + 1)
        exp = [-1] * (k + W)
        for j in range(min(k, C)):
            exp[j] = j                               # identical scores: lowest indices
        w = [j for j in range(t - W + 1, t + 1) if j >= 0]
        for i, j in enumerate(w):
            exp[k + i] = j
        g = O.select_global(np.ones(C), k)
        got = O.assemble_indices(g, t, k, W)
        assert got.dtype == np.int32 and got.shape == (k + W,)
        assert got.tolist() == exp, t


def check_sparse_identity(O):
    """If the selection keeps every visible position, sparse attention is dense causal
    attention of the same query (library routine)."""
    rng = np.random.default_rng(5)
    H, d, N, W, kg = 4, 16, 90, 8, 100
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    sm = 1.0 / math.sqrt(d)
    for t in (89, 50, 3):
        _, idx, _ = O.full_attn_select_row(q, k, v, t, sm, kg, W)
        o_sp = O.sparse_attention_row(q, k, v, idx, sm)
        assert np.max(np.abs(o_sp - _sdpa_causal_row(q, k, v, t, sm))) <= 1e-12


def check_sparse_order_invariance(O):
    rng = np.random.default_rng(6)
    H, d, N = 4, 16, 200
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    idx = rng.choice(N, size=40, replace=False).astype(np.int32)
    base = O.sparse_attention_row(q, k, v, idx, 0.3)
    for _ in range(5):
        perm = rng.permutation(np.concatenate([idx, -np.ones(9, dtype=np.int32)]))
        assert np.max(np.abs(O.sparse_attention_row(q, k, v, perm, 0.3) - base)) <= 1e-12
    # a direct per-head definition: o[h] = sum_j w_j v_j / sum_j w_j, w_j = exp(0.3 q.k_j)
    for h in range(H):
        w = np.array([math.exp(0.3 * float(q[h] @ k[j])) for j in idx])
        ref = (w[:, None] * v[idx]).sum(axis=0) / w.sum()
        assert np.max(np.abs(base[h] - ref)) <= 1e-12


def check_needles(O):
    """A key planted as 4x a query head wins that head's softmax, is selected, and the
    head's output is (nearly) that key's value row."""
    rng = np.random.default_rng(7)
    H, d, N, W, kg = 8, 64, 3000, 128, 64
    q = rng.standard_normal((H, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    t, h, p = N - 1, 3, 1234
    k[p] = 4.0 * q[h]
    o, idx, score = O.full_attn_select_row(q, k, v, t, 1.0 / math.sqrt(d), kg, W)
    assert p in set(idx[:kg].tolist())
    assert score[p] >= 0.99
    assert np.max(np.abs(o[h] - v[p])) <= 1e-6


def check_bf16(O):
    # all 2^16 patterns against torch's bfloat16 decoding
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # encoder: exact ties round to even (closed forms), values beyond a tie round up
    cases = {1.0 + 2.0 ** -8: 1.0, 1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,
             1.0 + 2.0 ** -8 + 2.0 ** -40: 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -8): -1.0,
             3.0: 3.0, 2.0 ** -130: 2.0 ** -130, 0.0: 0.0}
    xs = np.array(list(cases.keys()))
    got = O.bf16_bits_to_f64(O.f64_to_bf16_bits_rne(xs))
    assert np.array_equal(got, np.array(list(cases.values())))
    # float32-representable inputs: torch's conversion is a single RNE rounding
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    ties = (rng.integers(0, 1 << 16, 4000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits_rne(x.astype(np.float64)), ref)


def check_e4m3fn(O):
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3fn_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # closed-form points of the format: max normal, min normal, min subnormal, one
    pts = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
           0x38: 1.0, 0xB8: -1.0, 0x00: 0.0}
    for c, val in pts.items():
        assert mine[c] == val, (hex(c), mine[c], val)
    sc = np.array([0.5, 3.0], dtype=np.float32)
    dec = O.decode(np.array([[0x38, 0x7E], [0x01, 0xB8]], dtype=np.uint8), "fp8", sc)
    assert np.array_equal(dec, np.array([[0.5, 224.0], [3.0 * 2.0 ** -9, -3.0]]))


def check_bridge(O):
    """Small-integer operands make every float64 sum exact; |sums| <= 256 are exact in bf16,
    so the result must equal the integer matmul.  Ties in the final rounding go to even."""
    rng = np.random.default_rng(9)
    T, D, d = 37, 16, 8
    h = rng.integers(-2, 3, size=(T, D))
    wk = rng.integers(-2, 3, size=(D, d))
    wv = rng.integers(-2, 3, size=(D, d))

    def bits(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    k, v = O.kv_bridge(bits(h), bits(wk), bits(wv), row_block=5)
    exp_k = [[sum(int(h[r, i]) * int(wk[i, c]) for i in range(D)) for c in range(d)] for r in range(T)]
    exp_v = [[sum(int(h[r, i]) * int(wv[i, c]) for i in range(D)) for c in range(d)] for r in range(T)]
    assert np.array_equal(O.bf16_bits_to_f64(k), np.array(exp_k, dtype=np.float64))
    assert np.array_equal(O.bf16_bits_to_f64(v), np.array(exp_v, dtype=np.float64))
    # rounding of the sum: [1, 1] . [a, b] with a + b exactly halfway between bf16 values
    hh = bits(np.array([[1.0, 1.0]]))
    w = np.array([[1.0, 1.0 + 2.0 ** -7], [2.0 ** -8, 2.0 ** -8]])
    kk, _ = O.kv_bridge(hh, bits(w), bits(w))
    assert np.array_equal(O.bf16_bits_to_f64(kk)[0], np.array([1.0, 1.0 + 2.0 ** -6]))


def _block_beats(s, a, b, block):
    """Block a outranks block b: some member of a scores above every member of b, or neither
    block has such a member (equal maxima) and a comes first."""
    A = s[a * block: (a + 1) * block]
    Bm = s[b * block: (b + 1) * block]
    a_over = any(all(x > y for y in Bm) for x in A)
    b_over = any(all(y > x for x in A) for y in Bm)
    return a_over or (not b_over and a < b)


def check_block_selection(O):
    """Block-level selection from its definition: a block is kept iff fewer than k_b blocks
    outrank it (brute force, tiny inputs with many ties); block = 1 is token-level selection;
    a block with one important member is kept whole; the maximum, not the sum, ranks blocks;
    a short last block is cut at the candidate count."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        block = int(rng.choice([1, 2, 3, 4]))
        C = int(rng.integers(1, 14))
        s = rng.integers(0, 4, size=C).astype(np.float64)
        nb = -(-C // block)
        for kb in range(0, nb + 2):
            exp = [b for b in range(nb) if sum(1 for a in range(nb) if a != b and _block_beats(s, a, b, block)) < kb]
            got = O.select_blocks(s, kb, block)
            assert got.tolist() == exp, (s.tolist(), block, kb, got, exp)
            toks = O.expand_blocks(got, C, block)
            assert toks.tolist() == [j for b in exp for j in range(b * block, min(C, (b + 1) * block))]
        if block == 1:
            for kb in range(0, C + 2):
                assert np.array_equal(O.select_blocks(s, kb, 1), O.select_global(s, kb))
    # one important member keeps its whole group of 64
    s = np.full(64 * 40, 1e-4)
    s[64 * 17 + 5] = 0.9
    s[64 * 3: 64 * 4] = 0.5                    # a whole group of medium members
    assert O.select_blocks(s, 1, 64).tolist() == [17]      # the maximum ranks, not the sum (32.0)
    assert O.expand_blocks(O.select_blocks(s, 2, 64), s.shape[0], 64).tolist() == \
        list(range(64 * 3, 64 * 4)) + list(range(64 * 17, 64 * 18))
    # a short last block: C = 64 * 5 + 7, its best member is the last candidate
    s = np.zeros(64 * 5 + 7)
    s[-1] = 1.0
    assert O.select_blocks(s, 1, 64).tolist() == [5]
    assert O.expand_blocks([5], s.shape[0], 64).tolist() == list(range(320, 327))


def check_block_rows(O, k_b=16, block=64, W=128):
    """Whole rows on identical keys (all scores equal): the lowest blocks, the token layout of
    the indices (global budget k_b * block, then the window), for positions around the edges."""
    H, d = 2, 4
    for t in (0, 127, 128, 191, 192, 300, 1151, 1152, 1200, 1500):
        N = t + 1
        k = np.ones((N, d))
        v = np.arange(N * d, dtype=np.float64).reshape(N, d)
        q = np.ones((H, d))
        o, bid, idx, score = O.full_attn_select_blocks_row(q, k, v, t, 0.5, k_b, block, W)
        C = max(0, t - W + 1)
        nb = -(-C // block)
        assert bid.tolist() == list(range(min(k_b, nb))) + [-1] * (k_b - min(k_b, nb))
        g = list(range(min(C, k_b * block)))
        win = list(range(max(0, t - W + 1), t + 1))
        assert idx.tolist() == g + [-1] * (k_b * block - len(g)) + win + [-1] * (W - len(win))
        assert np.allclose(o, v.mean(axis=0)[None, :], rtol=0, atol=1e-12)


def check_e4m3fn_encode(O):
    """The E4M3FN encoder against torch's float8_e4m3fn conversion (a library routine): every
    finite code value and its negative, every midpoint between neighbouring codes (ties to the
    even code), random fp32 values in range; values past 448 saturate to +-448."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = O.e4m3fn_bits_to_f64(codes)
    assert np.array_equal(O.e4m3fn_encode_rne(vals), codes)
    assert np.array_equal(O.e4m3fn_encode_rne(-vals[1:]), codes[1:] | 0x80)
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(12)
    rnd = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000))).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    for x in (mids, -mids, rnd.astype(np.float64)):
        ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(O.e4m3fn_encode_rne(x), ref)
    assert O.e4m3fn_encode_rne(np.array([448.5, 1e6, -470.0])).tolist() == [0x7E, 0x7E, 0xFE]


def check_bridge_fp8(O):
    """Multi-target FP8 bridge: the codes equal torch's E4M3FN conversion of x / scale computed in
    fp32 from an independent float64 product; every non-zero row reaches +-448; the decoded value is
    within half an E4M3 step of the exact product; a zero row gets scale 1 and zero codes; a target
    whose Wk is another target's Wv reproduces that V."""
    rng = np.random.default_rng(13)
    T, D, d = 41, 64, 16

    def bits(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def dec(u):
        return torch.from_numpy(u.view(np.int16)).view(torch.bfloat16).double().numpy()

    h = bits(rng.standard_normal((T, D)))
    h[5] = 0
    wk = [bits(rng.standard_normal((d, D)) * 0.05) for _ in range(2)]
    wv = [bits(rng.standard_normal((d, D)) * 0.05) for _ in range(2)]
    wk[1] = wv[0].copy()
    out = O.kv_bridge_fp8(h, wk, wv, row_block=16)
    assert len(out) == 2
    for tgt in range(2):
        for (codes, scale), w in (((out[tgt][0], out[tgt][1]), wk[tgt]), ((out[tgt][2], out[tgt][3]), wv[tgt])):
            x = torch.from_numpy(dec(h)) @ torch.from_numpy(dec(w)).T          # float64
            x32 = x.float()
            amax = x32.abs().amax(dim=1)
            sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
            ref = (x32 / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes, ref)
            assert np.array_equal(scale, sc.numpy())
            mags = np.max(codes & 0x7F, axis=1)
            nz = amax.numpy() > 0
            assert np.all(mags[nz] == 0x7E) and np.all(codes[~nz] == 0) and np.all(scale[~nz] == 1.0)
            val = O.e4m3fn_bits_to_f64(codes) * scale.astype(np.float64)[:, None]
            ex = x.numpy()
            a = np.abs(ex) / scale.astype(np.float64)[:, None]
            step = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
            assert np.all(np.abs(val - ex) <= (0.5 * step + 1e-6 * a) * scale.astype(np.float64)[:, None] + 1e-12)
    assert np.array_equal(out[1][0], out[0][2]) and np.array_equal(out[1][1], out[0][3])


ALL_CHECKS = [check_dense_vs_sdpa, check_identical_keys, check_score_mass, check_onehot_keys,
              check_selection_bruteforce, check_selection_exhaustive, check_window_enumeration,
              check_sparse_identity, check_sparse_order_invariance, check_needles, check_bf16,
              check_e4m3fn, check_bridge, check_block_selection, check_block_rows,
              check_e4m3fn_encode, check_bridge_fp8]
