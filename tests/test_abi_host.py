"""CPU: the C-ABI library loads, exports every function include/hs2.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

import token_level_sparse_mqa_amd as hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000        # never dereferenced: validation fails before any launch


def _declared():
    src = open(os.path.join(ROOT, "include", "hs2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs2_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = hs2.lib()
    names = _declared()
    assert {"hs2_kv_bridge", "hs2_full_attn_select", "hs2_sparse_attn",
            "hs2_full_attn_select_workspace_size", "hs2_last_error", "hs2_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in hs2.hs2_version()


def _fas(**kw):
    a = dict(q=FAKE, qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, qp=FAKE, kl=FAKE,
             B=1, Tq=1, H=32, d=128, N=4096, kg=1024, W=128, sm=0.088, o=FAKE, idx=FAKE, dbg=None,
             ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return hs2.lib().hs2_full_attn_select(a["q"], a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["qp"],
                                          a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["kg"], a["W"],
                                          a["sm"], a["o"], a["idx"], a["dbg"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), hs2.HS2_ERR_UNSUPPORTED),
    (dict(H=33), hs2.HS2_ERR_UNSUPPORTED),
    (dict(H=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(qd=hs2.HS2_F32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(kvd=hs2.HS2_FP8_E4M3), hs2.HS2_ERR_INVALID_ARG),            # scales missing
    (dict(ks=FAKE, vs=FAKE), hs2.HS2_ERR_INVALID_ARG),               # scales on a bf16 cache
    (dict(kg=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(kg=5000), hs2.HS2_ERR_INVALID_ARG),
    (dict(W=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(sm=0.0), hs2.HS2_ERR_INVALID_ARG),
    (dict(sm=float("inf")), hs2.HS2_ERR_INVALID_ARG),
    (dict(q=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(idx=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(qp=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=1024), hs2.HS2_ERR_WORKSPACE),
    (dict(B=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(N=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), hs2.HS2_ERR_INVALID_ARG),     # misaligned pointers
    (dict(k=FAKE + 4), hs2.HS2_ERR_INVALID_ARG),
    (dict(o=FAKE + 4), hs2.HS2_ERR_INVALID_ARG),
    (dict(idx=FAKE + 2), hs2.HS2_ERR_INVALID_ARG),
    (dict(kl=FAKE + 1), hs2.HS2_ERR_INVALID_ARG),
    (dict(ws=FAKE + 8), hs2.HS2_ERR_INVALID_ARG),
])
def test_full_attn_select_rejects(kw, status):
    assert _fas(**kw) == status
    assert hs2.hs2_last_error()


def test_empty_batch_returns_ok_without_launch():
    assert _fas(B=0, q=None, k=None, v=None, o=None, idx=None, ws=None) == hs2.HS2_OK
    assert _fas(Tq=0) == hs2.HS2_OK


def test_workspace_size():
    n = hs2.hs2_full_attn_select_workspace_size(8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16)
    # at least the fp32 score rows of every query
    assert n >= 8 * 131072 * 4
    assert hs2.hs2_full_attn_select_workspace_size(1, 1, 32, 96, 100, 1024, 128, hs2.HS2_BF16) == 0
    assert hs2.hs2_full_attn_select_workspace_size(1, 1, 32, 128, 100, 0, 128, hs2.HS2_BF16) == 0
    # monotone in the sizes it is given
    a = hs2.hs2_full_attn_select_workspace_size(1, 16, 16, 64, 4096, 1024, 128, hs2.HS2_F32)
    b = hs2.hs2_full_attn_select_workspace_size(1, 16, 16, 64, 8192, 1024, 128, hs2.HS2_F32)
    assert 0 < a < b


def _sp(**kw):
    a = dict(q=FAKE, qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, idx=FAKE, S=1152,
             kl=None, B=1, Tq=1, H=32, d=128, N=4096, sm=0.088, o=FAKE, ws=None, wsb=0, stream=None)
    a.update(kw)
    return hs2.lib().hs2_sparse_attn(a["q"], a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["idx"],
                                     a["S"], a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["sm"], a["o"],
                                     a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(S=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(S=9000), hs2.HS2_ERR_INVALID_ARG),
    (dict(idx=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(d=32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(kvd=hs2.HS2_F32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(o=None), hs2.HS2_ERR_INVALID_ARG),
])
def test_sparse_rejects(kw, status):
    assert _sp(**kw) == status


def _fasb(**kw):
    a = dict(q=FAKE, qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, qp=FAKE, kl=FAKE,
             B=1, Tq=1, H=32, d=128, N=4096, kb=16, blk=64, W=128, sm=0.088, o=FAKE, bidx=FAKE, idx=FAKE,
             dbg=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return hs2.lib().hs2_full_attn_select_blocks(a["q"], a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"],
                                                 a["qp"], a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["kb"],
                                                 a["blk"], a["W"], a["sm"], a["o"], a["bidx"], a["idx"], a["dbg"],
                                                 a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(blk=3), hs2.HS2_ERR_INVALID_ARG),              # not a power of two
    (dict(blk=128), hs2.HS2_ERR_INVALID_ARG),            # above 64
    (dict(blk=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(kb=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(kb=65), hs2.HS2_ERR_INVALID_ARG),              # 65 * 64 > 4096
    (dict(N=(16384 * 64) + 1), hs2.HS2_ERR_UNSUPPORTED), # more than 16384 blocks per row
    (dict(blk=1, N=16385), hs2.HS2_ERR_UNSUPPORTED),
    (dict(bidx=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(bidx=FAKE + 2), hs2.HS2_ERR_INVALID_ARG),
    (dict(W=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(d=96), hs2.HS2_ERR_UNSUPPORTED),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=4096), hs2.HS2_ERR_WORKSPACE),
    (dict(B=0, q=None, k=None, v=None, o=None, idx=None, bidx=None, ws=None), hs2.HS2_OK),
])
def test_full_attn_select_blocks_rejects(kw, status):
    assert _fasb(**kw) == status
    if status != hs2.HS2_OK:
        assert hs2.hs2_last_error()


def test_blocks_workspace_size():
    tok = hs2.hs2_full_attn_select_workspace_size(8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16)
    blk = hs2.hs2_full_attn_select_blocks_workspace_size(8, 1, 32, 128, 131072, 16, 64, 128, hs2.HS2_BF16)
    # the token-level plan plus the block maxima [R, Nmax / 64] fp32
    assert blk >= tok + 8 * 2048 * 4
    assert hs2.hs2_full_attn_select_blocks_workspace_size(8, 1, 32, 128, 131072, 16, 48, 128, hs2.HS2_BF16) == 0
    assert hs2.hs2_full_attn_select_blocks_workspace_size(1, 1, 32, 128, 1 << 21, 16, 64, 128, hs2.HS2_BF16) == 0


def _spl(L=3, qarr=True, oarr=True, **kw):
    a = dict(qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, idx=FAKE, S=1152,
             kl=None, B=1, Tq=1, H=32, d=128, N=4096, sm=0.088, ws=None, wsb=0, stream=None)
    a.update(kw)
    n = max(L, 1)
    qa = ctypes.cast((ctypes.c_void_p * n)(*([kw.get("q", FAKE)] * n)), ctypes.c_void_p) if qarr else None
    oa = ctypes.cast((ctypes.c_void_p * n)(*([kw.get("o", FAKE)] * n)), ctypes.c_void_p) if oarr else None
    return hs2.lib().hs2_sparse_attn_layers(qa, L, a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["idx"],
                                            a["S"], a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["sm"], oa,
                                            a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(L=9), hs2.HS2_ERR_INVALID_ARG),
    (dict(qarr=False), hs2.HS2_ERR_INVALID_ARG),
    (dict(oarr=False), hs2.HS2_ERR_INVALID_ARG),
    (dict(q=None), hs2.HS2_ERR_INVALID_ARG),          # a null layer query
    (dict(o=None), hs2.HS2_ERR_INVALID_ARG),          # a null layer output
    (dict(S=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(d=32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(B=0), hs2.HS2_OK),                          # empty batch: nothing launched
    (dict(v=FAKE + 8), hs2.HS2_ERR_INVALID_ARG),      # misaligned pointers
    (dict(idx=FAKE + 2), hs2.HS2_ERR_INVALID_ARG),
])
def test_sparse_layers_rejects(kw, status):
    assert _spl(**kw) == status


def test_sparse_layers_workspace_size():
    one = hs2.hs2_sparse_attn_workspace_size(8, 1, 32, 128, 1152)
    assert one > 0
    assert hs2.hs2_sparse_attn_layers_workspace_size(8, 1, 32, 128, 1152, 3) == 3 * one
    assert hs2.hs2_sparse_attn_layers_workspace_size(8, 1, 32, 128, 1152, 0) == 0
    assert hs2.hs2_sparse_attn_layers_workspace_size(8, 1, 32, 128, 1152, 9) == 0


@pytest.mark.parametrize("args,status", [
    ((FAKE, 10, 100, FAKE, FAKE, 128, FAKE, FAKE, 128, None), hs2.HS2_ERR_INVALID_ARG),   # D % 64
    ((FAKE, 10, 128, FAKE, FAKE, 96, FAKE, FAKE, 128, None), hs2.HS2_ERR_UNSUPPORTED),
    ((FAKE, 10, 128, FAKE, FAKE, 128, FAKE, FAKE, 64, None), hs2.HS2_ERR_INVALID_ARG),    # stride < d
    ((None, 10, 128, FAKE, FAKE, 128, FAKE, FAKE, 128, None), hs2.HS2_ERR_INVALID_ARG),
    ((None, 0, 128, None, None, 128, None, None, 128, None), hs2.HS2_OK),                 # T == 0
    ((FAKE + 8, 10, 128, FAKE, FAKE, 128, FAKE, FAKE, 128, None), hs2.HS2_ERR_INVALID_ARG),  # hidden alignment
    ((FAKE, 10, 128, FAKE, FAKE + 2, 128, FAKE, FAKE, 128, None), hs2.HS2_ERR_INVALID_ARG),  # w_v alignment
    ((FAKE, 10, 128, FAKE, FAKE, 128, FAKE + 1, FAKE, 128, None), hs2.HS2_ERR_INVALID_ARG),  # k_out alignment
])
def test_bridge_rejects(args, status):
    assert hs2.lib().hs2_kv_bridge(*args) == status


def _b8(T=10, D=128, L=2, d=128, stride=128, hidden=FAKE, arrays=True, **slot):
    def arr(v):
        return ctypes.cast((ctypes.c_void_p * max(L, 1))(*([v] * max(L, 1))), ctypes.c_void_p) if arrays else None
    return hs2.lib().hs2_kv_bridge_fp8(hidden, T, D, arr(slot.get("wk", FAKE)), arr(slot.get("wv", FAKE)), L, d,
                                       arr(slot.get("ko", FAKE)), arr(slot.get("vo", FAKE)),
                                       arr(slot.get("ks", FAKE)), arr(slot.get("vs", FAKE)), stride, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(L=9), hs2.HS2_ERR_INVALID_ARG),
    (dict(D=100), hs2.HS2_ERR_INVALID_ARG),
    (dict(d=96, stride=96), hs2.HS2_ERR_UNSUPPORTED),
    (dict(stride=64), hs2.HS2_ERR_INVALID_ARG),
    (dict(arrays=False), hs2.HS2_ERR_INVALID_ARG),
    (dict(hidden=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(hidden=FAKE + 8), hs2.HS2_ERR_INVALID_ARG),
    (dict(wk=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(wv=FAKE + 2), hs2.HS2_ERR_INVALID_ARG),
    (dict(ks=FAKE + 2), hs2.HS2_ERR_INVALID_ARG),
    (dict(T=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(T=0, hidden=None), hs2.HS2_OK),
])
def test_bridge_fp8_rejects(kw, status):
    assert _b8(**kw) == status


def _db(L=2, qarr=True, oarr=True, **kw):
    a = dict(q=FAKE, qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, qp=FAKE, kl=FAKE,
             B=1, Tq=1, H=32, d=128, N=4096, kg=1024, W=128, sm=0.088, o=FAKE, idx=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    n = max(L, 1)
    qa = ctypes.cast((ctypes.c_void_p * n)(*([kw.get("qs", FAKE)] * n)), ctypes.c_void_p) if qarr else None
    oa = ctypes.cast((ctypes.c_void_p * n)(*([kw.get("os", FAKE)] * n)), ctypes.c_void_p) if oarr else None
    return hs2.lib().hs2_decode_block(a["q"], qa, L, a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"], a["qp"],
                                      a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["kg"], a["W"], a["sm"],
                                      a["o"], a["idx"], oa, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Tq=8), hs2.HS2_ERR_UNSUPPORTED),            # query chunks: the separate calls
    (dict(qd=hs2.HS2_F32, kvd=hs2.HS2_F32), hs2.HS2_ERR_UNSUPPORTED),
    (dict(L=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(L=9), hs2.HS2_ERR_INVALID_ARG),
    (dict(qarr=False), hs2.HS2_ERR_INVALID_ARG),
    (dict(oarr=False), hs2.HS2_ERR_INVALID_ARG),
    (dict(qs=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(os=FAKE + 4), hs2.HS2_ERR_INVALID_ARG),
    (dict(B=300, kg=2048, W=128), hs2.HS2_ERR_UNSUPPORTED),    # unsplit rows of 2176 entries
    (dict(idx=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(ws=None), hs2.HS2_ERR_WORKSPACE),
    (dict(wsb=1024), hs2.HS2_ERR_WORKSPACE),
    (dict(B=0), hs2.HS2_OK),
])
def test_decode_block_rejects(kw, status):
    assert _db(**kw) == status


def test_decode_block_workspace_size():
    full = hs2.hs2_full_attn_select_workspace_size(8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16)
    both = hs2.hs2_decode_block_workspace_size(8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16, 3)
    # the token-level plan plus the sparse layers' split partials (3 layers x 8 rows x 9 splits x 32 heads)
    assert both >= full + 3 * 8 * 9 * 32 * 130 * 4
    assert hs2.hs2_decode_block_workspace_size(8, 8, 32, 128, 131072, 1024, 128, hs2.HS2_BF16, 3) == 0
    assert hs2.hs2_decode_block_workspace_size(8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16, 0) == 0


def test_select_cache_length_limit():
    """Calls that select take at most HS2_MAX_SELECT_NMAX rows per sequence (one selection grid row
    per 4096-key segment): above it they refuse before launching anything, and their size
    queries return 0."""
    big = hs2.HS2_MAX_SELECT_NMAX
    assert hs2.hs2_full_attn_select_workspace_size(1, 1, 32, 128, big, 1024, 128, hs2.HS2_BF16) > big * 4
    assert hs2.hs2_full_attn_select_workspace_size(1, 1, 32, 128, big + 1, 1024, 128, hs2.HS2_BF16) == 0
    assert hs2.hs2_decode_block_workspace_size(1, 1, 32, 128, big + 1, 1024, 128, hs2.HS2_BF16, 3) == 0
    assert _fas(N=big + 1) == hs2.HS2_ERR_UNSUPPORTED
    assert "selection supports" in hs2.hs2_last_error()
    assert _db(N=big + 1) == hs2.HS2_ERR_UNSUPPORTED


def _need(fn, **kw):
    """The exact workspace a call plans, read from its HS2_ERR_WORKSPACE message (a one-byte
    workspace is refused on the host, before anything is launched)."""
    assert fn(wsb=1, **kw) == hs2.HS2_ERR_WORKSPACE
    m = re.search(r"workspace of (\d+) bytes needed", hs2.hs2_last_error())
    assert m, hs2.hs2_last_error()
    return int(m.group(1))


@pytest.mark.parametrize("kvd,row_bytes", [(hs2.HS2_BF16, 256), (hs2.HS2_FP8_E4M3, 128)])
def test_long_chunk_takes_row_kernels(kvd, row_bytes):
    """Query chunks whose cache spans more than 2^31 bytes per sequence leave the chunk kernels
    (32-bit offsets) for the row kernels.  The chunk kernels' plan holds the sequence's V^T
    images (d rows of 80 bytes per 32 keys, whole 64-key stages); the row kernels' plan drops
    them and adds their key splits' partial results: 8 rows x 96 splits x 32 heads x (d + 2)
    floats (about 768 workgroups over the 8 rows)."""
    fit = (1 << 31) // row_bytes - 1                 # the largest cache the chunk kernels take
    ks = vs = FAKE if kvd == hs2.HS2_FP8_E4M3 else None
    a = _need(_fas, Tq=8, N=fit, kvd=kvd, ks=ks, vs=vs)
    b = _need(_fas, Tq=8, N=fit + 128, kvd=kvd, ks=ks, vs=vs)
    scores_growth = 8 * 128 * 4
    vt_images = 2 * ((fit + 63) // 64) * 128 * 80
    assert a > vt_images
    assert b - a >= scores_growth + 8 * 96 * 32 * 130 * 4 - vt_images
    assert b - a <= scores_growth + 8 * 96 * 32 * 130 * 4 - vt_images + (1 << 12)
    # decode rows take the row kernels at every length: no jump there
    c = _need(_fas, Tq=4, N=fit, kvd=kvd, ks=ks, vs=vs)
    e = _need(_fas, Tq=4, N=fit + 128, kvd=kvd, ks=ks, vs=vs)
    assert 0 <= e - c < 1 << 20


@pytest.mark.parametrize("kvd", [hs2.HS2_BF16, hs2.HS2_FP8_E4M3])
def test_chunk_size_covers_decode_calls(kvd):
    """A size queried for a query chunk (chunk kernels, no split partials) also covers every decode
    call with fewer query tokens (row kernels, split partials) at the same cache length."""
    ks = vs = FAKE if kvd == hs2.HS2_FP8_E4M3 else None
    for B in (1, 3):
        size = hs2.hs2_full_attn_select_workspace_size(B, 8, 32, 128, 131072, 1024, 128, kvd)
        for b in range(1, B + 1):
            for tq in range(1, 9):
                assert _need(_fas, B=b, Tq=tq, N=131072, kvd=kvd, ks=ks, vs=vs) <= size, (B, b, tq)


def test_workspace_sizes_cover_smaller_calls():
    """Property: for random sizes, the queried workspace is at least the exact plan of every call
    with no larger sizes (B, Tq, H, d, Nmax, k, window, L) and the same KV dtype."""
    import random
    rng = random.Random(20261203)
    for _ in range(150):
        kvd = rng.choice([hs2.HS2_F32, hs2.HS2_BF16, hs2.HS2_FP8_E4M3])
        qd = hs2.HS2_F32 if kvd == hs2.HS2_F32 else hs2.HS2_BF16
        ks = vs = FAKE if kvd == hs2.HS2_FP8_E4M3 else None
        B, Tq = rng.randint(1, 12), rng.randint(1, 40)
        H, d = rng.randint(1, 32), rng.choice([64, 128])
        N, kg, W = rng.randint(1, 300000), rng.randint(1, 4096), rng.randint(0, 512)
        size = hs2.hs2_full_attn_select_workspace_size(B, Tq, H, d, N, kg, W, kvd)
        bsz = hs2.hs2_full_attn_select_blocks_workspace_size(B, Tq, H, d, N, max(1, kg // 64), 64, W, kvd)
        for _ in range(6):
            b, tq, h = rng.randint(1, B), rng.randint(1, Tq), rng.randint(1, H)
            dd = rng.choice([64, d]) if d == 128 else 64
            n, k = rng.randint(1, N), rng.randint(1, kg)
            assert _need(_fas, B=b, Tq=tq, H=h, d=dd, N=n, kg=k, W=W, qd=qd, kvd=kvd, ks=ks, vs=vs) <= size
            if bsz:
                kb = max(1, k // 64)
                if kb <= max(1, kg // 64):
                    assert _need(_fasb, B=b, Tq=tq, H=h, d=dd, N=n, kb=kb, W=W, qd=qd, kvd=kvd, ks=ks, vs=vs) <= bsz
        if qd == hs2.HS2_BF16 and Tq < 8 and kg + W <= 1152:
            L = rng.randint(1, 8)
            dsz = hs2.hs2_decode_block_workspace_size(B, Tq, H, d, N, kg, W, kvd, L)
            for _ in range(4):
                b, tq, h, n = rng.randint(1, B), rng.randint(1, Tq), rng.randint(1, H), rng.randint(1, N)
                k, l = rng.randint(1, kg), rng.randint(1, L)
                assert _need(_db, L=l, B=b, Tq=tq, H=h, d=d, N=n, kg=k, W=W, kvd=kvd, ks=ks, vs=vs) <= dsz


def _fna(**kw):
    a = dict(q=FAKE, qd=hs2.HS2_BF16, k=FAKE, v=FAKE, kvd=hs2.HS2_BF16, ks=None, vs=None, qp=FAKE, kl=FAKE,
             B=1, Tq=1, H=32, d=128, N=4096, kg=1024, W=128, sm=0.088, o=FAKE, idx=FAKE, dbg=None, stream=None)
    a.update(kw)
    return hs2.lib().hs2_full_attn_select_noalloc(a["q"], a["qd"], a["k"], a["v"], a["kvd"], a["ks"], a["vs"],
                                                  a["qp"], a["kl"], a["B"], a["Tq"], a["H"], a["d"], a["N"], a["kg"],
                                                  a["W"], a["sm"], a["o"], a["idx"], a["dbg"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), hs2.HS2_ERR_UNSUPPORTED),
    (dict(kg=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(idx=None), hs2.HS2_ERR_INVALID_ARG),
    (dict(o=FAKE + 4), hs2.HS2_ERR_INVALID_ARG),
    (dict(B=0), hs2.HS2_OK),
    # more workspace than the static scratch holds: refused before anything is enqueued
    (dict(B=256, N=131072), hs2.HS2_ERR_WORKSPACE),
    (dict(B=1, Tq=4096, N=69632), hs2.HS2_ERR_WORKSPACE),
])
def test_noalloc_rejects(kw, status):
    assert _fna(**kw) == status
    if status == hs2.HS2_ERR_WORKSPACE:
        assert "static scratch holds" in hs2.hs2_last_error()


def test_noalloc_limit_is_the_workspace_size():
    """The static scratch takes every call whose workspace size is within HS2_NOALLOC_SCRATCH_BYTES:
    decode128k (8 x 131072 keys) and decode1m_fp8 fit; 64 sequences of 131072 keys fit too."""
    cap = hs2.HS2_NOALLOC_SCRATCH_BYTES
    assert cap == 64 << 20
    for args in ((8, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16), (1, 1, 32, 128, 1 << 20, 1024, 128, hs2.HS2_FP8_E4M3),
                 (64, 1, 32, 128, 131072, 1024, 128, hs2.HS2_BF16)):
        assert 0 < hs2.hs2_full_attn_select_workspace_size(*args) <= cap
