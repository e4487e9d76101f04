"""The slice-bucketed layout (VQ_LAYOUT_BUCKETED) on the host: sizes, the packer and the
validation of the calls that take it, with no GPU.

The packer is checked by reading its output back with a decoder written here from the
layout's definition in include/vq.h (prefix table of bucket offsets, one 32-bit word per
vector: position in its 1024-vector chunk, idx1 & 8191, idx2), and recovering every
index of the original tensors; the zero padding and the prefix table's consistency are
checked on the way.  The order of words inside a bucket is the packer's choice (it lines
the main-book reads up with the LDS banks): checked to be deterministic and to place most
words where the column group of their main index matches that of their lane.
"""
import ctypes

import numpy as np
import pytest

import synth

CHUNK = 1024


@pytest.fixture(scope="module")
def vq():
    import os

    import gemv_bit_unpack_amd as g

    if not os.path.exists(g.LIB_PATH):
        from gemv_bit_unpack_amd import build

        build.build()
    g.lib()
    return g


def _desc(vq, n, i, b2=8, layout=2):
    return vq.make_desc(n, i, 8, 16, b2, layout)


def _header_bytes(n, i):
    nv = i // 8
    chunks = -(-nv // CHUNK)
    return -(-(4 * (8 * chunks * n + 1)) // 256) * 256


def decode(packed: np.ndarray, n: int, i: int, b2: int):
    """idx1, idx2 [N, nv] back from a slice-bucketed buffer (asserting its invariants)."""
    nv = i // 8
    chunks = -(-nv // CHUNK)
    nb = 8 * chunks * n
    hb = _header_bytes(n, i)
    assert packed.size == hb + 4 * n * nv
    start = packed[: 4 * (nb + 1)].view(np.uint32).astype(np.int64)
    assert (packed[4 * (nb + 1): hb] == 0).all(), "header padding is zero"
    assert start[0] == 0 and start[-1] == n * nv and (np.diff(start) >= 0).all()
    words = packed[hb:].view(np.uint32)
    assert ((words >> 31) == 0).all()
    idx1 = np.full((n, nv), -1, dtype=np.int64)
    idx2 = np.full((n, nv), -1, dtype=np.int64)
    for c in range(chunks):
        for s in range(8):
            for o in range(n):
                b = (c * 8 + s) * n + o
                wd = words[start[b]:start[b + 1]].astype(np.int64)
                pos = wd & 0x3FF
                assert np.unique(pos).size == pos.size, "each position once in a bucket"
                j = c * CHUNK + pos
                assert (j < nv).all()
                assert (idx1[o, j] == -1).all(), "each vector once"
                idx1[o, j] = (s << 13) | ((wd >> 10) & 0x1FFF)
                idx2[o, j] = (wd >> 23) & 0xFF
    assert (idx1 >= 0).all(), "every vector present"
    if b2 == 0:
        assert (idx2 == 0).all()
    return idx1, idx2


@pytest.mark.parametrize("n,i,b2", [
    (1, 8, 8), (3, 8192, 8), (7, 8200, 0), (64, 16384, 8), (65, 1024, 8), (130, 24, 0), (5, 28672, 8),
])
def test_bucketed_pack_round_trip(vq, n, i, b2):
    lay = synth.make_layer(n, i, 8, 16, b2, wid=70, copy=n + i)
    d = _desc(vq, n, i, b2)
    assert vq.packed_bytes(d) == _header_bytes(n, i) + 4 * n * (i // 8)
    p = vq.pack(d, lay["idx1"], lay["idx2"])
    idx1, idx2 = decode(p, n, i, b2)
    assert np.array_equal(idx1, lay["idx1"].astype(np.int64))
    if b2:
        assert np.array_equal(idx2, lay["idx2"].astype(np.int64))


def test_bucketed_pack_skewed_slices(vq):
    """Rows whose indices all fall in one slice, and rows that leave most buckets empty."""
    n, i = 12, 8 * 2500
    nv = i // 8
    g = np.random.default_rng(3)
    idx1 = g.integers(0, 1 << 16, (n, nv), dtype=np.uint32)
    idx1[0] = 5 << 13 | g.integers(0, 8192, nv, dtype=np.uint32)       # all in slice 5
    idx1[1] = 0                                                        # all index 0
    idx1[2] = 65535
    idx1[3, :1500] = 7 << 13                                           # half one slice
    idx2 = g.integers(0, 256, (n, nv), dtype=np.uint32)
    d = _desc(vq, n, i, 8)
    p = vq.pack(d, idx1, idx2)
    r1, r2 = decode(p, n, i, 8)
    assert np.array_equal(r1, idx1.astype(np.int64)) and np.array_equal(r2, idx2.astype(np.int64))
    start = p[: 4 * (8 * 3 * n + 1)].view(np.uint32)
    # row 0, chunk 0: every one of its 1024 vectors in bucket (0, 5, 0)
    b = (0 * 8 + 5) * n + 0
    assert start[b + 1] - start[b] == CHUNK


def test_bucketed_pack_matches_workload_rows(vq):
    """The 70B-class down layer's first rows (3.5 chunks per row) survive the round trip."""
    lay = synth.workload_layer("l70b", 1)
    n, i = 40, lay["in_features"]
    idx1, idx2 = lay["idx1"][:n], lay["idx2"][:n]
    p = vq.pack(_desc(vq, n, i, 8), idx1, idx2)
    r1, r2 = decode(p, n, i, 8)
    assert np.array_equal(r1, idx1.astype(np.int64)) and np.array_equal(r2, idx2.astype(np.int64))


@pytest.mark.parametrize("fields", [
    dict(v=6), dict(bits1=12), dict(bits2=4), dict(bits2=16), dict(in_features=8196), dict(v=16),
])
def test_bucketed_layout_defined_only_for_its_shapes(vq, fields):
    base = dict(out_features=64, in_features=8192, v=8, bits1=16, bits2=8, layout=2)
    base.update(fields)
    d = vq.Desc(**base)
    n = ctypes.c_size_t(77)
    assert vq.lib().vq_packed_bytes(ctypes.byref(d), ctypes.byref(n)) == vq.VQ_ERR_UNSUPPORTED
    assert n.value == 77


def test_bucketed_pack_errors(vq):
    d = _desc(vq, 2, 16, 8)
    nb = vq.packed_bytes(d)
    good = np.array([[1, 65535], [8192, 5]], dtype=np.uint32)
    bad2 = np.array([[1, 256], [0, 5]], dtype=np.uint32)
    out = np.full(nb, 0xAB, dtype=np.uint8)
    f = vq.lib().vq_pack
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert f(ctypes.byref(d), vp(good), vp(bad2), vp(out), nb) == vq.VQ_ERR_INDEX_RANGE
    assert (out == 0xAB).all()
    assert f(ctypes.byref(d), vp(good), vp(good), vp(out), nb - 1) == vq.VQ_ERR_BUFFER_SIZE
    assert (out == 0xAB).all()
    assert f(ctypes.byref(d), vp(good), None, vp(out), nb) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), vp(good), vp(good % 256), vp(out), nb) == vq.VQ_OK


def _ws_bytes(vq, desc, m, xt):
    n = ctypes.c_size_t(12345)
    st = vq.lib().vq_gemv_workspace_bytes(ctypes.byref(desc), m, xt, ctypes.byref(n))
    return st, int(n.value)


def test_bucketed_workspace_bytes(vq):
    d = _desc(vq, 8192, 28672)  # 3.5 chunks per row: 4 chunks
    st, b = _ws_bytes(vq, d, 1, vq.VQ_BF16)
    assert st == vq.VQ_OK and b == -(-(8 * 4 * 8192 * 4) // 256) * 256 + 256
    assert _ws_bytes(vq, d, 1, vq.VQ_F16) == (vq.VQ_OK, b)
    assert _ws_bytes(vq, d, 0, vq.VQ_F16) == (vq.VQ_OK, 0)
    assert _ws_bytes(vq, d, 2, vq.VQ_F16) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _ws_bytes(vq, d, 17, vq.VQ_F16) == (vq.VQ_ERR_SHAPE, 12345)
    assert _ws_bytes(vq, d, 1, vq.VQ_F32) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _ws_bytes(vq, _desc(vq, 8192, 0), 1, vq.VQ_F16) == (vq.VQ_OK, 0)
    # small shapes have the path too (there is no other for this layout)
    assert _ws_bytes(vq, _desc(vq, 1, 8), 1, vq.VQ_F16)[1] > 0


P = ctypes.c_void_p(0x10000)


def _call(vq, fn, desc, ws=P, ws_bytes=1 << 30, packed=P, cb1=P, cb2=P, x=P, xt=1, m=1, y=P, yt=2):
    f = getattr(vq.lib(), fn)
    if fn == "vq_gemv_ws":
        return f(ctypes.byref(desc), packed, cb1, cb2, None, None, x, xt, m, y, yt, ws, ws_bytes, None)
    return f(ctypes.byref(desc), packed, cb1, cb2, None, None, x, xt, m, y, yt, None)


@pytest.mark.parametrize("fn", ["vq_gemv_ws", "vq_gemv_noalloc"])
def test_bucketed_product_validation(vq, fn):
    d = _desc(vq, 4096, 8192)
    assert _call(vq, fn, d, m=2) == vq.VQ_ERR_UNSUPPORTED
    assert _call(vq, fn, d, m=17) == vq.VQ_ERR_SHAPE
    assert _call(vq, fn, d, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert _call(vq, fn, d, y=None) == vq.VQ_ERR_NULL
    assert _call(vq, fn, d, cb2=None) == vq.VQ_ERR_NULL
    for k in ("packed", "cb1", "cb2", "x"):
        assert _call(vq, fn, d, **{k: ctypes.c_void_p(0x10008)}) == vq.VQ_ERR_ALIGN, k
    assert _call(vq, fn, d, m=0, y=None, x=None, packed=None) == vq.VQ_OK
    if fn == "vq_gemv_ws":
        assert _call(vq, fn, d, ws=None) == vq.VQ_ERR_NULL
        need = _ws_bytes(vq, d, 1, vq.VQ_BF16)[1]
        assert _call(vq, fn, d, ws_bytes=need - 1) == vq.VQ_ERR_BUFFER_SIZE
        assert _call(vq, fn, d, ws=ctypes.c_void_p(0x10010)) == vq.VQ_ERR_ALIGN


def test_other_calls_refuse_the_bucketed_layout(vq):
    d = _desc(vq, 64, 8192)
    f = vq.lib()
    args = (ctypes.byref(d), P, P, P, None, None, P, 0, 1, P, 2)
    assert f.vq_gemv(*args, None) == vq.VQ_ERR_UNSUPPORTED
    assert f.vq_gemm(*args, None) == vq.VQ_ERR_UNSUPPORTED
    assert f.vq_gemm_ws(*args, P, 1 << 20, None) == vq.VQ_ERR_UNSUPPORTED
    assert f.vq_dequant(ctypes.byref(d), P, P, P, None, P, 2, None) == vq.VQ_ERR_UNSUPPORTED
    n = ctypes.c_size_t(0)
    assert f.vq_gemm_workspace_bytes(ctypes.byref(d), 32, 0, ctypes.byref(n)) == vq.VQ_ERR_UNSUPPORTED
    assert f.vq_rht_product_workspace_bytes(ctypes.byref(d), 1, 0, 0, ctypes.byref(n)) == vq.VQ_ERR_UNSUPPORTED
    assert f.vq_gemv_ws_rht(ctypes.byref(d), P, P, P, None, None, P, 0, 1, P, P, 2, P, 1 << 20,
                            None) == vq.VQ_ERR_UNSUPPORTED


def _quad_match(words):
    """Fraction of the words of a bucket whose main-index column group (bits [2, 4) of
    idx1) equals that of their slot (bits [2, 4) of the word's place in the bucket)."""
    k = np.arange(words.size)
    return float(np.mean(((words.astype(np.int64) >> 12) & 3) == ((k >> 2) & 3))) if words.size else 1.0


def test_bucketed_pack_lines_up_main_index_columns_deterministically(vq):
    n, i = 64, 8192
    lay = synth.make_layer(n, i, 8, 16, 8, wid=71)
    d = _desc(vq, n, i, 8)
    p1 = vq.pack(d, lay["idx1"], lay["idx2"])
    p2 = vq.pack(d, lay["idx1"], lay["idx2"])
    assert np.array_equal(p1, p2)
    nb = 8 * n
    start = p1[: 4 * (nb + 1)].view(np.uint32)
    words = p1[_header_bytes(n, i):].view(np.uint32)
    ours, plain = [], []
    for b in range(nb):
        wb = words[start[b]:start[b + 1]]
        ours.append(_quad_match(wb))
        plain.append(_quad_match(wb[np.argsort(wb & 0x3FF, kind="stable")]))  # ascending positions
    # position order matches a quarter of the slots by chance; the packer's order most of them
    assert np.mean(plain) < 0.35 and np.mean(ours) > 0.85, (np.mean(ours), np.mean(plain))


def test_bucketed_layout_size_limits(vq):
    """The product addresses the words and the prefix table with 32-bit offsets: a layer of
    2^29 or more vectors is refused by every call that takes the layout."""
    n = ctypes.c_size_t(77)
    big = _desc(vq, 1 << 19, 8192)  # 2^19 rows x 1024 vectors = 2^29 vectors
    assert vq.lib().vq_packed_bytes(ctypes.byref(big), ctypes.byref(n)) == vq.VQ_ERR_UNSUPPORTED
    assert _ws_bytes(vq, big, 1, vq.VQ_F16) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _call(vq, "vq_gemv_ws", big) == vq.VQ_ERR_UNSUPPORTED
    ok = _desc(vq, (1 << 19) - 8, 8192)  # just below: accepted
    assert vq.lib().vq_packed_bytes(ctypes.byref(ok), ctypes.byref(n)) == vq.VQ_OK
