"""The C ABI on the host (no GPU): symbols, sizes, the packer, and every validation
path that must return before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def vq():
    import gemv_bit_unpack_amd as g

    if not os.path.exists(g.LIB_PATH):
        from gemv_bit_unpack_amd import build

        build.build()
    g.lib()
    return g


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "vq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(vq):
    names = _declared_symbols()
    assert set(names) == set(vq.EXPORTED)
    for name in names:
        assert hasattr(vq.lib(), name), name
    assert vq.abi_version() == 1


def test_status_strings(vq):
    for code in range(-8, 1):
        s = vq.lib().vq_status_string(code).decode()
        assert s.startswith("VQ_")
    assert vq.lib().vq_status_string(-99).decode() == "unknown vq_status"


@pytest.mark.parametrize("n,i,v,b1,b2", [
    (256, 256, 8, 8, 0), (4096, 4096, 8, 16, 0), (4096, 4096, 8, 16, 8), (14336, 4096, 6, 12, 12),
    (4096, 14336, 6, 12, 12), (28672, 8192, 8, 16, 8), (8192, 28672, 8, 16, 8), (7, 13, 3, 5, 7),
    (1, 1, 1, 1, 0), (0, 64, 8, 8, 0), (64, 0, 8, 8, 8), (3, 1000, 16, 16, 16),
])
def test_packed_bytes_matches_oracle(vq, n, i, v, b1, b2):
    assert vq.packed_bytes(vq.make_desc(n, i, v, b1, b2)) == oracle.packed_bytes(n, i, v, b1, b2)


@pytest.mark.parametrize("n,i,v,b1,b2", [
    (3, 40, 8, 16, 8), (5, 37, 6, 12, 12), (2, 100, 3, 5, 0), (4, 64, 8, 8, 0), (1, 7, 1, 13, 3),
    (7, 200, 16, 16, 16), (9, 13, 4, 1, 2), (33, 300, 6, 12, 0), (17, 512, 8, 3, 0),
])
def test_pack_byte_equal_to_oracle(vq, n, i, v, b1, b2):
    lay = synth.make_layer(n, i, v, b1, b2, wid=60, copy=n)
    d = vq.make_desc(n, i, v, b1, b2)
    ours = vq.pack(d, lay["idx1"], lay["idx2"])
    ref = oracle.pack(n, i, v, b1, b2, lay["idx1"], lay["idx2"])
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("key", ["dec4k_res", "mlp8b", "l70b"])
def test_pack_workloads_row_sample_equal_to_oracle(vq, key):
    w = synth.WORKLOADS[key]
    for layer, (n, i) in enumerate(w.layers):
        lay = synth.workload_layer(key, layer)
        ours = vq.pack(vq.make_desc(n, i, w.v, w.bits1, w.bits2), lay["idx1"], lay["idx2"])
        rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(layer).integers(0, n, 30)]))
        sub2 = lay["idx2"][rows] if w.bits2 else None
        ref = oracle.pack(rows.size, i, w.v, w.bits1, w.bits2, lay["idx1"][rows], sub2)
        s1 = oracle.row_stride(i, w.v, w.bits1)
        s2 = oracle.row_stride(i, w.v, w.bits2)
        mine1 = ours[: n * s1].reshape(n, s1)[rows].reshape(-1)
        assert np.array_equal(mine1, ref[: rows.size * s1])
        if w.bits2:
            mine2 = ours[n * s1:].reshape(n, s2)[rows].reshape(-1)
            assert np.array_equal(mine2, ref[rows.size * s1:])


def _raw_pack(vq, desc, idx1, idx2, nbytes, out=None):
    out = np.full(max(nbytes, 16) + 16, 0xAB, dtype=np.uint8) if out is None else out
    st = vq.lib().vq_pack(ctypes.byref(desc) if desc is not None else None,
                          None if idx1 is None else idx1.ctypes.data_as(ctypes.c_void_p),
                          None if idx2 is None else idx2.ctypes.data_as(ctypes.c_void_p),
                          out.ctypes.data_as(ctypes.c_void_p), nbytes)
    return st, out


def test_pack_errors_leave_output_untouched(vq):
    d = vq.make_desc(2, 16, 8, 3, 0)
    good = np.array([[1, 7], [0, 5]], dtype=np.uint32)
    bad = np.array([[1, 8], [0, 5]], dtype=np.uint32)
    nb = vq.packed_bytes(d)
    st, out = _raw_pack(vq, d, bad, None, nb)
    assert st == vq.VQ_ERR_INDEX_RANGE and (out == 0xAB).all()
    st, out = _raw_pack(vq, d, good, None, nb - 1)
    assert st == vq.VQ_ERR_BUFFER_SIZE and (out == 0xAB).all()
    st, out = _raw_pack(vq, None, good, None, nb)
    assert st == vq.VQ_ERR_NULL and (out == 0xAB).all()
    st, out = _raw_pack(vq, vq.make_desc(2, 16, 8, 3, 2), good, None, 64)
    assert st == vq.VQ_ERR_NULL and (out == 0xAB).all()
    st, out = _raw_pack(vq, d, good, None, nb)
    assert st == vq.VQ_OK and not out[:nb].tolist() == [0xAB] * nb


@pytest.mark.parametrize("fields,code", [
    (dict(v=0), -3), (dict(v=17), -3), (dict(bits1=0), -3), (dict(bits1=17), -3), (dict(bits2=-1), -3),
    (dict(bits2=17), -3), (dict(out_features=-1), -2), (dict(in_features=-5), -2), (dict(layout=2), -4),
])
def test_descriptor_validation(vq, fields, code):
    base = dict(out_features=8, in_features=64, v=8, bits1=8, bits2=0, layout=1)
    base.update(fields)
    d = vq.Desc(**base)
    n = ctypes.c_size_t(0)
    assert vq.lib().vq_packed_bytes(ctypes.byref(d), ctypes.byref(n)) == code
    assert vq.lib().vq_packed_bytes(None, ctypes.byref(n)) == vq.VQ_ERR_NULL


# Fake, never-dereferenced device addresses: every call below must be refused on the host.
P = ctypes.c_void_p(0x10000)
P_MIS = ctypes.c_void_p(0x10002)


def _gemv(vq, fn, desc, packed=P, cb1=P, cb2=P, scale=None, bias=None, x=P, xt=0, m=1, y=P, yt=2):
    return getattr(vq.lib(), fn)(ctypes.byref(desc) if desc is not None else None, packed, cb1, cb2, scale, bias, x,
                                 xt, m, y, yt, None)


@pytest.mark.parametrize("fn", ["vq_gemv", "vq_gemm"])
def test_product_validation_paths(vq, fn):
    d = vq.make_desc(64, 64, 8, 8, 8)
    assert _gemv(vq, fn, None) == vq.VQ_ERR_NULL
    assert _gemv(vq, fn, vq.make_desc(64, 64, 8, 0, 0)) == vq.VQ_ERR_BITS
    assert _gemv(vq, fn, d, m=-1) == vq.VQ_ERR_SHAPE
    assert _gemv(vq, fn, d, xt=2) == vq.VQ_ERR_UNSUPPORTED  # fp32 activations are not an input type
    assert _gemv(vq, fn, d, yt=7) == vq.VQ_ERR_UNSUPPORTED
    assert _gemv(vq, fn, d, y=None) == vq.VQ_ERR_NULL
    assert _gemv(vq, fn, d, cb2=None) == vq.VQ_ERR_NULL
    assert _gemv(vq, fn, d, packed=None) == vq.VQ_ERR_NULL
    assert _gemv(vq, fn, d, x=None) == vq.VQ_ERR_NULL
    assert _gemv(vq, fn, d, packed=P_MIS) == vq.VQ_ERR_ALIGN
    assert _gemv(vq, fn, d, y=P_MIS, yt=2) == vq.VQ_ERR_ALIGN
    assert _gemv(vq, fn, d, x=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    assert _gemv(vq, fn, vq.Desc(64, 64, 8, 8, 8, 3)) == vq.VQ_ERR_UNSUPPORTED
    # nothing to do: no launch, no pointer needed
    assert _gemv(vq, fn, d, m=0, y=None, x=None, packed=None) == vq.VQ_OK
    assert _gemv(vq, fn, vq.make_desc(0, 64, 8, 8, 8), y=None, x=None, packed=None) == vq.VQ_OK
    if fn == "vq_gemv":
        assert _gemv(vq, fn, d, m=17) == vq.VQ_ERR_SHAPE


def test_dequant_validation_paths(vq):
    f = vq.lib().vq_dequant
    d = vq.make_desc(64, 64, 8, 8, 8)
    assert f(None, P, P, P, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), P, P, None, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), P, P, P, None, P, 9, None) == vq.VQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), P_MIS, P, P, None, P, 2, None) == vq.VQ_ERR_ALIGN
    assert f(ctypes.byref(d), P, P, P, None, P_MIS, 2, None) == vq.VQ_ERR_ALIGN
    assert f(ctypes.byref(vq.make_desc(64, 0, 8, 8, 8)), None, None, None, None, None, 2, None) == vq.VQ_OK


def _gemv_ws(vq, desc, ws=None, ws_bytes=0, packed=P, cb1=P, cb2=P, x=P, xt=0, m=1, y=P, yt=2):
    return vq.lib().vq_gemv_ws(ctypes.byref(desc) if desc is not None else None, packed, cb1, cb2, None, None, x, xt,
                               m, y, yt, ws, ws_bytes, None)


def _ws_bytes(vq, desc, m, xt):
    n = ctypes.c_size_t(12345)
    st = vq.lib().vq_gemv_workspace_bytes(ctypes.byref(desc) if desc is not None else None, m, xt, ctypes.byref(n))
    return st, int(n.value)


def test_gemv_workspace_bytes(vq):
    big = vq.make_desc(8192, 4096, 8, 16, 0)  # 2^22 vectors: sliced from M = 1
    st, f16 = _ws_bytes(vq, big, 1, vq.VQ_F16)
    assert st == vq.VQ_OK and f16 > 0 and f16 % 256 == 0
    assert _ws_bytes(vq, big, 1, vq.VQ_BF16)[1] > f16          # + the fp16 copy of x
    assert _ws_bytes(vq, big, 16, vq.VQ_F16)[1] > f16          # partials per batch row
    # at least one fp32 partial per slice and row
    assert _ws_bytes(vq, vq.make_desc(16384, 4096, 8, 16, 8), 1, vq.VQ_F16)[1] >= 8 * 16384 * 4
    dec = vq.make_desc(4096, 4096, 8, 16, 0)  # 2^21 vectors: sliced from M = 8 only
    assert _ws_bytes(vq, dec, 1, vq.VQ_F16) == (vq.VQ_OK, 0)
    assert _ws_bytes(vq, dec, 7, vq.VQ_F16) == (vq.VQ_OK, 0)
    assert _ws_bytes(vq, dec, 8, vq.VQ_F16)[1] > 0
    # shapes without the sliced path need none
    for d in (vq.make_desc(14336, 4096, 6, 12, 12), vq.make_desc(4096, 4096, 8, 12, 0),
              vq.make_desc(4096, 4096, 8, 16, 4), vq.make_desc(4096, 4100, 8, 16, 0),
              vq.make_desc(256, 256, 8, 16, 0), vq.make_desc(0, 4096, 8, 16, 0)):
        assert _ws_bytes(vq, d, 8, vq.VQ_F16) == (vq.VQ_OK, 0), d
    assert _ws_bytes(vq, big, 0, vq.VQ_F16) == (vq.VQ_OK, 0)
    # errors leave the output alone
    assert _ws_bytes(vq, big, 17, vq.VQ_F16) == (vq.VQ_ERR_SHAPE, 12345)
    assert _ws_bytes(vq, big, -1, vq.VQ_F16) == (vq.VQ_ERR_SHAPE, 12345)
    assert _ws_bytes(vq, big, 1, vq.VQ_F32) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _ws_bytes(vq, None, 1, vq.VQ_F16) == (vq.VQ_ERR_NULL, 12345)
    assert _ws_bytes(vq, vq.make_desc(64, 64, 8, 0, 0), 1, vq.VQ_F16) == (vq.VQ_ERR_BITS, 12345)
    assert vq.lib().vq_gemv_workspace_bytes(ctypes.byref(big), 1, 0, None) == vq.VQ_ERR_NULL


def test_gemv_ws_validation_paths(vq):
    d = vq.make_desc(8192, 4096, 8, 16, 0)  # a shape with the sliced path
    need = _ws_bytes(vq, d, 1, vq.VQ_F16)[1]
    # the vq_gemv argument checks come first
    assert _gemv_ws(vq, None, ws=P, ws_bytes=need) == vq.VQ_ERR_NULL
    assert _gemv_ws(vq, d, ws=P, ws_bytes=need, m=17) == vq.VQ_ERR_SHAPE
    assert _gemv_ws(vq, d, ws=P, ws_bytes=need, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert _gemv_ws(vq, d, ws=P, ws_bytes=need, x=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    # then the workspace: size, 256-byte alignment
    assert _gemv_ws(vq, d, ws=P, ws_bytes=need - 1) == vq.VQ_ERR_BUFFER_SIZE
    assert _gemv_ws(vq, d, ws=P, ws_bytes=0) == vq.VQ_ERR_BUFFER_SIZE
    assert _gemv_ws(vq, d, ws=ctypes.c_void_p(0x10010), ws_bytes=need) == vq.VQ_ERR_ALIGN
    # nothing to do
    assert _gemv_ws(vq, d, ws=P, ws_bytes=0, m=0, y=None, x=None, packed=None) == vq.VQ_OK


def _gemm_ws_bytes(vq, desc, m, xt):
    n = ctypes.c_size_t(12345)
    st = vq.lib().vq_gemm_workspace_bytes(ctypes.byref(desc) if desc is not None else None, m, xt, ctypes.byref(n))
    return st, int(n.value)


def _r256(b):
    return (b + 255) // 256 * 256


def test_gemm_workspace_bytes(vq):
    """The workspace of vq_gemm_ws: for bf16 activations the fp16 copy [M][IN] and the M
    powers of two, then fp32 partial sums [splits][M][N] when the K range is split (the
    split count is chosen so that row blocks x splits cover about 192 of the 256 CUs)."""
    down = vq.make_desc(8192, 28672, 8, 16, 8)  # 32 row blocks of 256: eight splits
    st, nb = _gemm_ws_bytes(vq, down, 128, vq.VQ_BF16)
    assert st == vq.VQ_OK
    assert nb == _r256(128 * 28672 * 2) + _r256(128 * 4) + _r256(8 * 128 * 8192 * 4)
    assert _gemm_ws_bytes(vq, down, 128, vq.VQ_F16)[1] == _r256(8 * 128 * 8192 * 4)
    up = vq.make_desc(28672, 8192, 8, 16, 8)  # 112 row blocks: two splits
    assert _gemm_ws_bytes(vq, up, 128, vq.VQ_F16)[1] == _r256(2 * 128 * 28672 * 4)
    wide = vq.make_desc(50000, 512, 8, 16, 8)  # 196 row blocks: no split
    assert _gemm_ws_bytes(vq, wide, 128, vq.VQ_F16) == (vq.VQ_OK, 0)
    assert _gemm_ws_bytes(vq, wide, 128, vq.VQ_BF16)[1] == _r256(128 * 512 * 2) + _r256(128 * 4)
    short = vq.make_desc(5000, 136, 8, 16, 8)  # two K-tiles of 128 columns: no split
    assert _gemm_ws_bytes(vq, short, 7, vq.VQ_F16) == (vq.VQ_OK, 0)
    # shapes without the gather path need none
    for d in (vq.make_desc(14336, 4096, 6, 12, 12), vq.make_desc(4096, 4096, 8, 12, 0),
              vq.make_desc(4096, 4096, 8, 16, 4), vq.make_desc(4096, 4100, 8, 16, 0),
              vq.make_desc(4096, 0, 8, 16, 0), vq.make_desc(0, 4096, 8, 16, 0)):
        assert _gemm_ws_bytes(vq, d, 64, vq.VQ_BF16) == (vq.VQ_OK, 0), d
    assert _gemm_ws_bytes(vq, down, 0, vq.VQ_BF16) == (vq.VQ_OK, 0)
    # errors leave the output alone
    assert _gemm_ws_bytes(vq, down, -1, vq.VQ_F16) == (vq.VQ_ERR_SHAPE, 12345)
    assert _gemm_ws_bytes(vq, down, 1, vq.VQ_F32) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _gemm_ws_bytes(vq, None, 1, vq.VQ_F16) == (vq.VQ_ERR_NULL, 12345)
    assert vq.lib().vq_gemm_workspace_bytes(ctypes.byref(down), 1, 0, None) == vq.VQ_ERR_NULL


def test_gemm_ws_validation_paths(vq):
    d = vq.make_desc(8192, 28672, 8, 16, 0)
    need = _gemm_ws_bytes(vq, d, 64, vq.VQ_BF16)[1]
    f = lambda d, ws=P, nbytes=need, m=64, xt=1, x=P: vq.lib().vq_gemm_ws(
        ctypes.byref(d) if d is not None else None, P, P, P, None, None, x, xt, m, P, 2, ws, nbytes, None)
    assert f(None) == vq.VQ_ERR_NULL
    assert f(d, m=-1) == vq.VQ_ERR_SHAPE
    assert f(d, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert f(d, x=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    assert f(d, nbytes=need - 1) == vq.VQ_ERR_BUFFER_SIZE
    assert f(d, ws=ctypes.c_void_p(0x10010)) == vq.VQ_ERR_ALIGN
    assert f(d, m=0) == vq.VQ_OK


def _rht_ws(vq, desc, m, xt, gemm):
    n = ctypes.c_size_t(12345)
    st = vq.lib().vq_rht_product_workspace_bytes(ctypes.byref(desc) if desc is not None else None, m, xt, gemm,
                                                 ctypes.byref(n))
    return st, int(n.value)


def test_rht_product_workspace_bytes(vq):
    """Transform-fused products: the fused path's workspace (x pass and partial sums, never
    less than the transformed activations) where the shape has it, else room for x~ [M][IN]."""
    up = vq.make_desc(28672, 8192, 8, 16, 8)
    st, nb = _rht_ws(vq, up, 1, vq.VQ_BF16, 0)
    assert st == vq.VQ_OK and nb % 256 == 0
    assert nb >= _ws_bytes(vq, up, 1, vq.VQ_BF16)[1] + 8192 * 2  # the sliced workspace plus the fp16 copy
    st, nb = _rht_ws(vq, up, 128, vq.VQ_F16, 1)
    assert st == vq.VQ_OK and nb >= _gemm_ws_bytes(vq, up, 128, vq.VQ_F16)[1] + 128 * 8192 * 2
    dec = vq.make_desc(4096, 4096, 8, 16, 0)  # no sliced path at M = 1: x~ only
    assert _rht_ws(vq, dec, 1, vq.VQ_F16, 0) == (vq.VQ_OK, _r256(4096 * 2))
    v6 = vq.make_desc(300, 1024, 6, 12, 12)
    assert _rht_ws(vq, v6, 48, vq.VQ_BF16, 1) == (vq.VQ_OK, _r256(48 * 1024 * 2))
    wide = vq.make_desc(64, 65536, 8, 16, 0)  # beyond the fused pass's 32768 columns: x~ only
    assert _rht_ws(vq, wide, 64, vq.VQ_F16, 1) == (vq.VQ_OK, _r256(64 * 65536 * 2))
    assert _rht_ws(vq, up, 0, vq.VQ_F16, 0) == (vq.VQ_OK, 0)
    # errors leave the output alone
    assert _rht_ws(vq, up, 17, vq.VQ_F16, 0) == (vq.VQ_ERR_SHAPE, 12345)
    assert _rht_ws(vq, up, -1, vq.VQ_F16, 1) == (vq.VQ_ERR_SHAPE, 12345)
    assert _rht_ws(vq, up, 1, vq.VQ_F32, 0) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _rht_ws(vq, up, 1, vq.VQ_F16, 2) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _rht_ws(vq, vq.make_desc(64, 1000, 8, 16, 0), 1, vq.VQ_F16, 0) == (vq.VQ_ERR_UNSUPPORTED, 12345)
    assert _rht_ws(vq, None, 1, vq.VQ_F16, 0) == (vq.VQ_ERR_NULL, 12345)


def test_rht_product_validation_paths(vq):
    d = vq.make_desc(28672, 8192, 8, 16, 8)
    for gemm, fn in ((0, vq.lib().vq_gemv_ws_rht), (1, vq.lib().vq_gemm_ws_rht)):
        need = _rht_ws(vq, d, 1, vq.VQ_BF16, gemm)[1]
        f = lambda desc, ws=P, nbytes=need, x=P, sg=P, m=1: fn(ctypes.byref(desc) if desc is not None else None, P, P, P,
                                                               None, None, x, 1, m, sg, P, 2, ws, nbytes, None)
        assert f(None) == vq.VQ_ERR_NULL
        assert f(vq.make_desc(64, 1000, 8, 16, 0)) == vq.VQ_ERR_UNSUPPORTED
        assert f(d, sg=None) == vq.VQ_ERR_NULL
        assert f(d, ws=None) == vq.VQ_ERR_NULL
        assert f(d, x=ctypes.c_void_p(0x10008)) == vq.VQ_ERR_ALIGN
        assert f(d, nbytes=need - 1) == vq.VQ_ERR_BUFFER_SIZE
        assert f(d, ws=ctypes.c_void_p(0x10010)) == vq.VQ_ERR_ALIGN
        assert f(d, m=0) == vq.VQ_OK
    assert vq.lib().vq_gemv_ws_rht(ctypes.byref(d), P, P, P, None, None, P, 1, 17, P, P, 2, P, 1 << 30,
                                   None) == vq.VQ_ERR_SHAPE


def test_gemv_noalloc_validation_paths(vq):
    """vq_gemv_noalloc checks its arguments like vq_gemv, then rejects shapes whose sliced-path
    workspace exceeds the library's fixed 16 MiB before touching the device."""
    f = lambda d, m=1, xt=0, x=P: vq.lib().vq_gemv_noalloc(ctypes.byref(d) if d is not None else None, P, P, P,
                                                           None, None, x, xt, m, P, 2, None)
    d = vq.make_desc(8192, 4096, 8, 16, 0)
    assert f(None) == vq.VQ_ERR_NULL
    assert f(d, m=17) == vq.VQ_ERR_SHAPE
    assert f(d, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert f(d, x=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    assert f(d, m=0) == vq.VQ_OK
    # 2^19 rows of 8 vectors: 8 slices x 2^19 rows x 4 bytes of partials = 16 MiB + x exponents
    huge = vq.make_desc(1 << 19, 64, 8, 16, 8)
    assert _ws_bytes(vq, huge, 1, vq.VQ_BF16)[1] > 16 << 20
    assert f(huge, xt=1) == vq.VQ_ERR_BUFFER_SIZE
    m16 = vq.make_desc(1 << 16, 512, 8, 16, 0)  # fine at M = 1, too large at M = 16
    assert _ws_bytes(vq, m16, 1, vq.VQ_F16)[1] <= 16 << 20 < _ws_bytes(vq, m16, 16, vq.VQ_F16)[1]
    assert f(m16, m=16) == vq.VQ_ERR_BUFFER_SIZE


def _svq(vq, desc, packed=P, a=P, b=P, scale=None, bias=None, x=P, xt=0, m=1, y=P, yt=2, fn=None):
    fn = fn or vq.lib().vq_svq_gemv
    return fn(ctypes.byref(desc) if desc is not None else None, packed, a, b, scale, bias, x, xt, m, y, yt, None)


def test_svq_gemv_validation_paths(vq):
    d = vq.svq_desc(64, 64)
    assert _svq(vq, None) == vq.VQ_ERR_NULL
    assert _svq(vq, vq.make_desc(64, 64, 4, 0, 0)) == vq.VQ_ERR_BITS
    # only the lattice stream: v = 4, one 8-bit field per vector, no residual
    for other in (vq.make_desc(64, 64, 8, 8, 0), vq.make_desc(64, 64, 4, 8, 8), vq.make_desc(64, 64, 4, 16, 0)):
        assert _svq(vq, other) == vq.VQ_ERR_UNSUPPORTED, other
    assert _svq(vq, d, m=-1) == vq.VQ_ERR_SHAPE
    assert _svq(vq, d, m=17) == vq.VQ_ERR_SHAPE
    assert _svq(vq, d, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert _svq(vq, d, yt=7) == vq.VQ_ERR_UNSUPPORTED
    assert _svq(vq, d, y=None) == vq.VQ_ERR_NULL
    assert _svq(vq, d, packed=None) == vq.VQ_ERR_NULL
    assert _svq(vq, d, a=None) == vq.VQ_ERR_NULL
    assert _svq(vq, d, b=None) == vq.VQ_ERR_NULL
    assert _svq(vq, d, x=None) == vq.VQ_ERR_NULL
    assert _svq(vq, d, packed=ctypes.c_void_p(0x10008)) == vq.VQ_ERR_ALIGN  # 16-byte code loads
    assert _svq(vq, d, a=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    assert _svq(vq, d, x=ctypes.c_void_p(0x10001)) == vq.VQ_ERR_ALIGN
    assert _svq(vq, d, y=P_MIS, yt=2) == vq.VQ_ERR_ALIGN
    # nothing to do
    assert _svq(vq, d, m=0, y=None, x=None, packed=None, a=None, b=None) == vq.VQ_OK
    assert _svq(vq, vq.svq_desc(0, 64), y=None, x=None, packed=None) == vq.VQ_OK


def test_svq_gemm_validation_paths(vq):
    """vq_svq_gemm takes any M >= 0 and otherwise validates like vq_svq_gemv."""
    g = lambda desc, **kw: _svq(vq, desc, **kw, fn=vq.lib().vq_svq_gemm)
    d = vq.svq_desc(64, 64)
    assert g(None) == vq.VQ_ERR_NULL
    assert g(vq.make_desc(64, 64, 8, 8, 0)) == vq.VQ_ERR_UNSUPPORTED
    assert g(d, m=-1) == vq.VQ_ERR_SHAPE
    assert g(d, m=128 * 65535 + 1) == vq.VQ_ERR_SHAPE
    assert g(d, xt=2) == vq.VQ_ERR_UNSUPPORTED
    assert g(d, yt=7) == vq.VQ_ERR_UNSUPPORTED
    assert g(d, m=17, y=None) == vq.VQ_ERR_NULL   # M > 16 passes the shape check
    assert g(d, m=300, x=None) == vq.VQ_ERR_NULL
    assert g(d, a=None) == vq.VQ_ERR_NULL
    assert g(d, packed=ctypes.c_void_p(0x10008)) == vq.VQ_ERR_ALIGN
    assert g(d, y=P_MIS, yt=2) == vq.VQ_ERR_ALIGN
    assert g(d, m=0, y=None, x=None, packed=None, a=None, b=None) == vq.VQ_OK


def test_svq_dequant_validation_paths(vq):
    f = vq.lib().vq_svq_dequant
    d = vq.svq_desc(64, 64)
    assert f(None, P, P, P, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(vq.make_desc(64, 64, 8, 16, 0)), P, P, P, None, P, 2, None) == vq.VQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), None, P, P, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), P, None, P, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), P, P, None, None, P, 2, None) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(d), P, P, P, None, P, 9, None) == vq.VQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), P, P, P, None, P_MIS, 2, None) == vq.VQ_ERR_ALIGN
    assert f(ctypes.byref(vq.svq_desc(64, 0)), None, None, None, None, None, 2, None) == vq.VQ_OK


def test_svq_pack_through_the_abi(vq):
    """vq_svq_pack on integer grid coordinates: the oracle's lattice decode with the identity
    grid (A = I, B = 0) returns every coordinate, and the bytes equal the oracle's own packing
    of the same layer; coordinates above 3, a codebook descriptor and a short buffer are
    refused."""
    g = np.random.default_rng(5)
    n, i = 5, 37  # nv = 10, the last vector has one live lane
    nv = (i + 3) // 4
    q = g.integers(0, 4, size=(n, nv, 4), dtype=np.uint8)
    d = vq.svq_desc(n, i)
    packed = vq.svq_pack(d, q)
    eye = np.eye(4, dtype=np.float16).view(np.uint16)
    w = oracle.svq_dequant(n, i, packed, eye, np.zeros(4, np.uint16))
    assert np.array_equal(w, q.reshape(n, nv * 4)[:, :i].astype(np.float32))
    lay = synth.make_svq_layer(n, i)
    q2 = np.stack([(lay["codes"] >> (2 * u)) & 3 for u in range(4)], axis=-1).astype(np.uint8)
    assert np.array_equal(vq.svq_pack(d, q2), oracle.pack(n, i, 4, 8, 0, lay["codes"]))
    f = vq.lib().vq_svq_pack
    buf = np.zeros(vq.packed_bytes(d), dtype=np.uint8)
    bad = q.copy()
    bad[3, 4, 2] = 4
    bp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert f(ctypes.byref(d), bp(bad), bp(buf), buf.size) == vq.VQ_ERR_INDEX_RANGE
    assert not buf.any()
    assert f(ctypes.byref(vq.make_desc(n, i, 4, 8, 2)), bp(q), bp(buf), buf.size) == vq.VQ_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), bp(q), bp(buf), buf.size - 1) == vq.VQ_ERR_BUFFER_SIZE
    assert f(ctypes.byref(d), None, bp(buf), buf.size) == vq.VQ_ERR_NULL
    assert f(ctypes.byref(vq.svq_desc(0, 16)), None, None, 0) == vq.VQ_OK


def test_rht_block_and_validation(vq):
    for n in (16, 48, 96, 1000, 4096, 4100, 14336, 28672, 32768, 65536, 7, 0, -3):
        assert vq.rht_block(n) == (oracle.rht_block(n) if n > 0 else 0), n
    f = vq.lib().vq_rht
    assert f(-1, 64, P, 0, P, 0, P, 2, None) == vq.VQ_ERR_SHAPE
    assert f(1, -64, P, 0, P, 0, P, 2, None) == vq.VQ_ERR_SHAPE
    assert f(1, 64, P, 7, P, 0, P, 2, None) == vq.VQ_ERR_UNSUPPORTED
    assert f(1, 64, P, 0, P, 0, P, 9, None) == vq.VQ_ERR_UNSUPPORTED
    assert f(1, 64, P, 0, P, 2, P, 2, None) == vq.VQ_ERR_UNSUPPORTED   # transpose is 0 or 1
    assert f(1, 1000, P, 0, P, 0, P, 2, None) == vq.VQ_ERR_UNSUPPORTED  # block 8: n must be a multiple of 16
    assert f(1, 64, None, 0, P, 0, P, 2, None) == vq.VQ_ERR_NULL
    assert f(1, 64, P, 0, None, 0, P, 2, None) == vq.VQ_ERR_NULL
    assert f(1, 64, P, 0, P, 0, None, 2, None) == vq.VQ_ERR_NULL
    assert f(1, 64, ctypes.c_void_p(0x10008), 0, P, 0, P, 2, None) == vq.VQ_ERR_ALIGN
    assert f(1, 64, P, 0, P, 0, P_MIS, 2, None) == vq.VQ_ERR_ALIGN
    assert f(0, 64, None, 0, None, 0, None, 2, None) == vq.VQ_OK
    assert f(3, 0, None, 0, None, 0, None, 2, None) == vq.VQ_OK


def test_assign_workspace_and_validation(vq):
    up = lambda b: (b + 255) // 256 * 256
    # fp64 records {|c|^2, c} of both books, one fp64 {max |c_t|, max |c|^2} pair per 256
    # centroids of each book, then for K1 >= 256 the matrix-core tables of the main book (K1
    # rounded up to 512 rows: fp16 -c in 8-wide blocks, fp32 |c|^2 / 2, one fp32 maxima pair
    # per 256 rows)
    maxima = lambda k1, k2: up(-(-k1 // 256) * 16) + up(-(-k2 // 256) * 16)
    d = vq.make_desc(4096, 4096, 8, 16, 8)
    assert vq.assign_workspace_bytes(d) == (up((65536 + 256) * 9 * 8) + maxima(65536, 256) + 65536 * 16 + 65536 * 4
                                            + 256 * 8)
    d16 = vq.make_desc(5, 64, 16, 9, 0)
    assert vq.assign_workspace_bytes(d16) == up(512 * 17 * 8) + maxima(512, 0) + 512 * 32 + 512 * 4 + up(2 * 8)
    d1 = vq.make_desc(7, 12, 3, 5, 0)
    assert vq.assign_workspace_bytes(d1) == up(32 * 4 * 8) + maxima(32, 0)
    f = vq.lib().vq_assign
    big = ctypes.c_size_t(1 << 30)
    ok = vq.make_desc(8, 64, 8, 8, 4)
    br = ctypes.byref
    assert f(None, P, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_NULL
    assert f(br(vq.make_desc(8, 64, 17, 8, 4)), P, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_BITS
    assert f(br(vq.make_desc(8, 64, 8, 0, 4)), P, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_BITS
    assert f(br(vq.make_desc(-8, 64, 8, 8, 4)), P, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_SHAPE
    assert f(br(vq.make_desc(8, 60, 8, 8, 4)), P, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_UNSUPPORTED  # IN % v
    assert f(br(ok), P, 5, P, P, P, P, P, big, None) == vq.VQ_ERR_UNSUPPORTED                          # w dtype
    assert f(br(ok), None, 0, P, P, P, P, P, big, None) == vq.VQ_ERR_NULL
    assert f(br(ok), P, 0, None, P, P, P, P, big, None) == vq.VQ_ERR_NULL
    assert f(br(ok), P, 0, P, None, P, P, P, big, None) == vq.VQ_ERR_NULL      # cb2 with bits2 > 0
    assert f(br(ok), P, 0, P, P, None, P, P, big, None) == vq.VQ_ERR_NULL
    assert f(br(ok), P, 0, P, P, P, None, P, big, None) == vq.VQ_ERR_NULL      # idx2 with bits2 > 0
    assert f(br(ok), P, 0, P, P, P, P, None, big, None) == vq.VQ_ERR_NULL      # workspace
    need = vq.assign_workspace_bytes(ok)
    assert f(br(ok), P, 0, P, P, P, P, P, need - 1, None) == vq.VQ_ERR_BUFFER_SIZE
    assert f(br(ok), P, 0, P, P, P, P, P_MIS, big, None) == vq.VQ_ERR_ALIGN     # workspace 256-byte aligned
    assert f(br(ok), P_MIS, 2, P, P, P, P, P, big, None) == vq.VQ_ERR_ALIGN     # fp32 w
    assert f(br(ok), P, 0, P, P, P_MIS, P, P, big, None) == vq.VQ_ERR_ALIGN     # idx1
    assert f(br(vq.make_desc(0, 64, 8, 8, 4)), None, 0, None, None, None, None, None, 0, None) == vq.VQ_OK
    assert f(br(vq.make_desc(8, 0, 8, 8, 4)), None, 0, None, None, None, None, None, 0, None) == vq.VQ_OK
