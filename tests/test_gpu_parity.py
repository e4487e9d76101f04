"""GPU parity: the HIP path through the C ABI against the CPU oracle.

- vq_dequant: bit-exact fp32 W^, and fp16 / bf16 outputs equal to the oracle's
  nearest-even rounding of it;
- vq_gemv (1 <= M <= 16) and vq_gemm (any M): max |y - y64| <= 2e-3 * ||y64||_inf with
  fp32 outputs, and the same bound after half an output ulp for fp16 / bf16 outputs;
- a one-hot x reproduces columns of W^ bit-exactly through vq_gemv;
- edge cases: ragged N / IN / M, tail vectors, bias, no scale, empty shapes, a
  non-default stream, the generic (any v) path, batches above one MFMA chunk.
Full-size workloads are checked on sampled rows that the oracle computes one by one.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from vqtest import DeviceLayer, check_y, oracle_w, oracle_y, sample_rows, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


@functools.lru_cache(maxsize=8)
def _workload_layer(key, layer):
    return synth.workload_layer(key, layer)


@functools.lru_cache(maxsize=8)
def _device_workload(key, layer):
    import gemv_bit_unpack_amd as g

    return DeviceLayer(g, _workload_layer(key, layer))


BIG = {"mlp8b", "l70b"}
WL_LAYERS = [(k, i) for k, w in synth.WORKLOADS.items() for i in range(len(w.layers))]


def _rows_for(key, n):
    return None if key not in BIG else sample_rows(n, 48, seed=n)


# ------------------------------------------------------------------ dequant


@pytest.mark.parametrize("key,layer", WL_LAYERS)
def test_dequant_bit_exact_workloads(vq, key, layer):
    print("dequant", key, layer, flush=True)
    lay = _workload_layer(key, layer)
    dl = _device_workload(key, layer)
    rows = _rows_for(key, lay["n"])
    w = vq.dequant(*dl.args()[:5])
    torch.cuda.synchronize()
    sel = w if rows is None else w[torch.from_numpy(rows).cuda()]
    got = sel.cpu().numpy()
    ref = oracle_w(lay, rows)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    del w
    for dt, conv in ((torch.float16, oracle.f32_array_to_f16_rne), (torch.bfloat16, oracle.f32_array_to_bf16_rne)):
        wn = vq.dequant(*dl.args()[:5], w_dtype=dt)
        seln = wn if rows is None else wn[torch.from_numpy(rows).cuda()]
        bits = seln.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(bits, conv(ref))


@pytest.mark.parametrize("n,i,v,b1,b2,scale", [
    (37, 100, 3, 5, 7, True), (33, 70, 6, 12, 12, True), (5, 4097, 6, 12, 12, True), (3, 1, 1, 1, 0, False),
    (9, 200, 16, 16, 16, True), (64, 1000, 8, 8, 8, False), (2, 13, 4, 1, 2, True),
])
def test_dequant_bit_exact_shapes(vq, n, i, v, b1, b2, scale):
    lay = synth.make_layer(n, i, v, b1, b2, wid=70, copy=n + i, with_scale=scale)
    dl = DeviceLayer(vq, lay)
    w = vq.dequant(*dl.args()[:5]).cpu().numpy()
    ref = oracle_w(lay)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_dequant_fp16_identity_codebook(vq):
    """v = 1, K = 65536, C[k] = fp16 with bit pattern k: any finite fp16 matrix comes back."""
    n, i = 24, 136
    g = np.random.default_rng(5)
    wb = g.integers(0, 65536, (n, i), dtype=np.uint32).astype(np.uint16)
    wb[~np.isfinite(wb.view(np.float16))] = 0
    lay = dict(n=n, in_features=i, v=1, bits1=16, bits2=0, idx1=wb.astype(np.uint32), idx2=None,
               cb1=np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(-1, 1), cb2=None, scale=None,
               bias=None)
    dl = DeviceLayer(vq, lay)
    w = vq.dequant(*dl.args()[:5], w_dtype=torch.float16)
    assert np.array_equal(w.view(torch.int16).cpu().numpy().view(np.uint16), wb)


# ------------------------------------------------------------------ gemv


GEMV_CASES = [(k, i, m) for (k, i) in WL_LAYERS for m in synth.WORKLOADS[k].ms if m <= 16]


@pytest.mark.parametrize("key,layer,m", GEMV_CASES)
def test_gemv_parity_workloads(vq, key, layer, m):
    print("gemv", key, layer, m, flush=True)
    w = synth.WORKLOADS[key]
    lay = _workload_layer(key, layer)
    dl = _device_workload(key, layer)
    xb = synth.workload_x(key, layer, m)
    x = x_tensor(xb, w.x_dtype)
    rows = _rows_for(key, lay["n"])
    y64 = oracle_y(lay, xb, w.x_dtype, rows)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, torch.from_numpy(rows).cuda()])
    y = vq.gemv(*dl.args(), x, y_dtype=torch.float32)
    check_y(sel(y), y64, "f32")
    yn = vq.gemv(*dl.args(), x)  # output in the activation type
    check_y(sel(yn), y64, w.x_dtype)


@pytest.mark.parametrize("n,i,v,b1,b2,m,xd,bias,scale", [
    (37, 100, 3, 5, 7, 3, "f16", True, True),      # generic path (v = 3)
    (70, 4097, 6, 12, 12, 5, "bf16", True, True),  # ragged IN with v = 6: last vector keeps 5 lanes
    (65, 1000, 8, 16, 8, 16, "f16", False, False),  # IN*2 not a multiple of 16: generic path
    (129, 1024, 8, 16, 8, 2, "bf16", True, False),
    (1, 8, 8, 16, 0, 1, "f16", True, True),
    (300, 4096, 8, 12, 4, 7, "f16", False, True),   # 12-bit main book staged in LDS
    (17, 256, 16, 16, 16, 4, "bf16", True, True),   # v = 16, two 65536-entry books
    (100, 4104, 16, 16, 0, 1, "f16", True, True),   # v = 16: last vector keeps 8 lanes
    (70, 1032, 16, 16, 8, 3, "bf16", True, False),  # v = 16 with a residual in LDS
    (9, 200, 16, 16, 16, 16, "f16", False, True),   # v = 16, two global books, M = 16
    (65, 512, 8, 16, 16, 2, "f16", False, True),    # two global books (AQLM 2 x 2^16)
    (33, 1000, 8, 16, 16, 16, "bf16", True, True),
    (5, 104, 16, 12, 0, 2, "f16", True, False),     # v = 16 with an LDS main book: generic path
    # the gather kernel takes 4 vectors per lane for rows of <= 512 vectors at M <= 2, else 8
    (96, 4096, 8, 16, 8, 2, "f16", True, True),     # 512 vectors: two steps of 4 per lane
    (96, 4104, 8, 16, 0, 1, "bf16", False, True),   # 513 vectors: 8 per lane, ragged last group
    # v = 6, fp16 x, M = 1, 12-bit fields, IN % 8 == 0: books and x in LDS, fields from registers
    (1000, 4104, 6, 12, 12, 1, "f16", True, True),  # 4 rows per workgroup, 12 items over 16 wavefronts
    (3000, 2048, 6, 12, 0, 1, "f16", True, False),  # 12 rows per workgroup; no residual
    (5, 48, 6, 12, 12, 1, "f16", False, True),      # five workgroups of one row, one chunk each
    # v = 6, fp16 x, 2 <= M <= 16, 12-bit fields, IN % 8 == 0: the matrix-core kernel
    (1000, 4104, 6, 12, 12, 16, "f16", True, True),  # 63 tiles, 257-step rows over 16 wavefronts
    (37, 48, 6, 12, 0, 5, "f16", False, True),       # 3 tiles of one step: most wavefronts idle
    (5000, 2048, 6, 12, 12, 2, "f16", True, True),   # 2 tiles per workgroup; last tile ragged
    (300, 4096, 6, 12, 12, 9, "f16", True, False),   # last vector keeps 4 lanes, odd M
    # v = 6, fp16 x, M <= 2, books in LDS: the packed-dot kernel with LDS-staged index chunks
    (1000, 4100, 6, 12, 12, 1, "f16", True, True),  # last vector keeps 2 lanes
    (333, 1538, 6, 11, 9, 2, "f16", False, True),   # odd index widths; 257 vectors: two chunks
    (17, 14336, 6, 12, 0, 1, "f16", True, False),   # no residual, ten chunks per row
    (4099, 96, 6, 12, 12, 2, "f16", True, True),    # more rows than wavefronts in the grid
    (5, 6, 6, 4, 3, 1, "f16", False, False),        # one vector per row
    (40, 2000, 6, 12, 12, 3, "f16", True, True),    # M = 3, IN % 8 == 0: the matrix-core kernel
    (40, 2002, 6, 12, 12, 3, "f16", True, True),    # M = 3, IN % 8 == 2: the general v = 6 kernel
])
def test_gemv_parity_shapes(vq, n, i, v, b1, b2, m, xd, bias, scale):
    lay = synth.make_layer(n, i, v, b1, b2, wid=71, copy=n, with_scale=scale, with_bias=bias)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n), m, i, xd)
    x = x_tensor(xb, xd)
    y64 = oracle_y(lay, xb, xd)
    check_y(vq.gemv(*dl.args(), x, y_dtype=torch.float32), y64, "f32")
    check_y(vq.gemv(*dl.args(), x), y64, xd)


@pytest.mark.parametrize("n,i,v,b1,b2", [(64, 512, 8, 16, 8), (48, 96, 6, 12, 12), (32, 256, 8, 8, 0),
                                         (40, 4096, 8, 16, 8), (40, 1032, 16, 16, 8), (32, 512, 8, 16, 16),
                                         (24, 264, 16, 16, 16)])
def test_gemv_one_hot_columns_bit_exact(vq, n, i, v, b1, b2):
    """x = e_col gives y[o] = s_o * (c1 + c2)[col], the exact fp32 W^ entry."""
    lay = synth.make_layer(n, i, v, b1, b2, wid=72, copy=i)
    dl = DeviceLayer(vq, lay)
    w32 = oracle_w(lay)
    cols = np.array([0, 1, v - 1, v, i // 2, i - 1][: min(6, i)])
    xb = np.zeros((cols.size, i), dtype=np.uint16)
    xb[np.arange(cols.size), cols] = 0x3C00  # 1.0
    y = vq.gemv(*dl.args(), x_tensor(xb, "f16"), y_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(y, w32[:, cols].T)  # == comparison: +0 and -0 both accepted


@pytest.mark.parametrize("n,i,b2,m", [(48, 96, 12, 1), (40, 4100, 0, 1), (33, 1538, 9, 2), (300, 1544, 12, 1),
                                      (20, 1544, 0, 1), (64, 1544, 12, 4), (40, 200, 0, 16)])
def test_gemv6_one_hot_columns_bit_exact(vq, n, i, b2, m):
    """The v = 6 LDS-book kernels (fp16 x; with 12-bit fields and IN % 8 == 0 the x-in-LDS
    one at M = 1 and the matrix-core one at 2 <= M <= 16): a one-hot x still gives the exact
    fp32 W^ entry, main centroid added first."""
    lay = synth.make_layer(n, i, 6, 12, b2, wid=76, copy=i)
    dl = DeviceLayer(vq, lay)
    w32 = oracle_w(lay)
    cols = np.array([0, 1, 5, 6, i // 2 + 1, i - 2, i - 1])
    for start in range(0, cols.size, m):
        cs = cols[start:start + m]
        xb = np.zeros((cs.size, i), dtype=np.uint16)
        xb[np.arange(cs.size), cs] = 0x3C00  # 1.0
        y = vq.gemv(*dl.args(), x_tensor(xb, "f16"), y_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(y, w32[:, cs].T), (start, cs)


@pytest.mark.parametrize("n", [262144, 262145])
def test_gemv6_row_limit(vq, n):
    """The v = 6 packed-dot kernel holds each wavefront's scales and biases in its lanes, one
    row each: at 262144 rows (64 per wavefront) the last lane is used; one row more goes to
    the general kernel.  Sampled rows, the last wavefront's rows included."""
    lay = synth.make_layer(n, 12, 6, 12, 12, wid=77, with_scale=True, with_bias=True)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(5), 1, 12, "f16")
    rows = np.unique(np.concatenate([sample_rows(n, 40, seed=n), np.arange(n - 4100, n, 97), [n - 1]]))
    y64 = oracle_y(lay, xb, "f16", rows)
    y = vq.gemv(*dl.args(), x_tensor(xb, "f16"), y_dtype=torch.float32)
    check_y(y[:, torch.from_numpy(rows).cuda()], y64, "f32")
    yb = vq.gemv(*dl.args(), x_tensor(xb, "f16"), y_dtype=torch.bfloat16)
    check_y(yb[:, torch.from_numpy(rows).cuda()], y64, "bf16")


def test_gemv_edge_cases(vq):
    lay = synth.make_layer(40, 64, 8, 8, 0, wid=73, with_bias=True)
    dl = DeviceLayer(vq, lay)
    # M = 0: nothing is written
    y = torch.full((0, 40), 7.0, device="cuda")
    vq.gemv(*dl.args(), torch.zeros((0, 64), dtype=torch.float16, device="cuda"), out=y)
    # IN = 0: y = bias
    lay0 = synth.make_layer(40, 0, 8, 8, 0, wid=73, with_bias=True)
    dl0 = DeviceLayer(vq, lay0)
    y0 = vq.gemv(*dl0.args(), torch.zeros((3, 0), dtype=torch.float16, device="cuda"), y_dtype=torch.float32)
    bias = lay0["bias"].view(np.float16).astype(np.float32)
    assert np.array_equal(y0.cpu().numpy(), np.tile(bias, (3, 1)))
    y0m = vq.gemm(*dl0.args(), torch.zeros((3, 0), dtype=torch.float16, device="cuda"), y_dtype=torch.float32)
    assert np.array_equal(y0m.cpu().numpy(), np.tile(bias, (3, 1)))
    # N = 0: no-op
    layn = synth.make_layer(0, 64, 8, 8, 0, wid=73)
    dln = DeviceLayer(vq, layn)
    assert vq.gemv(*dln.args(), torch.zeros((2, 64), dtype=torch.float16, device="cuda")).shape == (2, 0)


def test_gemv_and_gemm_on_side_stream(vq):
    lay = synth.make_layer(256, 1024, 8, 16, 8, wid=74)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(1), 8, 1024, "f16")
    x = x_tensor(xb, "f16")
    y64 = oracle_y(lay, xb, "f16")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1 = vq.gemv(*dl.args(), x, y_dtype=torch.float32)
        y2 = vq.gemm(*dl.args(), x, y_dtype=torch.float32)
    s.synchronize()
    check_y(y1, y64, "f32")
    check_y(y2, y64, "f32")


# ------------------------------------------------------------------ gemm


GEMM_CASES = [("tiny", 0, 1), ("tiny", 0, 33), ("dec4k", 0, 32), ("dec4k_res", 0, 16), ("dec4k_res", 0, 40),
              ("mlp8b", 1, 32), ("mlp8b", 0, 4), ("l70b", 0, 32), ("l70b", 0, 128), ("l70b", 1, 128),
              ("l70b", 0, 256), ("l70b", 1, 8), ("l70b", 1, 32), ("l70b", 1, 256)]


@pytest.mark.parametrize("key,layer,m", GEMM_CASES)
def test_gemm_parity_workloads(vq, key, layer, m):
    print("gemm", key, layer, m, flush=True)
    w = synth.WORKLOADS[key]
    lay = _workload_layer(key, layer)
    dl = _device_workload(key, layer)
    g = np.random.default_rng(1000 + m)
    xb = synth.activations(g, m, lay["in_features"], w.x_dtype)
    x = x_tensor(xb, w.x_dtype)
    rows = _rows_for(key, lay["n"])
    y64 = oracle_y(lay, xb, w.x_dtype, rows)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, torch.from_numpy(rows).cuda()])
    check_y(sel(vq.gemm(*dl.args(), x, y_dtype=torch.float32)), y64, "f32")
    check_y(sel(vq.gemm(*dl.args(), x)), y64, w.x_dtype)


@pytest.mark.parametrize("n,i,v,b1,b2,m,xd,bias,scale", [
    (37, 100, 3, 5, 7, 33, "f16", True, True),      # generic v, ragged everything
    (70, 4097, 6, 12, 12, 45, "bf16", True, True),  # ragged IN, v = 6
    (100, 1000, 8, 16, 8, 300, "f16", False, True),  # M above one 256-row chunk, unaligned x rows
    (64, 512, 8, 16, 0, 64, "bf16", True, False),
    (33, 256, 16, 16, 16, 31, "f16", True, True),
    (96, 2048, 8, 8, 8, 97, "bf16", False, True),
])
def test_gemm_parity_shapes(vq, n, i, v, b1, b2, m, xd, bias, scale):
    lay = synth.make_layer(n, i, v, b1, b2, wid=75, copy=n, with_scale=scale, with_bias=bias)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n + m), m, i, xd)
    x = x_tensor(xb, xd)
    y64 = oracle_y(lay, xb, xd)
    check_y(vq.gemm(*dl.args(), x, y_dtype=torch.float32), y64, "f32")
    check_y(vq.gemm(*dl.args(), x), y64, xd)


def test_vqlinear_picks_path_and_matches(vq):
    lay = synth.make_layer(128, 512, 8, 16, 8, wid=76, with_bias=True)
    dl = DeviceLayer(vq, lay)
    layer = vq.VQLinear(*dl.args())
    for m in (1, 16, 17, 64):
        xb = synth.activations(np.random.default_rng(m), m, 512, "bf16")
        y = layer(x_tensor(xb, "bf16").reshape(1, m, 512), y_dtype=torch.float32)
        assert y.shape == (1, m, 128)
        check_y(y.reshape(m, 128), oracle_y(lay, xb, "bf16"), "f32")
