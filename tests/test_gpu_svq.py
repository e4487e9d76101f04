"""GPU parity of the affine-lattice calls (UniSVQ summary: d = 4 vectors A q + B over
2-bit integer codes), vq_svq_dequant and vq_svq_gemv, against the CPU oracle through the
C ABI.

- dequant: fp32 output bit-exact on ragged shapes (IN not a multiple of 4, 16 or 64),
  with and without scale; fp16 / bf16 outputs equal the nearest-even rounding of the
  oracle's fp32;
- gemv: shapes with ragged rows and columns (vector tails of 1..3 lanes, rows ending
  inside a column slice, several slices), M from 1 to 16, bias and scale, every output
  dtype, fp16 and bf16 activations, every kernel shape (for M = 1: the whole row's
  activations resident in LDS with one or two rows per wavefront, or walked in slices);
  the workloads (4096^2 at M = 1, 4, 16; the 70B-class pair at M = 1, 8) on sampled rows
  at full size;
- the matrix-core product (vq_svq_gemm) for any M: ragged shapes, M from 1 to 300 (more
  than one batch chunk), every output dtype, fp16 and bf16 activations, IN = 0, the
  workloads at prefill batches on sampled rows;
- dyadic grids with one-hot activations reproduce columns of W^ bit-exactly;
- determinism and replays of a captured graph.
Tolerance: max |y - y64| <= 2e-3 * ||y64||_inf with fp32 outputs, plus half an output
ulp for fp16 / bf16 outputs.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from vqtest import check_y, f16_tensor, sample_rows, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


class SvqLayer:
    """A synthetic affine-lattice layer packed by the library's packer and uploaded."""

    def __init__(self, vq, lay, device="cuda"):
        self.lay = lay
        self.desc = vq.svq_desc(lay["n"], lay["in_features"])
        packed = vq.pack(self.desc, lay["codes"])
        self.packed = torch.from_numpy(packed if packed.size else np.zeros(16, np.uint8)).to(device)
        self.a = f16_tensor(lay["a"], device)
        self.b = f16_tensor(lay["b"], device)
        self.scale = f16_tensor(lay["scale"], device)
        self.bias = f16_tensor(lay["bias"], device)

    def gemv(self, vq, x, y_dtype=None):
        return vq.svq_gemv(self.desc, self.packed, self.a, self.b, self.scale, self.bias, x, y_dtype=y_dtype)

    def gemm(self, vq, x, y_dtype=None):
        return vq.svq_gemm(self.desc, self.packed, self.a, self.b, self.scale, self.bias, x, y_dtype=y_dtype)

    def dequant(self, vq, w_dtype):
        return vq.svq_dequant(self.desc, self.packed, self.a, self.b, self.scale, w_dtype=w_dtype)


def _sub(lay, rows):
    sub = dict(lay)
    sub["n"] = int(len(rows))
    sub["codes"] = lay["codes"][rows]
    sub["scale"] = lay["scale"][rows] if lay["scale"] is not None else None
    sub["bias"] = lay["bias"][rows] if lay["bias"] is not None else None
    return sub


def _oracle_packed(lay):
    return oracle.pack(lay["n"], lay["in_features"], 4, 8, 0, lay["codes"])


def _oracle_w(lay):
    return oracle.svq_dequant(lay["n"], lay["in_features"], _oracle_packed(lay), lay["a"], lay["b"], lay["scale"])


def _oracle_y(lay, x_bits, x_dtype, rows=None):
    sub = lay if rows is None else _sub(lay, rows)
    return oracle.svq_forward(sub["n"], sub["in_features"], _oracle_packed(sub), sub["a"], sub["b"], sub["scale"],
                              sub["bias"], x_bits, x_dtype == "bf16", x_bits.shape[0])


def _tdtype(name):
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


@pytest.mark.parametrize("n,in_features,with_scale", [
    (7, 13, False), (33, 64, True), (5, 70, True), (64, 4100, False), (3, 1, True), (2, 16387, True),
])
def test_svq_dequant_bit_exact(vq, n, in_features, with_scale):
    lay = synth.make_svq_layer(n, in_features, with_scale=with_scale)
    dl = SvqLayer(vq, lay)
    w_ref = _oracle_w(lay)
    w = dl.dequant(vq, torch.float32).cpu().numpy()
    assert np.array_equal(w.view(np.uint32), w_ref.view(np.uint32))
    w16 = dl.dequant(vq, torch.float16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w16, oracle.f32_array_to_f16_rne(w_ref))
    wb = dl.dequant(vq, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wb, oracle.f32_array_to_bf16_rne(w_ref))


SHAPES = [
    # n, in_features, M, x dtype, y dtype, scale, bias
    (1, 4, 1, "f16", "f32", False, False),
    (7, 13, 1, "f16", "f32", True, True),
    (9, 37, 2, "bf16", "f16", False, True),
    (33, 100, 3, "f16", "bf16", True, False),
    (130, 4096, 1, "f16", "f16", True, True),
    (61, 4100, 4, "bf16", "f32", False, False),
    (8, 8191, 16, "f16", "f32", True, True),
    (700, 5000, 8, "bf16", "bf16", True, False),
    (1000, 16385, 1, "f16", "f32", False, True),   # second slice holds one vector
    (17, 20000, 5, "f16", "f32", True, False),
    (2, 70000, 1, "bf16", "f32", False, False),    # five slices
    (16500, 64, 1, "f16", "f32", True, True),      # four rows per wavefront
    (16390, 36, 16, "bf16", "f16", False, True),   # four rows per wavefront, M = 16
    (16385, 520, 7, "f16", "f32", True, False),
    (300, 28670, 1, "bf16", "f32", True, True),    # M = 1, seven slices resident in LDS
    (9000, 28673, 1, "f16", "f32", False, True),   # M = 1, eight slices: the sliced pass
    (8200, 4098, 1, "f16", "bf16", True, False),   # M = 1, two rows per wavefront, ragged
    # routing: from M = 4 the matrix-core kernel runs
    (300, 777, 3, "bf16", "f32", True, True),      # VALU
    (300, 777, 4, "bf16", "f32", True, True),      # matrix cores (one row block, eight K-streams)
    (12288, 130, 4, "f16", "f16", False, True),    # matrix cores (96 row blocks: four K-streams)
    (12300, 68, 3, "bf16", "bf16", True, False),   # VALU
    (2000, 1030, 12, "f16", "f32", True, False),   # matrix cores (16 row blocks)
]


@pytest.mark.parametrize("n,in_features,m,xd,yt,with_scale,with_bias", SHAPES)
def test_svq_gemv_parity_shapes(vq, n, in_features, m, xd, yt, with_scale, with_bias):
    lay = synth.make_svq_layer(n, in_features, with_scale=with_scale, with_bias=with_bias)
    dl = SvqLayer(vq, lay)
    x_bits = synth.activations(np.random.default_rng(n * 31 + in_features), m, in_features, xd)
    y = dl.gemv(vq, x_tensor(x_bits, xd), y_dtype=_tdtype(yt))
    torch.cuda.synchronize()
    check_y(y, _oracle_y(lay, x_bits, xd), yt)


GEMM_SHAPES = [
    # n, in_features, M, x dtype, y dtype, scale, bias
    (1, 4, 1, "f16", "f32", False, False),
    (7, 13, 3, "bf16", "f16", True, True),
    (33, 100, 17, "f16", "f32", True, False),
    (65, 4100, 40, "bf16", "bf16", False, True),
    (130, 127, 64, "f16", "f32", True, True),
    (300, 1000, 100, "bf16", "f32", True, False),
    (97, 2000, 129, "f16", "f16", False, True),
    (40, 64, 300, "bf16", "f32", True, True),      # two 256-row batch chunks
    (1000, 4096, 16, "f16", "f32", True, False),
]


@pytest.mark.parametrize("n,in_features,m,xd,yt,with_scale,with_bias", GEMM_SHAPES)
def test_svq_gemm_parity_shapes(vq, n, in_features, m, xd, yt, with_scale, with_bias):
    lay = synth.make_svq_layer(n, in_features, with_scale=with_scale, with_bias=with_bias)
    dl = SvqLayer(vq, lay)
    x_bits = synth.activations(np.random.default_rng(n * 17 + m), m, in_features, xd)
    y = dl.gemm(vq, x_tensor(x_bits, xd), y_dtype=_tdtype(yt))
    torch.cuda.synchronize()
    check_y(y, _oracle_y(lay, x_bits, xd), yt)


def test_svq_gemm_empty_inner_dimension_gives_bias(vq):
    lay = synth.make_svq_layer(50, 0, with_scale=True, with_bias=True)
    desc = vq.svq_desc(50, 0)
    x = torch.zeros((40, 0), dtype=torch.float16, device="cuda")
    bias = f16_tensor(lay["bias"])
    y = vq.svq_gemm(desc, torch.zeros(16, dtype=torch.uint8, device="cuda"), None, None, None, bias, x,
                    y_dtype=torch.float32)
    torch.cuda.synchronize()
    want = lay["bias"].view(np.float16).astype(np.float32)
    assert np.array_equal(y.cpu().numpy(), np.broadcast_to(want, (40, 50)))


@functools.lru_cache(maxsize=2)
def _svq_workload(key, layer):
    import gemv_bit_unpack_amd as g

    lay = synth.svq_workload_layer(key, layer)
    return lay, SvqLayer(g, lay)


@pytest.mark.parametrize("key,layer,m", [
    ("svq4k", 0, 1), ("svq4k", 0, 4), ("svq4k", 0, 16),
    ("svq70b", 0, 1), ("svq70b", 0, 8), ("svq70b", 1, 1), ("svq70b", 1, 8),
])
def test_svq_gemv_workloads_sampled(vq, key, layer, m):
    lay, dl = _svq_workload(key, layer)
    xd = synth.SVQ_WORKLOADS[key].x_dtype
    x_bits = synth.svq_workload_x(key, layer, m)
    y = dl.gemv(vq, x_tensor(x_bits, xd), y_dtype=torch.float32).cpu().numpy()
    rows = sample_rows(lay["n"], 48, seed=layer + 7 * m)
    y64 = _oracle_y(lay, x_bits, xd, rows=rows)
    check_y(y[:, rows], y64, "f32")


@pytest.mark.parametrize("key,layer,m", [("svq4k", 0, 64), ("svq70b", 0, 128), ("svq70b", 1, 128)])
def test_svq_gemm_workloads_sampled(vq, key, layer, m):
    lay, dl = _svq_workload(key, layer)
    xd = synth.SVQ_WORKLOADS[key].x_dtype
    x_bits = synth.activations(np.random.default_rng(1000 + layer + m), m, lay["in_features"], xd)
    y = dl.gemm(vq, x_tensor(x_bits, xd), y_dtype=torch.float32).cpu().numpy()
    rows = sample_rows(lay["n"], 24, seed=layer + 3 * m)
    y64 = _oracle_y(lay, x_bits, xd, rows=rows)
    check_y(y[:, rows], y64, "f32")


@pytest.mark.parametrize("in_features", [4096, 5003, 20000])
def test_svq_one_hot_dyadic_grid_exact(vq, in_features):
    """With A, B on a coarse dyadic grid every product and partial sum is exact in fp32, so
    a one-hot x returns a column of W^ bit for bit."""
    g = np.random.default_rng(in_features)
    n = 257
    lay = synth.make_svq_layer(n, in_features, with_scale=False)
    lay["a"] = g.choice([-0.5, -0.25, 0.0, 0.25, 0.5], size=(4, 4)).astype(np.float16).view(np.uint16)
    lay["b"] = g.choice([-1.0, -0.5, 0.5, 1.0], size=4).astype(np.float16).view(np.uint16)
    dl = SvqLayer(vq, lay)
    w_ref = _oracle_w(lay)
    cols = [0, 1, 2, 3, in_features // 2, in_features - 1]
    x_bits = np.zeros((len(cols), in_features), dtype=np.uint16)
    for i, c in enumerate(cols):
        x_bits[i, c] = np.float16(1.0).view(np.uint16)
    y = dl.gemv(vq, x_tensor(x_bits, "f16"), y_dtype=torch.float32).cpu().numpy()
    for i, c in enumerate(cols):
        assert np.array_equal(y[i], w_ref[:, c]), c


def test_svq_deterministic_and_graph_replays(vq):
    lay = synth.make_svq_layer(8192, 8192, with_scale=True, with_bias=True)
    dl = SvqLayer(vq, lay)
    x = x_tensor(synth.activations(np.random.default_rng(5), 1, 8192, "f16"), "f16")
    y0 = dl.gemv(vq, x, y_dtype=torch.float32)
    y1 = dl.gemv(vq, x, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    out = torch.empty_like(y0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        vq.svq_gemv(dl.desc, dl.packed, dl.a, dl.b, dl.scale, dl.bias, x, out=out)  # warm-up on the stream
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        vq.svq_gemv(dl.desc, dl.packed, dl.a, dl.b, dl.scale, dl.bias, x, out=out)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y0), rep
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
