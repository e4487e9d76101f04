"""GPU parity of the batch-1 decode product over the slice-bucketed layout (vq_gemv_ws
and vq_gemv_noalloc with a VQ_LAYOUT_BUCKETED descriptor) against the CPU oracle, through
the C ABI.

The layer is packed twice from the same seeded indices: by the library into the bucketed
layout (what the kernel reads) and by the oracle into the row stream (what the oracle
reads); nothing the GPU computes reaches the oracle.
- the 70B-class up and down layers at full size, bf16 and fp16 x, sampled rows;
- ragged shapes: row counts off the 64-row tile, a last chunk of one vector, fewer units
  than workgroup groups, no residual book, bias, no scale, every output dtype;
- buckets longer than the 192 words held in registers (rows whose indices all fall in
  one slice) and empty buckets;
- one-hot x reproduces columns of W^ bit-exactly;
- bf16 activations far outside the fp16 range and tiny ones;
- determinism, vq_gemv_noalloc equal bit for bit, IN = 0, replays of a captured graph;
- VQLinear holding both layouts (one-row batches on the bucketed product).
Tolerance: max |y - y64| <= 2e-3 * ||y64||_inf with fp32 outputs, plus half an output ulp
for fp16 / bf16 outputs.
"""
import functools

import numpy as np
import pytest

import synth
from vqtest import check_y, f16_tensor, oracle_w, oracle_y, sample_rows, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


class BucketedLayer:
    """A layer packed by the library into the slice-bucketed layout and uploaded."""

    def __init__(self, vq, lay):
        self.lay = lay
        self.desc = vq.make_desc(lay["n"], lay["in_features"], 8, 16, lay["bits2"], vq.LAYOUT_BUCKETED)
        self.packed = torch.from_numpy(vq.pack(self.desc, lay["idx1"], lay["idx2"])).cuda()
        self.cb1 = f16_tensor(lay["cb1"])
        self.cb2 = f16_tensor(lay["cb2"])
        self.scale = f16_tensor(lay["scale"])
        self.bias = f16_tensor(lay["bias"])

    def args(self):
        return (self.desc, self.packed, self.cb1, self.cb2, self.scale, self.bias)


@functools.lru_cache(maxsize=2)
def _workload(layer):
    import gemv_bit_unpack_amd as g

    lay = synth.workload_layer("l70b", layer)
    return lay, BucketedLayer(g, lay)


def _tdtype(xd):
    return torch.bfloat16 if xd == "bf16" else torch.float16


def _run(vq, bl, x, y_dtype=torch.float32):
    ws = vq.workspace(bl.desc, 1, x.dtype)
    assert ws is not None
    return vq.gemv_ws(*bl.args(), x, ws, y_dtype=y_dtype)


@pytest.mark.parametrize("layer", [0, 1])
@pytest.mark.parametrize("xd", ["bf16", "f16"])
def test_bucketed_parity_l70b(vq, layer, xd):
    print("bucketed l70b", layer, xd, flush=True)
    lay, bl = _workload(layer)
    xb = synth.workload_x("l70b", layer, 1) if xd == "bf16" else synth.activations(
        np.random.default_rng(layer), 1, lay["in_features"], "f16")
    x = x_tensor(xb, xd)
    rows = sample_rows(lay["n"], 96, seed=lay["n"] + 7)
    y64 = oracle_y(lay, xb, xd, rows)
    sel = lambda t: t[:, torch.from_numpy(rows).cuda()]
    check_y(sel(_run(vq, bl, x)), y64, "f32")
    check_y(sel(_run(vq, bl, x, _tdtype(xd))), y64, xd)


@pytest.mark.parametrize("n,i,b2,xd,bias,scale", [
    (100, 8192, 8, "bf16", True, True),     # fewer tiles than groups; ragged row tile
    (1000, 8200, 8, "f16", False, True),    # nv = 1025: last chunk holds one vector
    (4097, 1024, 0, "bf16", True, False),   # no residual book; one row past a tile
    (64, 24576, 8, "f16", True, True),      # three chunks, one tile
    (3, 16, 8, "bf16", False, True),        # two vectors per row
    (2500, 3000 * 8, 0, "f16", False, False),
])
def test_bucketed_parity_shapes(vq, n, i, b2, xd, bias, scale):
    print("bucketed shape", n, i, b2, xd, flush=True)
    lay = synth.make_layer(n, i, 8, 16, b2, wid=83, copy=n + i, with_scale=scale, with_bias=bias)
    bl = BucketedLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n + i), 1, i, xd)
    x = x_tensor(xb, xd)
    rows = sample_rows(n, 128, seed=n)
    y64 = oracle_y(lay, xb, xd, rows)
    sel = lambda t: t[:, torch.from_numpy(rows).cuda()]
    check_y(sel(_run(vq, bl, x)), y64, "f32")
    for yt, name in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        check_y(sel(_run(vq, bl, x, yt)), y64, name)


def test_bucketed_long_and_empty_buckets(vq):
    """Rows whose 1024 vectors per chunk all sit in one slice (buckets of 1024 words: the
    loop past the 192 held in registers), alternating slices, and ordinary rows."""
    n, i = 200, 8 * 2100
    lay = synth.make_layer(n, i, 8, 16, 8, wid=84, copy=1, with_bias=True)
    nv = i // 8
    g = np.random.default_rng(9)
    idx1 = lay["idx1"].copy()
    for o in range(0, n, 3):
        idx1[o] = ((o % 8) << 13) | g.integers(0, 8192, nv)
    idx1[1] = 0
    idx1[4, :700] = 65535
    lay = dict(lay, idx1=idx1.astype(np.uint32))
    bl = BucketedLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(1), 1, i, "bf16")
    y64 = oracle_y(lay, xb, "bf16")
    check_y(_run(vq, bl, x_tensor(xb, "bf16")), y64, "f32")


@pytest.mark.parametrize("b2", [0, 8])
def test_bucketed_one_hot_columns_bit_exact(vq, b2):
    """x = e_col gives y[o] = s_o * (c1 + c2)[col], the exact fp32 W^ entry."""
    n, i = 300, 8 * 1100
    lay = synth.make_layer(n, i, 8, 16, b2, wid=85, copy=b2)
    bl = BucketedLayer(vq, lay)
    w32 = oracle_w(lay)
    for col in (0, 7, 8, 1023 * 8 + 5, 1024 * 8, i - 1):
        for xd, one in (("f16", 0x3C00), ("bf16", 0x3F80)):
            xb = np.zeros((1, i), dtype=np.uint16)
            xb[0, col] = one
            y = _run(vq, bl, x_tensor(xb, xd)).cpu().numpy()[0]
            assert np.array_equal(y.view(np.uint32), w32[:, col].view(np.uint32)), (col, xd)


@pytest.mark.parametrize("scale_exp", [40, -40])
def test_bucketed_bf16_outside_fp16_range(vq, scale_exp):
    """bf16 rows of values near 1e12 or 1e-12 (no bias: y is all product)."""
    n, i = 512, 8192
    lay = synth.make_layer(n, i, 8, 16, 8, wid=86, copy=scale_exp & 0xFF, with_bias=False)
    bl = BucketedLayer(vq, lay)
    xf = np.random.default_rng(5).standard_normal((1, i)).astype(np.float32) * np.float32(2.0 ** scale_exp)
    xb = synth.f32_to_bf16_bits(xf)
    y64 = oracle_y(lay, xb, "bf16")
    check_y(_run(vq, bl, x_tensor(xb, "bf16")), y64, "f32")


def test_bucketed_deterministic_and_noalloc_equal(vq):
    lay, bl = _workload(1)
    xb = synth.workload_x("l70b", 1, 1)
    x = x_tensor(xb, "bf16")
    y0 = _run(vq, bl, x)
    y1 = _run(vq, bl, x)
    y2 = torch.empty_like(y0)
    vq.gemv_noalloc(*bl.args(), x, y_dtype=torch.float32, out=y2)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(y0, y2)


def test_bucketed_empty_input_gives_bias(vq):
    n = 96
    lay = synth.make_layer(n, 64, 8, 16, 8, wid=87, with_bias=True)
    desc = vq.make_desc(n, 0, 8, 16, 8, vq.LAYOUT_BUCKETED)
    bias = f16_tensor(lay["bias"])
    x = torch.zeros((1, 0), dtype=torch.float16, device="cuda")
    packed = torch.zeros(256, dtype=torch.uint8, device="cuda")
    y = vq.gemv_ws(desc, packed, f16_tensor(lay["cb1"]), f16_tensor(lay["cb2"]), None, bias, x, None,
                   y_dtype=torch.float32)
    assert torch.equal(y[0].cpu(), bias.float().cpu())


def test_bucketed_graph_replays(vq):
    """A captured call replayed several times, with eager work between, equals eager."""
    lay, bl = _workload(0)
    xb = synth.workload_x("l70b", 0, 1)
    x = x_tensor(xb, "bf16")
    ws = vq.workspace(bl.desc, 1, x.dtype)
    ref = vq.gemv_ws(*bl.args(), x, ws, y_dtype=torch.float32)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        vq.gemv_ws(*bl.args(), x, ws, y_dtype=torch.float32, out=out)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vq.gemv_ws(*bl.args(), x, ws, y_dtype=torch.float32, out=out)
    for k in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), k
        vq.gemv_ws(*bl.args(), x, ws, y_dtype=torch.float32)  # eager work between replays
        torch.cuda.synchronize()


def test_vqlinear_with_decode_layout(vq):
    """VQLinear keeping both layouts: one-row batches take the bucketed product, larger ones
    the row-stream calls; every batch size matches the oracle, and the one-row result is the
    bucketed call's exactly."""
    n, i = 1536, 4096
    lay = synth.make_layer(n, i, 8, 16, 8, wid=88, with_bias=True)
    f = lambda b: f16_tensor(b)
    layer = vq.VQLinear.from_indices(vq.make_desc(n, i, 8, 16, 8), lay["idx1"], lay["idx2"], f(lay["cb1"]),
                                     f(lay["cb2"]), f(lay["scale"]), f(lay["bias"]), decode_layout=True)
    assert layer.decode_desc.layout == vq.LAYOUT_BUCKETED
    for m in (1, 3, 40):
        xb = synth.activations(np.random.default_rng(m), m, i, "bf16")
        x = x_tensor(xb, "bf16")
        y = layer(x, y_dtype=torch.float32)
        check_y(y, oracle_y(lay, xb, "bf16"), "f32")
        if m == 1:
            bl = BucketedLayer(vq, lay)
            assert torch.equal(y, _run(vq, bl, x))
