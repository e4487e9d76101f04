"""GPU parity of vq_gemv_ws, the codebook-sliced GEMV for the 65536-entry main book,
against the CPU oracle, through the C ABI.

- the workloads with that book (4096^2 with and without the 256-entry residual book,
  the 70B-style up / down layers) at every decode batch M <= 16 they list, on sampled
  rows at full size (the 4096^2 layers at M = 1 take the vq_gemv kernels: same check);
- shapes with ragged row counts, ragged last chunks (down to 1 vector), column
  splits, M from 1 to 16, bias / no scale, every output dtype;
- a one-hot x reproduces columns of W^ bit-exactly;
- bf16 activations beyond the fp16 range, and tiny ones;
- determinism, workspace reuse across shapes, the fallbacks (no workspace,
  misaligned x, a shape without the sliced path) and replays of a captured graph.
Tolerance: max |y - y64| <= 2e-3 * ||y64||_inf with fp32 outputs, plus half an output
ulp for fp16 / bf16 outputs.
"""
import functools

import numpy as np
import pytest

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


@functools.lru_cache(maxsize=4)
def _workload_layer(key, layer):
    return synth.workload_layer(key, layer)


@functools.lru_cache(maxsize=4)
def _device_workload(key, layer):
    import gemv_bit_unpack_amd as g

    return DeviceLayer(g, _workload_layer(key, layer))


def _tdtype(xd):
    return torch.bfloat16 if xd == "bf16" else torch.float16


def _ws_for(vq, dl, m, xd):
    ws = vq.workspace(dl.desc, m, _tdtype(xd))
    assert ws is not None, "shape %s should have the sliced path" % dl.desc
    return ws


def _ws_or_none(vq, dl, m, xd):
    return vq.workspace(dl.desc, m, _tdtype(xd))


SLICED_WL = [(k, i, m) for k in ("dec4k", "dec4k_res", "l70b") for i in range(len(synth.WORKLOADS[k].layers))
             for m in synth.WORKLOADS[k].ms if m <= 16]


@pytest.mark.parametrize("key,layer,m", SLICED_WL)
def test_gemv_ws_parity_workloads(vq, key, layer, m):
    print("gemv_ws", key, layer, m, flush=True)
    w = synth.WORKLOADS[key]
    lay = _workload_layer(key, layer)
    dl = _device_workload(key, layer)
    xb = synth.workload_x(key, layer, m)
    x = x_tensor(xb, w.x_dtype)
    rows = None if key != "l70b" else sample_rows(lay["n"], 64, seed=lay["n"] + m)
    y64 = oracle_y(lay, xb, w.x_dtype, rows)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, torch.from_numpy(rows).cuda()])
    ws = _ws_or_none(vq, dl, m, w.x_dtype)
    assert (ws is not None) == (m >= 8 or key == "l70b")  # 4096^2 has 2^21 vectors
    check_y(sel(vq.gemv_ws(*dl.args(), x, ws, y_dtype=torch.float32)), y64, "f32")
    check_y(sel(vq.gemv_ws(*dl.args(), x, ws)), y64, w.x_dtype)


@pytest.mark.parametrize("n,i,b2,m,xd,bias,scale", [
    (8200, 4096, 8, 1, "bf16", False, True),    # ragged last row block
    (4096, 8200, 0, 1, "f16", True, True),      # nv = 1025: last chunk holds one vector
    (4101, 1024, 0, 8, "bf16", True, False),
    (4096, 1280, 8, 12, "f16", False, True),
    (1100, 4096, 8, 9, "bf16", True, True),
    (8300, 512, 8, 16, "f16", True, True),
    (600, 7168, 0, 10, "f16", False, True),     # few row blocks: column splits fill the groups
    (1024, 32768, 8, 2, "bf16", True, True),    # 128 chunks per row; 2^22 vectors
])
def test_gemv_ws_parity_shapes(vq, n, i, b2, m, xd, bias, scale):
    print("gemv_ws shape", n, i, b2, m, xd, flush=True)
    lay = synth.make_layer(n, i, 8, 16, b2, wid=81, copy=n + i + m, with_scale=scale, with_bias=bias)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n + i + m), m, i, xd)
    x = x_tensor(xb, xd)
    rows = sample_rows(n, 96, seed=n + m)
    y64 = oracle_y(lay, xb, xd, rows)
    sel = lambda t: t[:, torch.from_numpy(rows).cuda()]
    ws = _ws_for(vq, dl, m, xd)
    check_y(sel(vq.gemv_ws(*dl.args(), x, ws, y_dtype=torch.float32)), y64, "f32")
    for yt, name in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        check_y(sel(vq.gemv_ws(*dl.args(), x, ws, y_dtype=yt)), y64, name)


@pytest.mark.parametrize("b2", [0, 8])
def test_gemv_ws_one_hot_columns_bit_exact(vq, b2):
    """x = e_col gives y[o] = s_o * (c1 + c2)[col], the exact fp32 W^ entry."""
    n, i = 2176, 256 * 9  # M = 8 below: sliced from 2^19 vectors
    lay = synth.make_layer(n, i, 8, 16, b2, wid=82, copy=b2)
    dl = DeviceLayer(vq, lay)
    cols = np.array([0, 7, 8, 131, 1031, 1500, 2048, i - 1])
    w32 = oracle_w(lay)[:, cols]
    xb = np.zeros((cols.size, i), dtype=np.uint16)
    xb[np.arange(cols.size), cols] = 0x3C00  # 1.0
    ws = _ws_for(vq, dl, cols.size, "f16")
    y = vq.gemv_ws(*dl.args(), x_tensor(xb, "f16"), ws, y_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(y, w32.T)


@functools.lru_cache(maxsize=1)
def _range_layer():
    import gemv_bit_unpack_amd as g

    lay = synth.make_layer(4096, 8192, 8, 16, 8, wid=83, with_bias=False)  # 2^22 vectors: sliced from M = 1
    return lay, DeviceLayer(g, lay)


@pytest.mark.parametrize("pick", [[4], [0, 2], [3, 1], list(range(8))])
def test_gemv_ws_bf16_outside_fp16_range(vq, pick):
    """Rows with values up to 3e5 (beyond fp16), rows of tiny values (4e-6 and 1e-12, the
    second below the smallest fp16 subnormal), and a zero row; M = 1 and 2 convert x inside
    the product kernel, M = 8 in the separate pass.  No bias, so each batch row's error is
    measured against its own product alone."""
    lay, dl = _range_layer()
    i = lay["in_features"]
    g = np.random.default_rng(83)
    xf = g.standard_normal((8, i)).astype(np.float32)
    xf[0] *= 1e5
    xf[1, ::7] *= 3e5
    xf[2] *= 1e-6
    xf[3] = 0.0
    xf[4] *= 1e-12
    xf = xf[pick]
    m = len(pick)
    xb = synth.f32_to_bf16_bits(xf)
    y64 = oracle_y(lay, xb, "bf16")
    ws = _ws_for(vq, dl, m, "bf16")
    y = vq.gemv_ws(*dl.args(), x_tensor(xb, "bf16"), ws, y_dtype=torch.float32)
    for r in range(m):  # each batch row against its own scale
        check_y(y[r:r + 1], y64[r:r + 1], "f32", norm=max(float(np.abs(y64[r]).max()), 1e-37))
        if pick[r] == 3:
            assert not torch.any(y[r] != 0)  # the zero row gives exact zeros


def test_gemv_ws_deterministic_and_reusable(vq):
    a = synth.make_layer(8192, 4096, 8, 16, 8, wid=84, with_bias=True)
    b = synth.make_layer(1536, 8192, 8, 16, 0, wid=85)
    da, db = DeviceLayer(vq, a), DeviceLayer(vq, b)
    xa = synth.activations(np.random.default_rng(1), 1, 4096, "f16")
    xbits = synth.activations(np.random.default_rng(2), 8, 8192, "f16")
    need = max(vq.gemv_workspace_bytes(da.desc, 1, torch.float16), vq.gemv_workspace_bytes(db.desc, 8, torch.float16))
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # contents need no initialisation
    ya1 = vq.gemv_ws(*da.args(), x_tensor(xa, "f16"), ws, y_dtype=torch.float32)
    yb = vq.gemv_ws(*db.args(), x_tensor(xbits, "f16"), ws, y_dtype=torch.float32)
    ya2 = vq.gemv_ws(*da.args(), x_tensor(xa, "f16"), ws, y_dtype=torch.float32)
    fresh = torch.zeros_like(ws)
    ya3 = vq.gemv_ws(*da.args(), x_tensor(xa, "f16"), fresh, y_dtype=torch.float32)
    assert torch.equal(ya1, ya2) and torch.equal(ya1, ya3)
    rows_a = sample_rows(8192, 96, seed=4)
    check_y(ya1[:, torch.from_numpy(rows_a).cuda()], oracle_y(a, xa, "f16", rows_a), "f32")
    rows = sample_rows(1536, 64, seed=3)
    check_y(yb[:, torch.from_numpy(rows).cuda()], oracle_y(b, xbits, "f16", rows), "f32")


def test_gemv_ws_fallbacks(vq):
    lay = synth.make_layer(8192, 4096, 8, 16, 0, wid=86)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(4), 1, 4096, "f16")
    y64 = oracle_y(lay, xb, "f16")
    x = x_tensor(xb, "f16")
    check_y(vq.gemv_ws(*dl.args(), x, None, y_dtype=torch.float32), y64, "f32")  # no workspace: vq_gemv
    buf = torch.empty(4096 + 8, dtype=torch.float16, device="cuda")
    xm = buf[1:4097].view(1, 4096)  # 2-byte aligned: the sliced path does not apply
    xm.copy_(x[0])
    ws = _ws_for(vq, dl, 1, "f16")
    ws.fill_(0x5A)
    check_y(vq.gemv_ws(*dl.args(), xm, ws, y_dtype=torch.float32), y64, "f32")
    assert bool((ws == 0x5A).all())  # untouched
    small = synth.make_layer(256, 256, 8, 16, 8, wid=87, with_bias=True)  # too small for the sliced path
    ds = DeviceLayer(vq, small)
    xs = synth.activations(np.random.default_rng(5), 2, 256, "bf16")
    check_y(vq.gemv_ws(*ds.args(), x_tensor(xs, "bf16"), ws, y_dtype=torch.float32), oracle_y(small, xs, "bf16"),
            "f32")
    layer = vq.VQLinear(dl.desc, dl.packed, dl.cb1, dl.cb2, dl.scale, dl.bias)
    check_y(layer(x, y_dtype=torch.float32), y64, "f32")


def test_gemv_ws_graph_replays(vq):
    """Captured once, replayed with new activations and eager work in between."""
    lay = synth.make_layer(8192, 4096, 8, 16, 8, wid=88, with_bias=True)
    dl = DeviceLayer(vq, lay)
    xs = [synth.activations(np.random.default_rng(10 + k), 1, 4096, "f16") for k in range(3)]
    refs = [oracle_y(lay, xb, "f16") for xb in xs]
    ws = _ws_for(vq, dl, 1, "f16")
    x = x_tensor(xs[0], "f16")
    y = torch.empty((1, 8192), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        vq.gemv_ws(*dl.args(), x, ws, out=y)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vq.gemv_ws(*dl.args(), x, ws, out=y)
    for k in (0, 1, 2, 0):
        x.copy_(x_tensor(xs[k], "f16"))
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        check_y(y, refs[k], "f32")
