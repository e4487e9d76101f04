"""GPU parity of vq_gemm_ws, the prefill product for the 65536-entry main book whose lanes
feed the matrix cores with the weight vectors they gather, against the CPU oracle,
through the C ABI.

- the workloads with that book (4096^2 with and without the 256-entry residual book,
  the 70B-style up / down layers) at prefill batches, on sampled rows at full size;
- shapes with ragged row blocks, ragged and odd K-tile counts, one and many K splits,
  batches across the 128-row chunk boundary, fp16 and bf16 activations, bias / no
  scale, every output dtype;
- a one-hot x returns the fp16-rounded weight times the scale bit-exactly;
- bf16 activations beyond the fp16 range and tiny ones;
- determinism, workspace reuse, the fallbacks (no workspace, misaligned x, a shape
  without the gather path, too small a workspace) and replays of a captured graph.
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


WL = [("dec4k", 0, 32), ("dec4k_res", 0, 40), ("l70b", 0, 32), ("l70b", 0, 128), ("l70b", 1, 128),
      ("l70b", 1, 256), ("l70b", 0, 17)]


@pytest.mark.parametrize("key,layer,m", WL)
def test_gemm_ws_parity_workloads(vq, key, layer, m):
    print("gemm_ws", key, layer, m, flush=True)
    w = synth.WORKLOADS[key]
    lay = _workload_layer(key, layer)
    dl = _device_workload(key, layer)
    xb = synth.activations(np.random.default_rng(2000 + m), m, lay["in_features"], w.x_dtype)
    x = x_tensor(xb, w.x_dtype)
    rows = sample_rows(lay["n"], 48, seed=lay["n"] + m) if key == "l70b" else None
    y64 = oracle_y(lay, xb, w.x_dtype, rows)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, torch.from_numpy(rows).cuda()])
    ws = vq.gemm_workspace(dl.desc, m, _tdtype(w.x_dtype))
    assert ws is not None  # bf16 x, or fp16 x on 16 row blocks (K split)
    check_y(sel(vq.gemm_ws(*dl.args(), x, ws, y_dtype=torch.float32)), y64, "f32")
    check_y(sel(vq.gemm_ws(*dl.args(), x, ws)), y64, w.x_dtype)


@pytest.mark.parametrize("n,i,b2,m,xd,bias,scale", [
    (300, 1000, 8, 33, "f16", True, True),      # ragged row block, IN % 128 = 104, many K splits
    (4100, 4104, 0, 129, "bf16", False, True),   # 33 K-tiles (odd), two batch chunks
    (5000, 136, 8, 7, "bf16", True, False),      # two K-tiles, one split
    (64, 8, 8, 300, "f16", True, True),          # IN = 8: one vector per row, three chunks, no split
    (50000, 512, 8, 128, "f16", False, True),    # 196 row blocks: no split, no workspace
    (257, 28672, 0, 64, "bf16", True, True),     # two row blocks, 16 K splits
])
def test_gemm_ws_parity_shapes(vq, n, i, b2, m, xd, bias, scale):
    print("gemm_ws shape", n, i, b2, m, xd, flush=True)
    lay = synth.make_layer(n, i, 8, 16, b2, wid=91, copy=n + i + m, with_scale=scale, with_bias=bias)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n + i + m), m, i, xd)
    x = x_tensor(xb, xd)
    rows = np.unique(np.concatenate([sample_rows(n, 64, seed=n + m), [0, n - 1]]))
    y64 = oracle_y(lay, xb, xd, rows)
    sel = lambda t: t[:, torch.from_numpy(rows).cuda()]
    ws = vq.gemm_workspace(dl.desc, m, _tdtype(xd))
    assert (ws is None) == (xd == "f16" and n in (50000, 64))  # fp16 x and no K split
    check_y(sel(vq.gemm_ws(*dl.args(), x, ws, y_dtype=torch.float32)), y64, "f32")
    for yt, name in ((torch.float16, "f16"), (torch.bfloat16, "bf16")):
        check_y(sel(vq.gemm_ws(*dl.args(), x, ws, y_dtype=yt)), y64, name)


@pytest.mark.parametrize("b2,xd", [(0, "f16"), (8, "f16"), (8, "bf16")])
def test_gemm_ws_one_hot_columns_bit_exact(vq, b2, xd):
    """x = e_col gives y[o] = fp32(fp16(c1 + c2)[col]) * s_o: the weight is rounded once to
    fp16 (nearest even) and everything after that is exact up to the scale's rounding."""
    n, i = 600, 1024
    lay = synth.make_layer(n, i, 8, 16, b2, wid=92, copy=b2)
    dl = DeviceLayer(vq, lay)
    cols = np.array([0, 7, 8, 127, 128, 513, 1000, i - 1] + list(range(200, 232)))
    nv = i // 8
    c1 = lay["cb1"].view(np.float16).reshape(-1, 8).astype(np.float32)
    w = c1[lay["idx1"].reshape(n, nv)].reshape(n, i)
    if b2:
        c2 = lay["cb2"].view(np.float16).reshape(-1, 8).astype(np.float32)
        w = w + c2[lay["idx2"].reshape(n, nv)].reshape(n, i)
    w16 = w.astype(np.float16).astype(np.float32)[:, cols]
    scale = lay["scale"].view(np.float16).astype(np.float32)
    expect = (w16 * scale[:, None]).astype(np.float32).T
    xb = np.zeros((cols.size, i), dtype=np.uint16)
    xb[np.arange(cols.size), cols] = 0x3C00 if xd == "f16" else 0x3F80  # 1.0
    ws = vq.gemm_workspace(dl.desc, cols.size, _tdtype(xd))
    y = vq.gemm_ws(*dl.args(), x_tensor(xb, xd), ws, y_dtype=torch.float32).cpu().numpy()
    assert np.array_equal(y, expect)
    # the fp16 rounding of the rebuilt weight stays inside the product tolerance
    assert np.abs(w16 * scale[:, None] - oracle_w(lay)[:, cols]).max() <= 2.0 ** -11 * np.abs(w).max() * 1.5


def test_gemm_ws_bf16_outside_fp16_range(vq):
    """Batch rows with values up to 3e5 (beyond fp16), rows of tiny values (4e-6 and 1e-12,
    below the smallest fp16 subnormal) and a zero row, each against its own scale."""
    lay = synth.make_layer(2048, 4096, 8, 16, 8, wid=93, with_bias=False)
    dl = DeviceLayer(vq, lay)
    g = np.random.default_rng(93)
    xf = g.standard_normal((40, 4096)).astype(np.float32)
    xf[0] *= 1e5
    xf[1, ::7] *= 3e5
    xf[2] *= 1e-6
    xf[3] = 0.0
    xf[4] *= 1e-12
    xb = synth.f32_to_bf16_bits(xf)
    rows = sample_rows(2048, 64, seed=93)
    y64 = oracle_y(lay, xb, "bf16", rows)
    ws = vq.gemm_workspace(dl.desc, 40, torch.bfloat16)
    y = vq.gemm_ws(*dl.args(), x_tensor(xb, "bf16"), ws, y_dtype=torch.float32)[:, torch.from_numpy(rows).cuda()]
    for r in range(40):
        check_y(y[r:r + 1], y64[r:r + 1], "f32", norm=max(float(np.abs(y64[r]).max()), 1e-37))
    assert not torch.any(y[3] != 0)  # the zero row gives exact zeros


def test_gemm_ws_deterministic_and_reusable(vq):
    a = synth.make_layer(1024, 8192, 8, 16, 8, wid=94, with_bias=True)  # K split: partial sums
    b = synth.make_layer(600, 2048, 8, 16, 0, wid=95)
    da, db = DeviceLayer(vq, a), DeviceLayer(vq, b)
    xa = synth.activations(np.random.default_rng(1), 64, 8192, "bf16")
    xbits = synth.activations(np.random.default_rng(2), 200, 2048, "bf16")
    need = max(vq.gemm_workspace_bytes(da.desc, 64, torch.bfloat16),
               vq.gemm_workspace_bytes(db.desc, 200, torch.bfloat16))
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # contents need no initialisation
    ya1 = vq.gemm_ws(*da.args(), x_tensor(xa, "bf16"), ws, y_dtype=torch.float32)
    yb = vq.gemm_ws(*db.args(), x_tensor(xbits, "bf16"), ws, y_dtype=torch.float32)
    ya2 = vq.gemm_ws(*da.args(), x_tensor(xa, "bf16"), ws, y_dtype=torch.float32)
    ya3 = vq.gemm_ws(*da.args(), x_tensor(xa, "bf16"), torch.zeros_like(ws), y_dtype=torch.float32)
    assert torch.equal(ya1, ya2) and torch.equal(ya1, ya3)
    rows_a = sample_rows(1024, 64, seed=4)
    check_y(ya1[:, torch.from_numpy(rows_a).cuda()], oracle_y(a, xa, "bf16", rows_a), "f32")
    rows = sample_rows(600, 64, seed=3)
    check_y(yb[:, torch.from_numpy(rows).cuda()], oracle_y(b, xbits, "bf16", rows), "f32")


@pytest.mark.parametrize("xd", ["bf16", "f16"])
def test_gemm_ws_two_splits_ragged_chunks(vq, xd):
    """Two K splits over 90 row blocks of 224 rows (the last ragged) x two batch chunks
    (128 + 72 rows), bf16 and fp16 activations; repeated calls on a workspace filled with
    garbage give identical results (the partial sums are added in a fixed order)."""
    c = synth.make_layer(20000, 2048, 8, 16, 8, wid=96, with_scale=True, with_bias=True)
    dc = DeviceLayer(vq, c)
    xc = synth.activations(np.random.default_rng(5), 200, 2048, xd)
    need = vq.gemm_workspace_bytes(dc.desc, 200, _tdtype(xd))
    assert need >= 2 * 200 * 20000 * 4
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    y1 = vq.gemm_ws(*dc.args(), x_tensor(xc, xd), ws, y_dtype=torch.float32)
    y2 = vq.gemm_ws(*dc.args(), x_tensor(xc, xd), ws, y_dtype=torch.float32)
    ws.fill_(0xFF)
    y3 = vq.gemm_ws(*dc.args(), x_tensor(xc, xd), ws, y_dtype=torch.float32)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    rows = np.unique(np.concatenate([sample_rows(20000, 64, seed=6), [0, 223, 224, 19935, 19999]]))
    check_y(y1[:, torch.from_numpy(rows).cuda()], oracle_y(c, xc, xd, rows), "f32")


def test_gemm_ws_fallbacks(vq):
    lay = synth.make_layer(512, 4096, 8, 16, 8, wid=96, with_bias=True)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(4), 48, 4096, "bf16")
    rows = sample_rows(512, 64, seed=5)
    y64 = oracle_y(lay, xb, "bf16", rows)
    sel = lambda t: t[:, torch.from_numpy(rows).cuda()]
    x = x_tensor(xb, "bf16")
    check_y(sel(vq.gemm_ws(*dl.args(), x, None, y_dtype=torch.float32)), y64, "f32")  # no workspace: vq_gemm
    need = vq.gemm_workspace_bytes(dl.desc, 48, torch.bfloat16)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    buf = torch.empty(48 * 4096 + 8, dtype=torch.bfloat16, device="cuda")
    xm = buf[1:48 * 4096 + 1].view(48, 4096)  # 2-byte aligned: the gather path does not apply
    xm.copy_(x)
    check_y(sel(vq.gemm_ws(*dl.args(), xm, ws, y_dtype=torch.float32)), y64, "f32")
    assert bool((ws == 0x5A).all())  # untouched
    with pytest.raises(vq.VQError) as err:
        vq.gemm_ws(*dl.args(), x, ws[:need - 256], y_dtype=torch.float32)
    assert err.value.status == vq.VQ_ERR_BUFFER_SIZE
    small = synth.make_layer(256, 256, 6, 12, 0, wid=97, with_bias=True)  # v = 6: no gather path
    ds = DeviceLayer(vq, small)
    assert vq.gemm_workspace_bytes(ds.desc, 48, torch.bfloat16) == 0
    xs = synth.activations(np.random.default_rng(5), 48, 256, "bf16")
    check_y(vq.gemm_ws(*ds.args(), x_tensor(xs, "bf16"), ws, y_dtype=torch.float32), oracle_y(small, xs, "bf16"),
            "f32")
    layer = vq.VQLinear(dl.desc, dl.packed, dl.cb1, dl.cb2, dl.scale, dl.bias)
    check_y(sel(layer(x, y_dtype=torch.float32)), y64, "f32")


def test_gemm_ws_graph_replays(vq):
    """Captured once (x pass, product, partial-sum pass), replayed with new activations and
    eager work in between."""
    lay = synth.make_layer(1024, 4096, 8, 16, 8, wid=98, with_bias=True)
    dl = DeviceLayer(vq, lay)
    xs = [synth.activations(np.random.default_rng(20 + k), 64, 4096, "bf16") for k in range(3)]
    rows = sample_rows(1024, 48, seed=6)
    refs = [oracle_y(lay, xb, "bf16", rows) for xb in xs]
    ws = vq.gemm_workspace(dl.desc, 64, torch.bfloat16)
    x = x_tensor(xs[0], "bf16")
    y = torch.empty((64, 1024), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        vq.gemm_ws(*dl.args(), x, ws, out=y)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vq.gemm_ws(*dl.args(), x, ws, out=y)
    for k in (0, 1, 2, 0):
        x.copy_(x_tensor(xs[k], "bf16"))
        junk = torch.randn(1 << 16, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        check_y(y[:, torch.from_numpy(rows).cuda()], refs[k], "f32")
