"""GPU parity of the products with the randomized Hadamard transform fused ahead of them
(vq_gemv_ws_rht, vq_gemm_ws_rht) against the oracle: the oracle's transform of x (fp64,
`oracle_rht`) followed by the oracle's product definition (its exact fp32 W^ rows times
x~ in fp64, plus bias), on sampled rows.

- the fused x pass on the workspace paths: the 70B-class up layer (one 8192-column block)
  and down layer (seven blocks of 4096) at M = 1 and 8 through vq_gemv_ws_rht, and at
  M = 128 through vq_gemm_ws_rht, bf16 and fp16 activations;
- the separate transform where no workspace path exists (the 4096^2 layer at M = 1, a
  v = 6 layer): x~ rounded to the activation type, then vq_gemv / vq_gemm; compared with
  the oracle product of x~ rounded the same way;
- the fused path equals vq_rht followed by vq_gemv_ws to the tolerance, and the argument
  checks (IN not a multiple of 16, no workspace, too small a workspace).
Tolerance: max |y - y64| <= 2e-3 * ||y64||_inf (fp32 outputs).
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


@functools.lru_cache(maxsize=2)
def _l70b(layer):
    import gemv_bit_unpack_amd as g

    lay = synth.workload_layer("l70b", layer)
    return lay, DeviceLayer(g, lay)


def _signs(n, seed):
    return np.random.default_rng(seed).integers(0, 256, (n + 7) // 8, dtype=np.uint8)


def _x64(xb, xd):
    return oracle.bf16_to_f64(xb) if xd == "bf16" else oracle.f16_to_f64(xb)


def _ref_fused(lay, xb, xd, signs, rows):
    """y64 = x~ W^[rows]^T + bias, x~ = the oracle's transform of x in fp64."""
    xt = oracle.rht(_x64(xb, xd).reshape(xb.shape), signs)
    w = oracle_w(lay, rows).astype(np.float64)
    y = xt @ w.T
    if lay["bias"] is not None:
        y = y + oracle.f16_to_f64(lay["bias"])[rows][None, :]
    return y


def _tdtype(xd):
    return torch.bfloat16 if xd == "bf16" else torch.float16


@pytest.mark.parametrize("layer,m,xd,gemm", [(0, 1, "bf16", False), (1, 1, "bf16", False), (0, 8, "bf16", False),
                                             (1, 2, "f16", False), (0, 128, "bf16", True), (1, 40, "f16", True)])
def test_fused_rht_products_70b(vq, layer, m, xd, gemm):
    print("rht fused", layer, m, xd, gemm, flush=True)
    lay, dl = _l70b(layer)
    i = lay["in_features"]
    xb = synth.activations(np.random.default_rng(50 + m + layer), m, i, xd)
    sg = _signs(i, 7 + layer)
    rows = sample_rows(lay["n"], 40, seed=m + layer)
    y64 = _ref_fused(lay, xb, xd, sg, rows)
    ws = vq.rht_workspace(dl.desc, m, _tdtype(xd), gemm)
    fn = vq.gemm_ws_rht if gemm else vq.gemv_ws_rht
    y = fn(*dl.args(), x_tensor(xb, xd), torch.from_numpy(sg).cuda(), ws, y_dtype=torch.float32)
    check_y(y[:, torch.from_numpy(rows).cuda()], y64, "f32")


def test_fused_matches_separate_transform(vq):
    lay, dl = _l70b(0)
    i = lay["in_features"]
    xb = synth.activations(np.random.default_rng(3), 2, i, "f16")
    sg = torch.from_numpy(_signs(i, 9)).cuda()
    x = x_tensor(xb, "f16")
    xt = vq.rht(x, sg, y_dtype=torch.float32)  # fp32 transform, then the plain workspace product
    ws = vq.rht_workspace(dl.desc, 2, torch.float16, False)
    y_fused = vq.gemv_ws_rht(*dl.args(), x, sg, ws, y_dtype=torch.float32)
    rows = sample_rows(lay["n"], 40, seed=11)
    y64 = _ref_fused(lay, xb, "f16", _signs(i, 9), rows)
    check_y(y_fused[:, torch.from_numpy(rows).cuda()], y64, "f32")
    # the separate route (transform rounded to fp16, then vq_gemv_ws) lands within the tolerance too
    y_sep = vq.gemv_ws(*dl.args(), xt.to(torch.float16), vq.workspace(dl.desc, 2, torch.float16), y_dtype=torch.float32)
    check_y(y_sep[:, torch.from_numpy(rows).cuda()], y64, "f32")


@pytest.mark.parametrize("n,i,v,b1,b2,m,xd,gemm", [
    (4096, 4096, 8, 16, 0, 1, "f16", False),     # 2^21 vectors: no codebook-sliced path
    (300, 1024, 6, 12, 12, 3, "bf16", False),    # v = 6
    (260, 2048, 6, 12, 12, 48, "f16", True),     # v = 6 prefill: no gather path
])
def test_separate_transform_without_workspace_path(vq, n, i, v, b1, b2, m, xd, gemm):
    """x~ is rounded to the activation type, then the plain product runs on it."""
    lay = synth.make_layer(n, i, v, b1, b2, wid=57, copy=n + m, with_bias=True)
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(n + i), m, i, xd)
    sg = _signs(i, n)
    xt = oracle.rht(_x64(xb, xd).reshape(xb.shape), sg)
    xtb = oracle.f64_to_bf16_rne(xt) if xd == "bf16" else oracle.f64_to_f16_rne(xt)
    rows = sample_rows(n, 48, seed=n)
    y64 = oracle_y(lay, xtb.reshape(m, i), xd, rows)
    ws = vq.rht_workspace(dl.desc, m, _tdtype(xd), gemm)
    assert ws is not None and ws.numel() >= m * i * 2
    fn = vq.gemm_ws_rht if gemm else vq.gemv_ws_rht
    y = fn(*dl.args(), x_tensor(xb, xd), torch.from_numpy(sg).cuda(), ws, y_dtype=torch.float32)
    check_y(y[:, torch.from_numpy(rows).cuda()], y64, "f32")


def test_fused_argument_checks(vq):
    lay = synth.make_layer(512, 1000, 8, 16, 0, wid=58)  # IN = 1000: not a multiple of 16
    dl = DeviceLayer(vq, lay)
    x = x_tensor(synth.activations(np.random.default_rng(1), 1, 1000, "f16"), "f16")
    sg = torch.zeros(125, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(vq.VQError) as err:
        vq.gemv_ws_rht(*dl.args(), x, sg, ws)
    assert err.value.status == vq.VQ_ERR_UNSUPPORTED
    lay2, dl2 = _l70b(0)
    x2 = x_tensor(synth.activations(np.random.default_rng(2), 1, 8192, "bf16"), "bf16")
    sg2 = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(vq.VQError) as err:
        vq.gemv_ws_rht(*dl2.args(), x2, sg2, None)
    assert err.value.status == vq.VQ_ERR_NULL
    need = vq.rht_product_workspace_bytes(dl2.desc, 1, torch.bfloat16, False)
    with pytest.raises(vq.VQError) as err:
        vq.gemv_ws_rht(*dl2.args(), x2, sg2, torch.zeros(need - 256, dtype=torch.uint8, device="cuda"))
    assert err.value.status == vq.VQ_ERR_BUFFER_SIZE
