"""GPU parity of vq_rht, the randomized Walsh-Hadamard transform of the activations (QuIP#
incoherence processing), against the CPU oracle through the C ABI.

- forward and transpose on row lengths with one block (16 ... 16384 columns) and with
  several (48, 14336, 28672, 32768), batches of 1, 3 and 16 rows, fp16 / bf16 / fp32 in
  and out;
- the round trip (forward, then transpose) returns x, in place as well;
- orthogonality: the transform keeps each block's norm.
Tolerance: the fast transform in fp32 adds at most one rounding per stage to values bounded
by the block's norm, so |y - y64| <= 2 (L + 2) 2^-24 ||x_block||_2 with L = log2(block),
plus half an output ulp for fp16 / bf16 outputs.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from vqtest import half_ulp, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(m, n, xd, seed):
    g = np.random.default_rng(seed)
    if xd == "f32":
        xf = g.standard_normal((m, n)).astype(np.float32)
        xt = torch.from_numpy(xf).cuda()
        x64 = xf.astype(np.float64)
    else:
        bits = synth.activations(g, m, n, xd)
        xt = x_tensor(bits, xd)
        x64 = (oracle.bf16_to_f64 if xd == "bf16" else oracle.f16_to_f64)(bits).reshape(m, n)
    signs = g.integers(0, 256, size=(n + 7) // 8, dtype=np.uint8)
    return xt, x64, signs


def _check(y, y64, x64, yd):
    n = x64.shape[1]
    b = oracle.rht_block(n)
    L = int(math.log2(b))
    norms = np.sqrt((x64.reshape(x64.shape[0], -1, b) ** 2).sum(axis=2))       # [M, blocks]
    tol = 2 * (L + 2) * 2.0 ** -24 * np.repeat(norms, b, axis=1)
    if yd != "f32":
        tol = tol + half_ulp(y64, yd)
    yn = y.float().cpu().numpy().astype(np.float64)
    err = np.abs(yn - y64)
    assert np.all(err <= tol), "max excess %.3e" % float((err - tol).max())


@pytest.mark.parametrize("m,n,xd,yd", [
    (1, 16, "f16", "f32"), (3, 48, "f32", "f32"), (1, 256, "bf16", "bf16"), (16, 4096, "f16", "f16"),
    (3, 14336, "bf16", "f32"), (1, 16384, "f32", "f32"), (2, 28672, "f16", "bf16"), (1, 32768, "bf16", "f32"),
    (16, 8192, "f16", "f32"), (5, 2064, "f32", "f16"),
])
@pytest.mark.parametrize("transpose", [False, True])
def test_rht_parity(vq, m, n, xd, yd, transpose):
    xt, x64, signs = _inputs(m, n, xd, seed=n + m)
    y = vq.rht(xt, torch.from_numpy(signs).cuda(), transpose=transpose, y_dtype=_DT[yd])
    torch.cuda.synchronize()
    _check(y, oracle.rht(x64, signs, transpose=transpose), x64, yd)


@pytest.mark.parametrize("n", [64, 4096, 14336])
def test_rht_round_trip_in_place_and_norm(vq, n):
    xt, x64, signs = _inputs(4, n, "f32", seed=7 * n)
    sg = torch.from_numpy(signs).cuda()
    y = vq.rht(xt, sg)
    b = oracle.rht_block(n)
    yb = y.double().cpu().numpy().reshape(4, -1, b)
    xb = x64.reshape(4, -1, b)
    assert np.allclose((yb ** 2).sum(axis=2), (xb ** 2).sum(axis=2), rtol=1e-5, atol=0)
    z = y.clone()
    vq.rht(z, sg, transpose=True, out=z)  # in place
    torch.cuda.synchronize()
    assert np.allclose(z.cpu().numpy(), x64, rtol=0, atol=1e-5 * np.abs(x64).max())
