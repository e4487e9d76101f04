"""vq_gemv_noalloc (the allocation-free vq_gemv_ws for callers that cannot allocate) through
the C ABI: on two calls in a row, the second with a smaller workspace need, its output
equals vq_gemv_ws's on the same inputs bit for bit (same kernels, fixed summation order)
and meets the oracle tolerance on sampled rows; a shape without the sliced path matches
vq_gemv; an oversized shape is refused and launches nothing.
"""
import numpy as np
import pytest

import synth
from vqtest import DeviceLayer, check_y, oracle_y, sample_rows, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


CALLS = [
    # N, IN, bits2, M, x dtype, bias: the first needs the larger workspace
    (8192, 4096, 8, 8, "bf16", True),
    (4096, 8192, 0, 1, "f16", False),
]


def test_noalloc_matches_gemv_ws_on_two_calls(vq):
    needs = []
    for n, i, b2, m, xd, bias in CALLS:
        print("noalloc", n, i, b2, m, xd, flush=True)
        lay = synth.make_layer(n, i, 8, 16, b2, wid=97, copy=n + m, with_bias=bias)
        dl = DeviceLayer(vq, lay)
        xb = synth.activations(np.random.default_rng(n + m), m, i, xd)
        x = x_tensor(xb, xd)
        tdt = torch.bfloat16 if xd == "bf16" else torch.float16
        needs.append(vq.gemv_workspace_bytes(dl.desc, m, tdt))
        ws = vq.workspace(dl.desc, m, tdt)
        assert ws is not None
        y_ws = vq.gemv_ws(*dl.args(), x, ws, y_dtype=torch.float32)
        out = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        y_na = vq.gemv_noalloc(*dl.args(), x, out=out)
        torch.cuda.synchronize()
        assert y_na.data_ptr() == out.data_ptr()
        assert torch.equal(y_na, y_ws)
        rows = sample_rows(n, 64, seed=n)
        check_y(y_na[:, torch.from_numpy(rows).cuda()], oracle_y(lay, xb, xd, rows), "f32")
        # narrow output too
        y16 = vq.gemv_noalloc(*dl.args(), x)
        assert torch.equal(y16, vq.gemv_ws(*dl.args(), x, ws))
    assert needs[1] < needs[0]


def test_noalloc_without_sliced_path_and_oversize(vq):
    lay = synth.make_layer(512, 1024, 8, 16, 8, wid=96, with_bias=True)  # 2^16 vectors: vq_gemv kernels
    dl = DeviceLayer(vq, lay)
    xb = synth.activations(np.random.default_rng(3), 2, 1024, "bf16")
    x = x_tensor(xb, "bf16")
    y = vq.gemv_noalloc(*dl.args(), x, y_dtype=torch.float32)
    assert torch.equal(y, vq.gemv(*dl.args(), x, y_dtype=torch.float32))
    check_y(y, oracle_y(lay, xb, "bf16"), "f32")
    # 2^16 rows x 64 vectors at M = 16: 32 MiB of partial sums, refused before any launch
    big = vq.make_desc(1 << 16, 512, 8, 16, 0)
    packed = torch.zeros(vq.packed_bytes(big), dtype=torch.uint8, device="cuda")
    cb1 = torch.zeros((65536, 8), dtype=torch.float16, device="cuda")
    xs = torch.zeros((16, 512), dtype=torch.float16, device="cuda")
    out = torch.full((16, 1 << 16), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(vq.VQError) as e:
        vq.gemv_noalloc(big, packed, cb1, None, None, None, xs, out=out)
    assert e.value.status == vq.VQ_ERR_BUFFER_SIZE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
