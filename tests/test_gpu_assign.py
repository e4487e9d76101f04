"""GPU parity of the residual VQ encode (vq_assign) against the CPU oracle through the C
ABI: indices are compared element by element and must be equal (both sides take the exact
minimum of |w - c|^2, ties to the lowest index).

- small shapes spanning several workgroups and a ragged tail of lanes, every v from 1 to
  16 among them, one and two stages, fp16 / bf16 / fp32 weights; with fp16 weights and
  K1 >= 256 the main stage runs on the matrix cores (fp32 distances, fp64 re-ranking
  within the proven error bound), every v from 1 to 16 there too;
- books made of fp16 subnormals (the matrix cores must multiply them exactly) and
  infinite / NaN weights and centroids (every centroid is then re-ranked in fp64);
- exact ties: duplicated centroids and vectors that equal a centroid;
- near ties far below fp64 rounding (an fp64 ranking gets them wrong), both stages, every
  weight type, the matrix-core stage among them, and the non-finite reading on hand cases;
- the 4096 x 4096 layer with a 65536-entry main book and a 256-entry residual book (the
  weights of the benchmark) on sampled rows at full size, plus the index range at any
  size;
- encode -> pack -> product through the library equals the oracle's product on the
  oracle's own indices;
- workspace reuse across calls and determinism.
"""
import functools

import numpy as np
import pytest

import neartie
import oracle
import synth
from vqtest import check_y, f16_tensor, x_tensor

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gemv_bit_unpack_amd as g

    g.lib()
    return g


def _w_tensor(p, device="cuda"):
    if p["w_dtype"] == "f32":
        return torch.from_numpy(np.ascontiguousarray(p["w"])).to(device)
    return x_tensor(p["w"], p["w_dtype"], device)


def _gpu_assign(vq, p):
    d = vq.make_desc(p["n"], p["in_features"], p["v"], p["bits1"], p["bits2"])
    i1, i2 = vq.assign(d, _w_tensor(p), f16_tensor(p["cb1"]), f16_tensor(p["cb2"]))
    torch.cuda.synchronize()
    u = lambda t: None if t is None else t.cpu().numpy().view(np.uint32)
    return u(i1), u(i2)


def _oracle_assign(p, rows=None):
    w = p["w_f32"] if rows is None else p["w_f32"][rows]
    return oracle.rvq_assign(w, p["v"], p["cb1"], p["cb2"])


SHAPES = [
    # n, in_features, v, bits1, bits2, w dtype
    (1, 8, 8, 1, 0, "f16"),
    (5, 64, 8, 8, 4, "f16"),
    (3, 48, 4, 5, 0, "f16"),
    (17, 96, 16, 10, 6, "bf16"),
    (33, 120, 6, 12, 12, "f16"),
    (2, 21, 3, 4, 2, "f32"),
    (1, 1, 1, 1, 1, "f16"),
    (600, 14, 2, 6, 3, "f16"),      # 4200 vectors: several workgroups, ragged tail
    (513, 10, 5, 7, 0, "bf16"),
    (257, 28, 7, 9, 5, "f32"),
    (130, 36, 9, 6, 6, "f16"),
    (71, 30, 10, 8, 2, "f16"),
    (40, 44, 11, 5, 5, "bf16"),
    (66, 48, 12, 7, 3, "f16"),
    (30, 39, 13, 6, 1, "f32"),
    (29, 42, 14, 4, 4, "f16"),
    (31, 45, 15, 8, 8, "f16"),
    (64, 256, 8, 16, 8, "f16"),     # the benchmark's book sizes
]


@pytest.mark.parametrize("n,in_features,v,bits1,bits2,wd", SHAPES)
def test_assign_parity_shapes(vq, n, in_features, v, bits1, bits2, wd):
    p = synth.make_encode_problem(n, in_features, v, bits1, bits2, wid=95, w_dtype=wd)
    g1, g2 = _gpu_assign(vq, p)
    o1, o2 = _oracle_assign(p)
    assert np.array_equal(g1, o1)
    if bits2:
        assert np.array_equal(g2, o2)
    else:
        assert g2 is None and o2 is None


MFMA_SHAPES = [
    # fp16 weights, K1 >= 256: n, in_features, v, bits1, bits2
    (100, 50, 1, 8, 0),
    (40, 60, 2, 9, 3),
    (33, 63, 3, 9, 0),
    (300, 80, 4, 10, 2),      # 6000 vectors: several workgroups of 1024, ragged tail
    (70, 45, 5, 8, 8),
    (61, 66, 6, 11, 0),
    (50, 49, 7, 12, 4),
    (300, 80, 8, 9, 0),       # 3000 vectors
    (20, 72, 9, 8, 5),
    (21, 70, 10, 10, 0),
    (22, 66, 11, 9, 2),
    (23, 72, 12, 8, 8),
    (24, 65, 13, 9, 0),
    (25, 70, 14, 11, 3),
    (26, 75, 15, 8, 0),
    (27, 80, 16, 10, 6),
    (1, 8, 8, 14, 0),         # one vector, K1 = 16384
    (1030, 8, 8, 8, 0),       # 1030 vectors: one workgroup plus a 6-vector tail
]


@pytest.mark.parametrize("n,in_features,v,bits1,bits2", MFMA_SHAPES)
def test_assign_matrix_core_shapes(vq, n, in_features, v, bits1, bits2):
    p = synth.make_encode_problem(n, in_features, v, bits1, bits2, wid=89)
    g1, g2 = _gpu_assign(vq, p)
    o1, o2 = _oracle_assign(p)
    assert np.array_equal(g1, o1)
    if bits2:
        assert np.array_equal(g2, o2)


@pytest.mark.parametrize("v", [4, 8, 12])
def test_assign_subnormal_book(vq, v):
    """Centroids and weights among the fp16 subnormals (|x| < 2^-14): a matrix core that
    flushed them would rank by |c|^2 alone and miss the nearest centroids."""
    g = np.random.default_rng(v)
    k1 = 512
    cb1 = g.integers(-1023, 1024, size=(k1, v)).astype(np.uint16)
    cb1 = np.where(cb1.view(np.int16) < 0, 0x8000 | (-cb1.view(np.int16)).astype(np.uint16), cb1).astype(np.uint16)
    w16 = cb1[g.integers(0, k1, size=200 * 4)] ^ (g.integers(0, 4, size=(800, v)).astype(np.uint16))
    p = {"n": 200, "in_features": 4 * v, "v": v, "bits1": 9, "bits2": 0, "w_dtype": "f16",
         "w": w16.reshape(200, 4 * v), "w_f32": w16.reshape(200, 4 * v).view(np.float16).astype(np.float32),
         "cb1": cb1, "cb2": None}
    assert np.all(np.abs(p["w_f32"]) < 2.0 ** -14)
    g1, _ = _gpu_assign(vq, p)
    o1, _ = _oracle_assign(p)
    assert np.array_equal(g1, o1)
    assert len(np.unique(o1)) > 100


@pytest.mark.parametrize("wd", ["f16", "f32"])
def test_assign_non_finite_values(vq, wd):
    """Infinite and NaN weights, an infinite centroid: both sides rank the same fp64 values."""
    p = synth.make_encode_problem(64, 64, 8, 9, 4, wid=88, w_dtype=wd)
    specials = np.array([np.inf, -np.inf, np.nan], dtype=np.float32)
    g = np.random.default_rng(2)
    pos = g.choice(p["w_f32"].size, size=12, replace=False)
    wf = p["w_f32"].copy().reshape(-1)
    wf[pos] = specials[np.arange(12) % 3]
    p["w_f32"] = wf.reshape(p["w_f32"].shape)
    p["w"] = p["w_f32"].astype(np.float16).view(np.uint16) if wd == "f16" else p["w_f32"]
    p["cb1"][17, 3] = np.float16(np.inf).view(np.uint16)
    g1, g2 = _gpu_assign(vq, p)
    o1, o2 = _oracle_assign(p)
    assert np.array_equal(g1, o1) and np.array_equal(g2, o2)


def test_assign_exact_ties_take_the_lowest_index(vq):
    """Duplicated centroids (later copies of earlier rows) and vectors equal to centroids."""
    p = synth.make_encode_problem(300, 64, 8, 9, 5, wid=94)
    g = np.random.default_rng(4)
    k1 = p["cb1"].shape[0]
    dst = g.choice(np.arange(1, k1), size=120, replace=False)
    for k in dst:
        p["cb1"][k] = p["cb1"][g.integers(0, k)]
    p["cb2"][7] = p["cb2"][3]
    p["cb2"][20] = 0
    p["cb2"][21] = 0
    g1, g2 = _gpu_assign(vq, p)
    o1, o2 = _oracle_assign(p)
    assert np.array_equal(g1, o1) and np.array_equal(g2, o2)
    # the book holds copies of W's vectors: those vectors land on the first copy
    vecs = p["w_f32"].reshape(-1, 8).astype(np.float16).view(np.uint16)
    book = {}
    for k in range(k1 - 1, -1, -1):
        book[p["cb1"][k].tobytes()] = k
    hits = [(i, book[vecs[i].tobytes()]) for i in range(vecs.shape[0]) if vecs[i].tobytes() in book]
    assert len(hits) > 100
    flat = g1.reshape(-1)
    assert all(flat[i] == k for i, k in hits)


NEAR_TIE_CASES = [
    # weights, v, book rows (2^bits), seed: fp16 with 256+ rows takes the matrix-core stage
    ("f16", 8, 256, 31), ("f16", 16, 512, 32), ("f16", 4, 16, 33), ("bf16", 8, 32, 34), ("f32", 8, 16, 35),
    ("f32", 5, 64, 36),
]


@pytest.mark.parametrize("wd,v,k,seed", NEAR_TIE_CASES)
def test_assign_near_ties_decided_exactly(vq, wd, v, k, seed):
    """Centroid pairs whose exact distances differ by ~2^-25 .. 2^-40 beside 2^31 .. 2^45
    terms, kept only where an fp64 ranking picks the other row; main and residual stages."""
    bits = int(np.log2(k))
    for w, book, want in neartie.disagreeing_cases(seed, 6, v, wd, k):
        wbits = w[None, :].astype(np.float16).view(np.uint16) if wd == "f16" else (
            synth.f32_to_bf16_bits(w[None, :]) if wd == "bf16" else w[None, :])
        wt = _w_tensor({"w": wbits, "w_dtype": wd})
        d = vq.make_desc(1, v, v, bits, 0)
        i1, _ = vq.assign(d, wt, f16_tensor(book.view(np.uint16)), None)
        torch.cuda.synchronize()
        o1, _ = oracle.rvq_assign(w[None, :], v, book.view(np.uint16))
        assert int(o1[0, 0]) == want
        assert int(i1.cpu().numpy().view(np.uint32)[0, 0]) == want
        # residual stage: main book = the zero vector (row 0, nearest) and far rows
        c1 = np.zeros((4, v), np.float16)
        c1[1:, 0] = np.float16(-65504.0)
        d2 = vq.make_desc(1, v, v, 2, bits)
        j1, j2 = vq.assign(d2, wt, f16_tensor(c1.view(np.uint16)), f16_tensor(book.view(np.uint16)))
        torch.cuda.synchronize()
        assert int(j1.cpu().numpy().view(np.uint32)[0, 0]) == 0
        assert int(j2.cpu().numpy().view(np.uint32)[0, 0]) == want


@pytest.mark.parametrize("wd,rows", [("f32", 8), ("f16", 256)])
def test_assign_non_finite_reading(vq, wd, rows):
    """The IEEE reading on hand cases (NaN distances never taken, finite before +inf, all
    NaN gives 0); rows past the first five are NaN centroids.  With 256 rows and fp16
    weights the book is non-finite, so every vector takes the general exact path."""
    inf, nan = np.inf, np.nan
    book = np.full((rows, 2), np.nan, np.float16)
    book[:5] = [[inf, 0], [1, 0], [0, nan], [-inf, 0], [0, 0]]
    ws = np.array([[nan, 0], [inf, 0], [-inf, 0], [0.5, 0], [0.25, 0]], np.float32)
    want = [0, 1, 0, 1, 4]
    wbits = ws.astype(np.float16).view(np.uint16) if wd == "f16" else ws
    d = vq.make_desc(5, 2, 2, int(np.log2(rows)), 0)
    i1, _ = vq.assign(d, _w_tensor({"w": wbits, "w_dtype": wd}), f16_tensor(book.view(np.uint16)), None)
    torch.cuda.synchronize()
    got = i1.cpu().numpy().view(np.uint32).reshape(-1).tolist()
    o1, _ = oracle.rvq_assign(ws, 2, book.view(np.uint16))
    assert o1.reshape(-1).tolist() == want
    assert got == want


@functools.lru_cache(maxsize=1)
def _bench_problem():
    return synth.make_encode_problem(4096, 4096, 8, 16, 8, wid=93)


def test_assign_full_size_sampled_rows(vq):
    p = _bench_problem()
    g1, g2 = _gpu_assign(vq, p)
    assert g1.shape == (4096, 512) and g2.shape == (4096, 512)
    assert int(g1.max()) < 65536 and int(g2.max()) < 256
    rows = np.array([0, 1, 1000, 2047, 3001, 4095])
    o1, o2 = _oracle_assign(p, rows)
    assert np.array_equal(g1[rows], o1)
    assert np.array_equal(g2[rows], o2)
    # every main centroid is a copy of some vector of W, so many vectors are exact hits
    assert len(np.unique(g1)) > 30000


def test_assign_then_pack_and_product(vq):
    """Encode, pack with the library's packer, multiply with the library: equal to the
    oracle's product on the oracle's own encode."""
    p = synth.make_encode_problem(96, 512, 8, 10, 6, wid=92)
    g1, g2 = _gpu_assign(vq, p)
    o1, o2 = _oracle_assign(p)
    assert np.array_equal(g1, o1) and np.array_equal(g2, o2)
    d = vq.make_desc(96, 512, 8, 10, 6)
    packed = torch.from_numpy(vq.pack(d, g1, g2)).cuda()
    x_bits = synth.activations(np.random.default_rng(9), 2, 512, "f16")
    y = vq.gemv(d, packed, f16_tensor(p["cb1"]), f16_tensor(p["cb2"]), None, None, x_tensor(x_bits, "f16"),
                y_dtype=torch.float32)
    torch.cuda.synchronize()
    opk = oracle.pack(96, 512, 8, 10, 6, o1, o2)
    y64 = oracle.forward(96, 512, 8, 10, 6, opk, p["cb1"], p["cb2"], None, None, x_bits, False, 2)
    check_y(y, y64, "f32")


def test_assign_workspace_reuse_and_determinism(vq):
    big = synth.make_encode_problem(200, 128, 8, 12, 8, wid=91)
    small = synth.make_encode_problem(50, 64, 8, 6, 4, wid=90)
    db = vq.make_desc(200, 128, 8, 12, 8)
    ws = torch.empty(vq.assign_workspace_bytes(db), dtype=torch.uint8, device="cuda")
    a1, a2 = vq.assign(db, _w_tensor(big), f16_tensor(big["cb1"]), f16_tensor(big["cb2"]), ws=ws)
    ds = vq.make_desc(50, 64, 8, 6, 4)
    b1, b2 = vq.assign(ds, _w_tensor(small), f16_tensor(small["cb1"]), f16_tensor(small["cb2"]), ws=ws)
    c1, c2 = vq.assign(db, _w_tensor(big), f16_tensor(big["cb1"]), f16_tensor(big["cb2"]), ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a1, c1) and torch.equal(a2, c2)
    o1, o2 = _oracle_assign(small)
    assert np.array_equal(b1.cpu().numpy().view(np.uint32), o1)
    assert np.array_equal(b2.cpu().numpy().view(np.uint32), o2)
