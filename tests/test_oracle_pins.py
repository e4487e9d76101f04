"""Pins for the CPU oracle: each test ties it to something other than itself.

- number formats: every fp16 / bf16 bit pattern against numpy / torch decoders, and
  round-to-nearest-even against numpy / torch converters;
- the index layout: the pages' bit-rate examples, hand-derived vectors, and numpy's own
  little-endian ``packbits``;
- dequant: codebooks that turn the decode into a known matrix (bit, fp16-identity and
  one-hot books), brute force over every index matrix of a tiny layer, and exact
  invariants (codebook permutation, commutation of the two books, zero residual);
- product: an independent numpy matmul, linearity, row-subset and thread-count
  independence.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import neartie
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ number formats


def test_f16_decode_every_pattern(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_every_pattern(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle_mod.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _rounding_probe_values(seed):
    g = np.random.default_rng(seed)
    # wide exponent sweep, subnormal and overflow regions, and exact midpoints
    a = (g.standard_normal(4000) * np.exp2(g.integers(-30, 20, 4000))).astype(np.float32)
    h = g.integers(0, 0x7BFF, 2000, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    ulp = np.spacing(h.astype(np.float16)).astype(np.float32)
    mids = (h + ulp / np.float32(2)).astype(np.float32)  # exact ties for fp16
    edges = np.array([65504, 65519.996, 65520, 65535, 70000, 6.1035156e-05, 5.9604645e-08, 2.9802322e-08,
                      2.9802326e-08, 0.0, -0.0, 1e-30, -3.0e38], dtype=np.float32)
    vals = np.concatenate([a, mids, -mids, edges]).astype(np.float32)
    return vals[np.isfinite(vals)]


def test_f16_round_nearest_even_matches_numpy(oracle_mod):
    vals = _rounding_probe_values(1)
    ours = oracle_mod.f64_to_f16_rne(vals.astype(np.float64))
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_round_nearest_even_matches_torch(oracle_mod):
    g = np.random.default_rng(2)
    a = (g.standard_normal(4000) * np.exp2(g.integers(-140, 120, 4000))).astype(np.float32)
    b = g.integers(0, 0x7F7F, 2000, dtype=np.uint32).astype(np.uint16)
    base = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)  # exactly half-way to the next bf16
    edges = np.array([3.3895314e38, 3.3961776e38, 3.4028235e38, 1.1754944e-38, 1e-45, 0.0, -0.0], dtype=np.float32)
    vals = np.concatenate([a, ties, -ties, edges])
    vals = vals[np.isfinite(vals)]
    ours = oracle_mod.f64_to_bf16_rne(vals.astype(np.float64))
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ layout and sizes


def test_bitrate_examples_from_pages(oracle_mod):
    gold = _golden("bitrate_examples.json")
    for ex in gold["examples"]:
        v, b1, b2 = ex["v"], ex["bits1"], ex["bits2"]
        # a layer whose rows hold a whole number of 128-bit units: packed size is exact
        n, in_features = 64, v * 128
        nbytes = oracle_mod.packed_bytes(n, in_features, v, b1, b2)
        assert nbytes * 8 / (n * in_features) == pytest.approx(ex["bits_index"], abs=0), ex["name"]
        if "overhead_below" in ex:
            n2, in2 = ex["overhead_layer"]
            books = (1 << b1) * v * 16 + ((1 << b2) * v * 16 if b2 else 0)
            overhead = books / (n2 * in2)
            assert overhead < ex["overhead_below"]
            beff = oracle_mod.packed_bytes(n2, in2, v, b1, b2) * 8 / (n2 * in2) + overhead
            assert beff == pytest.approx(ex["bits_index"] + overhead, abs=1e-12)
    for cb in gold["codebook_bytes"]:
        assert cb["k"] * cb["v"] * 2 * cb["books"] == cb["bytes"], cb["name"]


def test_harness_closed_forms(oracle_mod):
    h = _golden("bitrate_examples.json")["harness_closed_forms"]
    n, i, v = h["n"], h["in_features"], h["v"]
    packed = oracle_mod.packed_bytes(n, i, v, h["bits1"], h["bits2"])
    books = 2 * (1 << 8) * v * 2
    assert n * i * 2 == h["fp16_bytes"]
    assert packed + books == h["quant_bytes"]
    assert round(h["fp16_bytes"] / h["quant_bytes"], 3) == h["compression"]
    assert round(h["quant_bytes"] * 8 / (n * i), 4) == h["bits_per_param"]


@pytest.mark.parametrize("key,expected", [
    ("tiny", [8192]), ("dec4k", [4194304]), ("dec4k_res", [6291456]),
    ("mlp8b", [29818880, 29491200]), ("l70b", [88080384, 88080384]),
])
def test_workload_packed_sizes(oracle_mod, key, expected):
    w = synth.WORKLOADS[key]
    got = [oracle_mod.packed_bytes(n, i, w.v, w.bits1, w.bits2) for (n, i) in w.layers]
    assert got == expected
    for (n, i), nb in zip(w.layers, got):
        bits = nb * 8 / (n * i)
        target = (w.bits1 + w.bits2) / w.v
        assert target <= bits < target * 1.02  # exact when rows fill whole 128-bit units, else padding only


def test_pack_hand_vectors(oracle_mod):
    for vec in _golden("pack_vectors.json")["vectors"]:
        b, fields = vec["bits"], vec["fields"]
        nv = len(fields)
        packed = oracle_mod.pack(1, nv, 1, b, 0, np.array([fields], dtype=np.uint32))
        want = bytes.fromhex(vec["bytes_hex"])
        assert len(packed) % 16 == 0
        assert bytes(packed[: len(want)]) == want, vec
        assert not packed[len(want):].any()
        back, _, pad_ok = oracle_mod.unpack(1, nv, 1, b, 0, packed)
        assert pad_ok and list(back[0]) == fields


def _packbits_reference(idx, bits, row_bytes):
    """Independent construction with numpy: expand every field to its bits, LSB first, then packbits."""
    n, nv = idx.shape
    shifts = np.arange(bits, dtype=np.uint32)
    bitmat = ((idx[:, :, None] >> shifts) & 1).astype(np.uint8).reshape(n, nv * bits)
    pad = row_bytes * 8 - nv * bits
    bitmat = np.concatenate([bitmat, np.zeros((n, pad), dtype=np.uint8)], axis=1)
    return np.packbits(bitmat, axis=1, bitorder="little").reshape(-1)


@pytest.mark.parametrize("n,in_features,v,b1,b2", [
    (3, 40, 8, 16, 8), (5, 37, 6, 12, 12), (2, 100, 3, 5, 0), (4, 64, 8, 8, 0), (1, 7, 1, 13, 3),
    (7, 200, 16, 16, 16), (2, 13, 4, 1, 2), (3, 96, 6, 12, 0),
])
def test_pack_matches_numpy_packbits(oracle_mod, n, in_features, v, b1, b2):
    g = np.random.default_rng(n * 1000 + in_features)
    nv = oracle_mod.num_vectors(in_features, v)
    i1 = g.integers(0, 1 << b1, (n, nv), dtype=np.uint32)
    i2 = g.integers(0, 1 << b2, (n, nv), dtype=np.uint32) if b2 else None
    packed = oracle_mod.pack(n, in_features, v, b1, b2, i1, i2)
    s1 = oracle_mod.row_stride(in_features, v, b1)
    ref = _packbits_reference(i1, b1, s1)
    if b2:
        ref = np.concatenate([ref, _packbits_reference(i2, b2, oracle_mod.row_stride(in_features, v, b2))])
    assert np.array_equal(packed, ref)
    a1, a2, pad_ok = oracle_mod.unpack(n, in_features, v, b1, b2, packed)
    assert pad_ok and np.array_equal(a1, i1)
    if b2:
        assert np.array_equal(a2, i2)


def test_pack_rejects_out_of_range_and_small_buffer(oracle_mod):
    lib = oracle_mod._load()
    idx = np.array([[0, 8]], dtype=np.uint32)
    out = np.zeros(64, dtype=np.uint8)
    rc = lib.oracle_pack(1, 2, 1, 3, 0, oracle_mod._ptr(idx), None, oracle_mod._ptr(out), 64)
    assert rc == oracle_mod.INDEX_RANGE
    idx = np.array([[0, 7]], dtype=np.uint32)
    rc = lib.oracle_pack(1, 2, 1, 3, 0, oracle_mod._ptr(idx), None, oracle_mod._ptr(out), 15)
    assert rc == oracle_mod.BUFFER_SMALL


def test_unpack_flags_nonzero_pad(oracle_mod):
    packed = oracle_mod.pack(1, 3, 1, 4, 0, np.array([[1, 2, 3]], dtype=np.uint32))
    packed = packed.copy()
    packed[15] |= 0x80
    _, _, pad_ok = oracle_mod.unpack(1, 3, 1, 4, 0, packed)
    assert not pad_ok


# ------------------------------------------------------------------ dequant pins


def test_bit_codebook_reduces_to_plain_matmul(oracle_mod):
    """v = 8, K = 256, C[k][t] = bit t of k: W is an arbitrary 0/1 matrix."""
    n, in_features, v = 24, 256, 8
    g = np.random.default_rng(7)
    wbits = g.integers(0, 2, (n, in_features)).astype(np.uint8)
    idx = np.packbits(wbits.reshape(n, in_features // 8, 8), axis=2, bitorder="little").reshape(n, -1)
    cb = ((np.arange(256)[:, None] >> np.arange(8)[None, :]) & 1).astype(np.float16)
    packed = oracle_mod.pack(n, in_features, v, 8, 0, idx.astype(np.uint32))
    w = oracle_mod.dequant(n, in_features, v, 8, 0, packed, cb)
    assert np.array_equal(w, wbits.astype(np.float32))
    x = synth.activations(g, 3, in_features, "f16")
    y = oracle_mod.forward(n, in_features, v, 8, 0, packed, cb, None, None, None, x, False, 3)
    ref = x.view(np.float16).astype(np.float64) @ wbits.T.astype(np.float64)
    assert np.array_equal(y, ref)  # sums of fp16 values in fp64 are exact here


def test_fp16_identity_codebook_reproduces_any_matrix(oracle_mod):
    """v = 1, K = 65536, C[k] = the fp16 number with bit pattern k."""
    n, in_features = 16, 96
    g = np.random.default_rng(8)
    wbits = g.integers(0, 65536, (n, in_features), dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(wbits.view(np.float16))
    wbits[~finite] = 0x3C00
    cb = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(65536, 1)
    packed = oracle_mod.pack(n, in_features, 1, 16, 0, wbits.astype(np.uint32))
    w = oracle_mod.dequant(n, in_features, 1, 16, 0, packed, cb)
    want = wbits.view(np.float16).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), want.view(np.uint32))  # bit-exact, -0 included
    x = synth.activations(g, 2, in_features, "bf16")
    xf = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    y = oracle_mod.forward(n, in_features, 1, 16, 0, packed, cb, None, None, None, x, True, 2)
    ref = xf @ want.astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_one_hot_codebook_with_scale(oracle_mod):
    """K = v = 8 (B = 3), C[k] = e_k: W[o, 8j + t] = scale[o] if idx[o, j] == t else 0."""
    n, in_features, v = 10, 80, 8
    g = np.random.default_rng(9)
    idx = g.integers(0, 8, (n, in_features // 8), dtype=np.uint32)
    cb = np.eye(8, dtype=np.float16)
    scale = synth.scales(g, n)
    packed = oracle_mod.pack(n, in_features, v, 3, 0, idx)
    w = oracle_mod.dequant(n, in_features, v, 3, 0, packed, cb, None, scale)
    s = scale.view(np.float16).astype(np.float32)
    want = np.zeros((n, in_features), dtype=np.float32)
    for o in range(n):
        for j in range(in_features // 8):
            want[o, 8 * j + idx[o, j]] = s[o]
    assert np.array_equal(w, want)


def test_brute_force_every_index_matrix_tiny_layer(oracle_mod):
    """N = 2, IN = 4, v = 2, B1 = 2, B2 = 1: all 4^4 * 2^4 index matrices."""
    n, in_features, v = 2, 4, 2
    g = np.random.default_rng(10)
    cb1 = synth.codebook(g, 4, 2, 0.5)
    cb2 = synth.codebook(g, 2, 2, 0.1)
    scale = synth.scales(g, n)
    bias = synth.f16_bits(g.standard_normal(n).astype(np.float32))
    x = synth.activations(g, 3, in_features, "f16")
    c1 = cb1.view(np.float16).astype(np.float32)
    c2 = cb2.view(np.float16).astype(np.float32)
    s = scale.view(np.float16).astype(np.float32)
    xf = x.view(np.float16).astype(np.float64)
    bf = bias.view(np.float16).astype(np.float64)
    count = 0
    for a in range(4 ** 4):
        i1 = np.array([(a >> (2 * k)) & 3 for k in range(4)], dtype=np.uint32).reshape(2, 2)
        for b in range(2 ** 4):
            i2 = np.array([(b >> k) & 1 for k in range(4)], dtype=np.uint32).reshape(2, 2)
            packed = oracle_mod.pack(n, in_features, v, 2, 1, i1, i2)
            w = oracle_mod.dequant(n, in_features, v, 2, 1, packed, cb1, cb2, scale)
            dense = (c1[i1.reshape(-1)] + c2[i2.reshape(-1)]).reshape(n, in_features)  # numpy fp32 adds
            want = dense * s[:, None]  # numpy fp32 multiply
            assert np.array_equal(w.view(np.uint32), want.view(np.uint32))
            if a % 17 == 0:
                y = oracle_mod.forward(n, in_features, v, 2, 1, packed, cb1, cb2, scale, bias, x, False, 3)
                ref = xf @ want.astype(np.float64).T + bf[None, :]
                assert np.allclose(y, ref, rtol=1e-14, atol=1e-15)
            count += 1
    assert count == 4096


def _random_layer(oracle_mod, seed, n, in_features, v, b1, b2):
    lay = synth.make_layer(n, in_features, v, b1, b2, wid=50, copy=seed)
    packed = oracle_mod.pack(n, in_features, v, b1, b2, lay["idx1"], lay["idx2"])
    return lay, packed


def test_codebook_permutation_invariance(oracle_mod):
    n, in_features, v, b1, b2 = 12, 70, 6, 5, 4
    lay, packed = _random_layer(oracle_mod, 1, n, in_features, v, b1, b2)
    w = oracle_mod.dequant(n, in_features, v, b1, b2, packed, lay["cb1"], lay["cb2"], lay["scale"])
    g = np.random.default_rng(11)
    p1 = g.permutation(1 << b1)
    p2 = g.permutation(1 << b2)
    cb1p = np.empty_like(lay["cb1"]); cb1p[p1] = lay["cb1"]
    cb2p = np.empty_like(lay["cb2"]); cb2p[p2] = lay["cb2"]
    packed_p = oracle_mod.pack(n, in_features, v, b1, b2, p1[lay["idx1"]].astype(np.uint32),
                               p2[lay["idx2"]].astype(np.uint32))
    wp = oracle_mod.dequant(n, in_features, v, b1, b2, packed_p, cb1p, cb2p, lay["scale"])
    assert np.array_equal(w.view(np.uint32), wp.view(np.uint32))


def test_swapping_books_commutes(oracle_mod):
    n, in_features, v, b = 9, 64, 8, 6
    lay, packed = _random_layer(oracle_mod, 2, n, in_features, v, b, b)
    w = oracle_mod.dequant(n, in_features, v, b, b, packed, lay["cb1"], lay["cb2"], lay["scale"])
    packed_s = oracle_mod.pack(n, in_features, v, b, b, lay["idx2"], lay["idx1"])
    ws = oracle_mod.dequant(n, in_features, v, b, b, packed_s, lay["cb2"], lay["cb1"], lay["scale"])
    assert np.array_equal(w.view(np.uint32), ws.view(np.uint32))


def test_zero_residual_equals_no_residual(oracle_mod):
    n, in_features, v = 8, 48, 8
    lay, packed = _random_layer(oracle_mod, 3, n, in_features, v, 8, 4)
    cb1 = lay["cb1"].copy()
    cb1[:16] = np.uint16(0x8000)  # -0 centroids: the add turns them into +0
    zero_book = np.zeros_like(lay["cb2"])
    w_res = oracle_mod.dequant(n, in_features, v, 8, 4, packed, cb1, zero_book, lay["scale"])
    packed1 = oracle_mod.pack(n, in_features, v, 8, 0, lay["idx1"])
    w_one = oracle_mod.dequant(n, in_features, v, 8, 0, packed1, cb1, None, lay["scale"])
    assert np.array_equal(w_res, w_one)
    neg0 = (w_one == 0) & np.signbit(w_one)
    assert neg0.any()
    assert not np.signbit(w_res[neg0]).any()
    assert np.array_equal(w_res.view(np.uint32)[~neg0], w_one.view(np.uint32)[~neg0])


def test_unit_scale_equals_no_scale(oracle_mod):
    n, in_features, v = 6, 40, 8
    lay, packed = _random_layer(oracle_mod, 4, n, in_features, v, 7, 3)
    ones = np.full(n, 0x3C00, dtype=np.uint16)
    a = oracle_mod.dequant(n, in_features, v, 7, 3, packed, lay["cb1"], lay["cb2"], ones)
    b = oracle_mod.dequant(n, in_features, v, 7, 3, packed, lay["cb1"], lay["cb2"], None)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_tail_lanes_dropped(oracle_mod):
    """IN not a multiple of v: the last vector contributes only its first IN mod v lanes."""
    n, in_features, v = 3, 20, 6  # nv = 4, last vector keeps 2 lanes
    lay, packed = _random_layer(oracle_mod, 5, n, in_features, v, 4, 0)
    w = oracle_mod.dequant(n, in_features, v, 4, 0, packed, lay["cb1"], None, None)
    c = lay["cb1"].view(np.float16).astype(np.float32)
    full = c[lay["idx1"].reshape(-1)].reshape(n, 4 * v)
    assert np.array_equal(w, full[:, :in_features])


# ------------------------------------------------------------------ product pins


def test_forward_matches_numpy_matmul_and_is_linear(oracle_mod):
    n, in_features, v, b1, b2 = 33, 300, 6, 9, 5
    lay, packed = _random_layer(oracle_mod, 6, n, in_features, v, b1, b2)
    w = oracle_mod.dequant(n, in_features, v, b1, b2, packed, lay["cb1"], lay["cb2"], lay["scale"])
    g = np.random.default_rng(12)
    x1 = synth.f16_bits(g.integers(-8, 8, (2, in_features)).astype(np.float32))
    x2 = synth.f16_bits(g.integers(-8, 8, (2, in_features)).astype(np.float32))
    x12 = synth.f16_bits(x1.view(np.float16).astype(np.float32) + x2.view(np.float16).astype(np.float32))
    f = lambda xb: oracle_mod.forward(n, in_features, v, b1, b2, packed, lay["cb1"], lay["cb2"], lay["scale"], None,
                                      xb, False, 2)
    y1, y2, y12 = f(x1), f(x2), f(x12)
    ref = x1.view(np.float16).astype(np.float64) @ w.astype(np.float64).T
    tol = 1e-12 * np.abs(ref).max()
    assert np.allclose(y1, ref, rtol=0, atol=tol)
    assert np.allclose(y12, y1 + y2, rtol=0, atol=tol)


def test_rows_subset_and_thread_count(oracle_mod):
    n, in_features, v, b1, b2 = 40, 128, 8, 10, 6
    lay, packed = _random_layer(oracle_mod, 7, n, in_features, v, b1, b2)
    x = synth.activations(np.random.default_rng(13), 3, in_features, "bf16")
    args = (n, in_features, v, b1, b2, packed, lay["cb1"], lay["cb2"], lay["scale"], None, x, True, 3)
    y_all = oracle_mod.forward(*args, nthreads=1)
    y_mt = oracle_mod.forward(*args, nthreads=8)
    assert np.array_equal(y_all, y_mt)
    rows = np.array([39, 0, 17, 17, 5])
    y_sub = oracle_mod.forward(*args, rows=rows, nthreads=3)
    assert np.array_equal(y_sub, y_all[:, rows])


def test_bias_and_empty_shapes(oracle_mod):
    n, in_features, v = 4, 0, 8
    bias = synth.f16_bits(np.array([1.5, -2.0, 0.25, 0.0], dtype=np.float32))
    y = oracle_mod.forward(n, in_features, v, 8, 0, np.zeros(0, np.uint8), np.zeros((256, 8), np.uint16), None,
                           None, bias, np.zeros((2, 0), np.uint16), False, 2)
    assert np.array_equal(y, np.tile(np.array([1.5, -2.0, 0.25, 0.0]), (2, 1)))
    assert oracle_mod.packed_bytes(0, 4096, 8, 16, 8) == 0
    assert oracle_mod.packed_bytes(16, 0, 8, 16, 8) == 0
    y0 = oracle_mod.forward(0, 64, 8, 8, 0, np.zeros(0, np.uint8), np.zeros((256, 8), np.uint16), None, None, None,
                            np.zeros((1, 64), np.uint16), False, 1)
    assert y0.shape == (1, 0)


def test_array_rounding_matches_scalar_and_numpy(oracle_mod):
    vals = _rounding_probe_values(3)
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle_mod.f32_array_to_f16_rne(vals), vals.astype(np.float16).view(np.uint16))
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle_mod.f32_array_to_bf16_rne(vals), ref)


# ------------------------------------------------------------------ affine lattice (UniSVQ)
#
# The UniSVQ summary ("Mathematical Formulation") decodes a d = 4 vector as A q + B over
# integer grid coordinates q; "Efficiency" fixes d = 4, 2 bits per coordinate and 20 fp
# parameters per matrix.  The readings tested here: the code value itself is the
# integer coordinate, code u of a vector sits in bits [2u, 2u+2) of the vector's 8-bit
# field, and the 8-bit fields are packed like a v = 4, bits1 = 8 index stream.


def _svq_q(g, n, in_features):
    """Random integer coordinates q [n, nv, 4] in 0..3 and their 8-bit fields [n, nv]."""
    nv = (in_features + 3) // 4
    q = g.integers(0, 4, size=(n, nv, 4), dtype=np.uint32)
    fields = q[:, :, 0] | (q[:, :, 1] << 2) | (q[:, :, 2] << 4) | (q[:, :, 3] << 6)
    return q, fields


def _f16(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def _svq_packed(oracle_mod, n, in_features, fields):
    return oracle_mod.pack(n, in_features, 4, 8, 0, fields)


@pytest.mark.parametrize("in_features", [16, 13, 64, 70])
def test_svq_identity_grid_returns_the_codes(oracle_mod, in_features):
    g = np.random.default_rng(101)
    n = 7
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    w = oracle_mod.svq_dequant(n, in_features, packed, _f16(np.eye(4)), _f16(np.zeros(4)))
    want = q.reshape(n, -1)[:, :in_features].astype(np.float32)
    assert np.array_equal(w, want)


def test_svq_scalar_grid_closed_form(oracle_mod):
    g = np.random.default_rng(102)
    n, in_features = 5, 40
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    a, b = 0.25, -0.375  # both exact in fp16
    w = oracle_mod.svq_dequant(n, in_features, packed, _f16(a * np.eye(4)), _f16(np.full(4, b)))
    want = (a * q.reshape(n, -1)[:, :in_features] + b).astype(np.float32)
    assert np.array_equal(w, want)
    # the channel scale multiplies the decoded value once, in fp32
    scale = _f16(g.uniform(0.5, 1.5, size=n))
    ws = oracle_mod.svq_dequant(n, in_features, packed, _f16(a * np.eye(4)), _f16(np.full(4, b)), scale=scale)
    s32 = scale.view(np.float16).astype(np.float32)[:, None]
    assert np.array_equal(ws, want * s32)


def test_svq_matrix_orientation(oracle_mod):
    """A[t][u] feeds code u into coordinate t: a 3-cycle permutation tells A from its
    transpose (the transpose would apply the inverse cycle)."""
    g = np.random.default_rng(103)
    n, in_features = 4, 32
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    perm = [1, 2, 0, 3]  # coordinate t takes code perm[t]
    a = np.zeros((4, 4))
    for t, u in enumerate(perm):
        a[t, u] = 1.0
    w = oracle_mod.svq_dequant(n, in_features, packed, _f16(a), _f16(np.zeros(4)))
    want = q[:, :, perm].reshape(n, -1).astype(np.float32)
    assert np.array_equal(w, want)


def test_svq_exact_value_rounded_once(oracle_mod):
    """Brute force with exact rationals: every coordinate is the exact B[t] + sum A[t][u] q_u
    rounded once to fp32."""
    from fractions import Fraction

    g = np.random.default_rng(104)
    n, in_features = 6, 22
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    a_bits, b_bits = synth.lattice(np.random.default_rng(7))
    af = [Fraction(float(v)) for v in a_bits.view(np.float16).astype(np.float64).ravel()]
    bf = [Fraction(float(v)) for v in b_bits.view(np.float16).astype(np.float64)]
    w = oracle_mod.svq_dequant(n, in_features, packed, a_bits, b_bits)
    for o in range(n):
        for col in range(in_features):
            j, t = divmod(col, 4)
            exact = bf[t] + sum(af[t * 4 + u] * int(q[o, j, u]) for u in range(4))
            assert w[o, col] == np.float32(float(exact)), (o, col)


def test_svq_equals_the_256_entry_codebook(oracle_mod):
    """The grid is a 256-entry codebook of 4-vectors: with dyadic A and B every grid point
    is exact in fp16, and the codebook decode (pinned above) must give the same matrix."""
    g = np.random.default_rng(105)
    n, in_features = 9, 52
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    a = g.choice([-0.5, -0.25, 0.0, 0.25, 0.5], size=(4, 4))
    b = g.choice([-1.0, -0.5, 0.5], size=4)
    book = np.zeros((256, 4))
    for k in range(256):
        qq = np.array([(k >> (2 * u)) & 3 for u in range(4)], dtype=np.float64)
        book[k] = a @ qq + b
    scale = _f16(g.uniform(0.5, 1.5, size=n))
    w_grid = oracle_mod.svq_dequant(n, in_features, packed, _f16(a), _f16(b), scale=scale)
    w_book = oracle_mod.dequant(n, in_features, 4, 8, 0, packed, _f16(book), scale=scale)
    assert np.array_equal(w_grid, w_book)


@pytest.mark.parametrize("x_dtype", ["f16", "bf16"])
def test_svq_forward_matches_preapplied_activations(oracle_mod, x_dtype):
    """UniSVQ summary, "Efficiency": the affine map can be moved onto the activations,
    y = sum_j q_j . (A^T x_j) + B . sum_j x_j.  Evaluated here in fp64 from the exact
    parameters; the oracle rounds each weight to fp32 first, so the two differ by at most
    sum |x| |w| 2^-24 (plus fp64 noise)."""
    g = np.random.default_rng(106)
    n, in_features, M = 11, 45, 3
    q, fields = _svq_q(g, n, in_features)
    packed = _svq_packed(oracle_mod, n, in_features, fields)
    a_bits, b_bits = synth.lattice(np.random.default_rng(8))
    bias = _f16(g.standard_normal(n) * 0.1)
    x_bits = synth.activations(g, M, in_features, x_dtype)
    y = oracle_mod.svq_forward(n, in_features, packed, a_bits, b_bits, None, bias, x_bits, x_dtype == "bf16", M)
    dec = oracle_mod.bf16_to_f64 if x_dtype == "bf16" else oracle_mod.f16_to_f64
    x = dec(x_bits).reshape(M, in_features)
    nv = (in_features + 3) // 4
    xp = np.zeros((M, nv * 4))
    xp[:, :in_features] = x
    xg = xp.reshape(M, nv, 4)                      # [M, j, t]
    A = a_bits.view(np.float16).astype(np.float64)
    B = b_bits.view(np.float16).astype(np.float64)
    xhat = np.einsum("mjt,tu->mju", xg, A)         # A^T x_j
    c = xg.sum(axis=1) @ B                         # B . sum_j x_j
    y_pre = np.einsum("oju,mju->mo", q.astype(np.float64), xhat) + c[:, None]
    y_pre += bias.view(np.float16).astype(np.float64)[None, :]
    w_exact = (q.astype(np.float64) @ A.T + B).reshape(n, -1)[:, :in_features]
    bound = np.abs(x) @ np.abs(w_exact).T * 2.0 ** -24 + 1e-12
    assert np.all(np.abs(y - y_pre) <= bound)


def test_svq_sizes_from_the_pages(oracle_mod):
    """UniSVQ summary, "Efficiency": 2 bits per weight for d = 4 and 20 parameters
    (~40 bytes in fp16) per matrix, against ~2048 bytes for a standard d = 4, 2-bit VQ book."""
    gold = {e["name"]: e for e in _golden("bitrate_examples.json")["codebook_bytes"]}
    std = gold["unisvq-standard-vq-d4-2bit"]
    assert std["k"] * std["v"] * 2 == std["bytes"] == 2048
    a_bits, b_bits = synth.lattice(np.random.default_rng(9))
    assert a_bits.nbytes + b_bits.nbytes == 40
    for n, in_features in [(4096, 4096), (28672, 8192), (8192, 28672)]:
        assert oracle_mod.packed_bytes(n, in_features, 4, 8, 0) * 8 == 2 * n * in_features


# ------------------------------------------------------------------ randomized Hadamard transform
#
# QuIP# incoherence processing (production-VQ post; sub-4-bit lecture, "QuIP#: Incoherence
# Processing"; UniSVQ summary, "Preprocessing"): random signs, then a Walsh-Hadamard
# matrix, orthonormal, O(n log n).  Readings: blocks of the largest power of two dividing
# n (at most 16384), s applied before H (forward) or after it (transpose, the inverse).


@pytest.mark.parametrize("n,b", [(4096, 4096), (14336, 2048), (28672, 4096), (8192, 8192), (16384, 16384),
                                 (32768, 16384), (4100, 4), (7, 1), (1, 1), (96, 32)])
def test_rht_block_rule(oracle_mod, n, b):
    assert oracle_mod.rht_block(n) == b


def test_rht_two_point_closed_form(oracle_mod):
    a, c = 3.0, 1.0
    r2 = math.sqrt(2.0)
    no_sign, sign1 = np.array([0], np.uint8), np.array([2], np.uint8)
    assert np.allclose(oracle_mod.rht([[a, c]], no_sign), [[(a + c) / r2, (a - c) / r2]], rtol=0, atol=1e-15)
    assert np.allclose(oracle_mod.rht([[a, c]], sign1), [[(a - c) / r2, (a + c) / r2]], rtol=0, atol=1e-15)
    assert np.allclose(oracle_mod.rht([[a, c]], sign1, transpose=True), [[(a + c) / r2, -(a - c) / r2]], rtol=0,
                       atol=1e-15)


@pytest.mark.parametrize("n", [16, 256, 1024, 96])
def test_rht_matches_sylvester_matrix(oracle_mod, n):
    """Against scipy's Sylvester-construction Hadamard matrix, block by block."""
    import scipy.linalg

    g = np.random.default_rng(n)
    m = 3
    x = g.standard_normal((m, n))
    signs = g.integers(0, 256, size=(n + 7) // 8, dtype=np.uint8)
    s = np.where(np.unpackbits(signs, bitorder="little")[:n] == 1, -1.0, 1.0)
    b = oracle_mod.rht_block(n)
    h = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    want = np.concatenate([(x[:, k:k + b] * s[k:k + b]) @ h.T for k in range(0, n, b)], axis=1)
    assert np.allclose(oracle_mod.rht(x, signs), want, rtol=0, atol=1e-12)
    want_t = np.concatenate([(x[:, k:k + b] @ h.T) * s[k:k + b] for k in range(0, n, b)], axis=1)
    assert np.allclose(oracle_mod.rht(x, signs, transpose=True), want_t, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [64, 1000, 4096])
def test_rht_orthonormal_and_inverse(oracle_mod, n):
    g = np.random.default_rng(n + 1)
    x = g.standard_normal((2, n))
    signs = g.integers(0, 256, size=(n + 7) // 8, dtype=np.uint8)
    y = oracle_mod.rht(x, signs)
    assert np.allclose((y * y).sum(axis=1), (x * x).sum(axis=1), rtol=1e-12, atol=0)  # Parseval
    assert np.allclose(oracle_mod.rht(y, signs, transpose=True), x, rtol=0, atol=1e-12)  # inverse


def test_rht_blocks_are_independent(oracle_mod):
    n = 12  # b = 4: three blocks
    x = np.zeros((1, n))
    x[0, 5] = 1.0  # one-hot in block 1
    y = oracle_mod.rht(x, np.zeros(2, np.uint8))
    assert np.all(y[0, :4] == 0) and np.all(y[0, 8:] == 0)
    assert np.allclose(np.abs(y[0, 4:8]), 0.5, rtol=0, atol=1e-15)  # a column of H_4 / 2


# ------------------------------------------------------------------ residual VQ encode
# VPTQ guide, "Step 2: Multi-Stage Residual Vector Quantizer (RVQ)": nearest main centroid
# by Euclidean distance (argmin keeps the first of equal distances), then the nearest
# residual centroid of w - C1[idx1].


def _f16v(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


def _exact_nearest(vec, book_bits):
    """Lowest index minimising the exact squared distance (rational arithmetic)."""
    from fractions import Fraction

    c = book_bits.view(np.float16).astype(np.float64)
    d = [sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(vec, row)) for row in c]
    best = min(d)
    order = sorted(d)
    gap = order[1] - order[0] if len(order) > 1 else Fraction(1)
    return d.index(best), gap


@pytest.mark.parametrize("seed,v,k1,k2", [(1, 4, 16, 8), (2, 8, 32, 16), (3, 1, 8, 4), (4, 16, 12, 5)])
def test_rvq_matches_exact_rational_distances(oracle_mod, seed, v, k1, k2):
    g = np.random.default_rng(seed)
    n, nv = 3, 3
    w = (g.standard_normal((n, nv * v)) * 0.02).astype(np.float16).astype(np.float32)
    cb1 = _f16v(g.standard_normal((k1, v)) * 0.02)
    cb2 = _f16v(g.standard_normal((k2, v)) * 0.005)
    i1, i2 = oracle_mod.rvq_assign(w, v, cb1, cb2)
    for o in range(n):
        for j in range(nv):
            vec = w[o, j * v:(j + 1) * v]
            e1, gap1 = _exact_nearest(vec, cb1)
            assert gap1 > 1e-12 and i1[o, j] == e1
            r = (vec - cb1[e1].view(np.float16).astype(np.float32)).astype(np.float32)
            e2, gap2 = _exact_nearest(r, cb2)
            assert gap2 > 1e-12 and i2[o, j] == e2


def test_rvq_agrees_with_scipy_cdist(oracle_mod):
    from scipy.spatial.distance import cdist

    p = synth.make_encode_problem(64, 128, 8, 8, 6, wid=90)
    i1, i2 = oracle_mod.rvq_assign(p["w_f32"], 8, p["cb1"], p["cb2"])
    vecs = p["w_f32"].reshape(-1, 8).astype(np.float64)
    c1 = p["cb1"].view(np.float16).astype(np.float64)
    c2 = p["cb2"].view(np.float16).astype(np.float64)
    d1 = cdist(vecs, c1)
    ref1 = np.argmin(d1, axis=1)
    srt = np.sort(d1, axis=1)
    clear = srt[:, 1] - srt[:, 0] > 1e-9
    assert clear.mean() > 0.5  # main book holds copies of some vectors: exact-zero distances
    assert np.array_equal(i1.reshape(-1)[clear], ref1[clear])
    res = (vecs.astype(np.float32) - c1[i1.reshape(-1)].astype(np.float32)).astype(np.float64)
    d2 = cdist(res, c2)
    srt2 = np.sort(d2, axis=1)
    clear2 = srt2[:, 1] - srt2[:, 0] > 1e-9
    assert clear2.all()
    assert np.array_equal(i2.reshape(-1), np.argmin(d2, axis=1))


def test_rvq_codebook_holding_the_vectors(oracle_mod):
    """A main book made of the vectors themselves returns each vector's own row (the
    lowest one among duplicates); the residual is then zero, whose nearest residual
    centroid is the shortest one."""
    g = np.random.default_rng(7)
    v, nvec = 8, 40
    vecs = _f16v(g.standard_normal((nvec, v)) * 0.02)
    perm = g.permutation(nvec)
    book = np.concatenate([vecs[perm], vecs[perm[:5]]])  # rows 40..44 duplicate rows 0..4
    book = np.concatenate([book[40:], book[:40]])        # the duplicates come first now
    cb2 = _f16v(g.standard_normal((16, v)) * 0.005)
    w = vecs.view(np.float16).astype(np.float32).reshape(4, 10 * v)
    i1, i2 = oracle_mod.rvq_assign(w, v, book, cb2)
    pos = {int(p): i for i, p in enumerate(perm)}
    want = np.array([(pos[k] + 5) if pos[k] >= 5 else pos[k] for k in range(nvec)])
    assert np.array_equal(i1.reshape(-1), want)
    norms = (cb2.view(np.float16).astype(np.float64) ** 2).sum(axis=1)
    assert np.all(i2 == int(np.argmin(norms)))


def test_rvq_ties_go_to_the_lowest_index(oracle_mod):
    v = 4
    book = _f16v([[0, 0, 0, 0], [1, 0, 0, 0], [0, -1, 0, 0], [-1, 0, 0, 0], [0.5, 0, 0, 0], [0, 1, 0, 0]])
    w = np.array([[0.5, 0, 0, 0,      # |w - c| = 0.5 for rows 0 and 1, 0 for row 4: row 4
                   0.25, 0, 0, 0,     # rows 0 and 4 at 0.25: row 0
                   0, 0, 0, 0,        # row 0 exact
                   -0.5, 0, 0, 0,     # rows 0 and 3 at 0.5: row 0
                   -0.75, 0.5, 0, 0,  # row 3 (0.25^2 + 0.5^2) vs rows 0, 2: row 3
                   0, 0.5, 0, 0]],    # rows 0 and 5 at 0.5: row 0
                 dtype=np.float32)
    i1, _ = oracle_mod.rvq_assign(w, v, book)
    assert i1.tolist() == [[4, 0, 0, 0, 3, 0]]
    book2 = _f16v([[1, 1, 0, 0], [2, 0, 0, 0], [1, 1, 0, 0], [0, 2, 0, 0]])  # rows 0 and 2 equal
    w2 = np.array([[1, 1, 0, 0, 1.5, 0.5, 0, 0]], dtype=np.float32)     # second: rows 0, 1, 2 tie
    i1, _ = oracle_mod.rvq_assign(w2, v, book2)
    assert i1.tolist() == [[0, 0]]


def test_rvq_residual_stage_recovers_grid_sums(oracle_mod):
    """With the main book on an integer grid and small residual centroids (no u with -u
    also present), w = C1[j] + C2[m] is exact in fp16 and both indices come back; a
    residual taken the wrong way round (C1[j] - w) would pick other rows."""
    g = np.random.default_rng(11)
    v, k1, k2 = 4, 64, 32
    c1 = g.integers(-3, 4, size=(k1, v)).astype(np.float64)
    c1 = np.unique(c1, axis=0)
    k1 = c1.shape[0]
    c2 = (g.integers(1, 16, size=(k2, v)) / 64.0) * np.array([1, -1, 1, -1])  # |u| < 0.25, fixed sign pattern
    c2 = np.unique(c2, axis=0)
    k2 = c2.shape[0]
    j = g.integers(0, k1, size=30)
    m = g.integers(0, k2, size=30)
    w = (c1[j] + c2[m]).reshape(3, 10 * v).astype(np.float32)
    i1, i2 = oracle_mod.rvq_assign(w, v, _f16v(c1), _f16v(c2))
    assert np.array_equal(i1.reshape(-1), j)
    assert np.array_equal(i2.reshape(-1), m)


def test_rvq_scalar_levels_closed_form(oracle_mod):
    """v = 1 with sorted levels: the nearest level is the one whose midpoint cell holds w
    (lower level on a midpoint)."""
    levels = np.array([-1.0, -0.5, -0.125, 0.0, 0.25, 1.0])
    g = np.random.default_rng(3)
    w = np.concatenate([g.uniform(-1.5, 1.5, 200), (levels[1:] + levels[:-1]) / 2]).astype(np.float16)
    w = w.astype(np.float32)[None, :]
    i1, _ = oracle_mod.rvq_assign(w, 1, _f16v(levels))
    mids = (levels[1:] + levels[:-1]) / 2
    want = np.searchsorted(mids, w[0].astype(np.float64), side="left")
    assert np.array_equal(i1[0], want)


@pytest.mark.parametrize("w_dtype,v,k,seed", [("f32", 8, 16, 21), ("f16", 8, 256, 22), ("f32", 4, 8, 23),
                                           ("f16", 16, 64, 24), ("f32", 3, 2, 25), ("bf16", 8, 32, 26)])
def test_rvq_near_ties_decided_exactly(oracle_mod, w_dtype, v, k, seed):
    """Pairs of centroids whose exact squared distances differ by ~2^-40 (fp32 weights) or
    3 * 2^-36 (fp16 weights) beside terms of 2^45 / 2^31: only cases where an fp64 ranking
    of |c|^2 - 2 w.c picks the other row are kept, so a rounded-distance encode fails here."""
    for w, book, want in neartie.disagreeing_cases(seed, 6, v, w_dtype, k):
        assert want == neartie.exact_pick(w.astype(np.float64), book.astype(np.float64))
        i1, _ = oracle_mod.rvq_assign(w[None, :], v, book.view(np.uint16))
        assert int(i1[0, 0]) == want
        # the same decision in the residual stage: main book = the zero vector (row 0, nearest)
        # and far rows, so the fp32 residual is w itself
        c1 = np.zeros((4, v), np.float16)
        c1[1:, 0] = np.float16(-65504.0)
        j1, j2 = oracle_mod.rvq_assign(w[None, :], v, c1.view(np.uint16), book.view(np.uint16))
        assert int(j1[0, 0]) == 0 and int(j2[0, 0]) == want


def test_rvq_non_finite_reading(oracle_mod):
    """Distances under IEEE arithmetic on extended values: NaN when a coordinate is NaN or the
    same infinity sits in w and c; +inf when a coordinate is infinite; finite ones win, NaN
    ones are never taken, all-NaN gives index 0."""
    inf, nan = np.inf, np.nan
    book = _f16v([[inf, 0], [1, 0], [0, nan], [-inf, 0], [0, 0]])
    cases = [
        ([nan, 0], 0),      # every distance NaN
        ([inf, 0], 1),      # row 0: inf - inf = NaN; rows 1, 3, 4: +inf (row 2: NaN): first is 1
        ([-inf, 0], 0),     # row 0: -inf - inf = -inf, squared +inf: row 0 first
        ([0.5, 0], 1),      # finite rows 1 and 4 tie at 0.25: row 1; rows 0, 3 +inf, row 2 NaN
        ([0.25, 0], 4),     # finite: row 4 (0.0625) beats row 1 (0.5625)
    ]
    for w, want in cases:
        i1, _ = oracle_mod.rvq_assign(np.array([w], np.float32), 2, book)
        assert int(i1[0, 0]) == want, (w, int(i1[0, 0]), want)
    only_bad = _f16v([[nan, 0], [inf, 1], [0, -inf]])
    i1, _ = oracle_mod.rvq_assign(np.array([[1.0, 1.0]], np.float32), 2, only_bad)
    assert int(i1[0, 0]) == 1  # no finite distance: the first +inf one


def test_rvq_permuting_the_book_permutes_the_indices(oracle_mod):
    p = synth.make_encode_problem(8, 64, 8, 7, 5, wid=91)
    i1, i2 = oracle_mod.rvq_assign(p["w_f32"], 8, p["cb1"], p["cb2"])
    g = np.random.default_rng(5)
    q1, q2 = g.permutation(128), g.permutation(32)
    j1, j2 = oracle_mod.rvq_assign(p["w_f32"], 8, p["cb1"][q1], p["cb2"][q2])
    assert np.array_equal(q1[j1], i1)
    assert np.array_equal(q2[j2], i2)
    k1, k2 = oracle_mod.rvq_assign(p["w_f32"], 8, p["cb1"])
    assert k2 is None and np.array_equal(k1, i1)
