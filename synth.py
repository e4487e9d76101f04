"""Seeded synthetic inputs for the VQ dequantize-and-multiply path.

This module only draws random numbers and rounds them to the storage formats; it holds
none of the method's arithmetic (no packing, no decode, no product).  Both the CPU
oracle and the HIP library are fed from here.

Workloads (shapes from the pages' 8B / 70B-class layers; the pages print no layer
dimensions, so the sizes are the usual LLaMA-3 ones):

  tiny       256 x 256,            v=8, K1=256                 (1 bit/weight), M=1,   x fp16
  dec4k      4096 x 4096,          v=8, K1=65536               (2 bits),       M=1,   x fp16
  dec4k_res  4096 x 4096,          v=8, K1=65536 + K2=256      (3 bits),       M in {1,4,16}, fp16
  mlp8b      up 14336x4096 / down 4096x14336, v=6, K1=K2=4096  (4 bits),       M in {1,4,16}, fp16
  l70b       up 28672x8192 / down 8192x28672, v=8, K1=65536 + K2=256 (3 bits), M in {1,8,32,128,256}, bf16
  aqlm4k     4096 x 4096,          v=8, K1=K2=65536 (two additive books, 4 bits), M in {1,4,16}, x fp16
  v16_4k     4096 x 4096,          v=16, K1=65536 + K2=256     (1.5 bits),     M in {1,4},    x fp16

Distributions: main centroids 0.02*N(0,1) (the weight scale of the VPTQ guide's
verification harness), residual centroids 0.005*N(0,1), both rounded to fp16;
indices uniform on [0, 2^B); per-channel scale U(0.5, 1.5) in fp16; x ~ N(0,1) in
fp16 or bf16 (round-to-nearest-even).  Seeds: numpy PCG64 seeded with
[42, workload, layer, copy, tensor], tensor ids 0 c1, 1 c2, 2 idx1, 3 idx2, 4 scale,
5 x, 6 bias, 7 lattice, 8 dense weights, 9 codebook sample positions.

Encode inputs (make_encode_problem): dense W ~ 0.02*N(0,1) in fp16 (or bf16 / fp32); the
main book holds fp16 copies of W's own v-vectors taken at distinct random positions, the
way the VPTQ guide seeds its codebook for simulation (rows past the number of vectors are
0.02*N(0,1)); the residual book is 0.005*N(0,1) in fp16 (the guide samples residuals,
which would need the encoder's output here).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 42
T_C1, T_C2, T_IDX1, T_IDX2, T_SCALE, T_X, T_BIAS, T_LATTICE, T_W, T_PICK = range(10)


@dataclass(frozen=True)
class Workload:
    key: str
    wid: int
    layers: tuple  # ((N, IN), ...)
    v: int
    bits1: int
    bits2: int
    ms: tuple
    x_dtype: str  # "f16" | "bf16"
    sigma1: float = 0.02
    sigma2: float = 0.005
    labels: tuple = field(default=("layer",))


WORKLOADS = {
    "tiny": Workload("tiny", 0, ((256, 256),), 8, 8, 0, (1,), "f16"),
    "dec4k": Workload("dec4k", 1, ((4096, 4096),), 8, 16, 0, (1,), "f16"),
    "dec4k_res": Workload("dec4k_res", 2, ((4096, 4096),), 8, 16, 8, (1, 4, 16), "f16"),
    "mlp8b": Workload("mlp8b", 3, ((14336, 4096), (4096, 14336)), 6, 12, 12, (1, 4, 16), "f16",
                      labels=("up", "down")),
    "l70b": Workload("l70b", 4, ((28672, 8192), (8192, 28672)), 8, 16, 8, (1, 8, 32, 128, 256), "bf16",
                     labels=("up", "down")),
    # two large additive books (the production-VQ post's AQLM 2 x 2^16, d = 8: 4 bits/weight)
    "aqlm4k": Workload("aqlm4k", 7, ((4096, 4096),), 8, 16, 16, (1, 4, 16), "f16", sigma1=0.014, sigma2=0.014),
    # v = 16 with a 65536-entry main book and a 256-entry residual (the VPTQ guide's
    # 1.0-1.5 bits range: 1.5 bits/weight)
    "v16_4k": Workload("v16_4k", 8, ((4096, 4096),), 16, 16, 8, (1, 4), "f16"),
}


# Affine-lattice layers (UniSVQ summary: d = 4, 2 bits per coordinate): one 8-bit field per
# 4-vector (four 2-bit codes), packed like a v = 4, bits1 = 8 index stream.  Sizes follow the
# decode layers above: a 4096 x 4096 layer and the 70B-class MLP pair.
SVQ_WORKLOADS = {
    "svq4k": Workload("svq4k", 5, ((4096, 4096),), 4, 8, 0, (1, 4, 16), "f16"),
    "svq70b": Workload("svq70b", 6, ((28672, 8192), (8192, 28672)), 4, 8, 0, (1, 8), "bf16",
                       labels=("up", "down")),
}
SVQ_STEP = 0.018  # grid step: codes 0..3 around 1.5 give a weight spread near 0.02


def rng(workload: int, layer: int, copy: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([SEED, workload, layer, copy, tensor])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def num_vectors(in_features: int, v: int) -> int:
    return (in_features + v - 1) // v


def codebook(g: np.random.Generator, k: int, v: int, sigma: float) -> np.ndarray:
    """fp16 bits [k, v]."""
    return f16_bits(g.standard_normal((k, v), dtype=np.float32) * np.float32(sigma))


def indices(g: np.random.Generator, n: int, nv: int, bits: int) -> np.ndarray:
    return g.integers(0, 1 << bits, size=(n, nv), dtype=np.uint32)


def scales(g: np.random.Generator, n: int) -> np.ndarray:
    return f16_bits(g.uniform(0.5, 1.5, size=n).astype(np.float32))


def activations(g: np.random.Generator, m: int, in_features: int, dtype: str) -> np.ndarray:
    """uint16 bits [m, in_features] of fp16 or bf16 N(0,1) samples."""
    a = g.standard_normal((m, in_features), dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else f16_bits(a)


def make_layer(n: int, in_features: int, v: int, bits1: int, bits2: int, *, wid: int = 99, layer: int = 0,
               copy: int = 0, sigma1: float = 0.02, sigma2: float = 0.005, with_scale: bool = True,
               with_bias: bool = False) -> dict:
    """One synthetic quantized layer: indices (uint32 [n, nv]), fp16-bit codebooks, scale, bias."""
    nv = num_vectors(in_features, v)
    out = {
        "n": n, "in_features": in_features, "v": v, "bits1": bits1, "bits2": bits2,
        "cb1": codebook(rng(wid, layer, copy, T_C1), 1 << bits1, v, sigma1),
        "idx1": indices(rng(wid, layer, copy, T_IDX1), n, nv, bits1),
        "cb2": None, "idx2": None, "scale": None, "bias": None,
    }
    if bits2:
        out["cb2"] = codebook(rng(wid, layer, copy, T_C2), 1 << bits2, v, sigma2)
        out["idx2"] = indices(rng(wid, layer, copy, T_IDX2), n, nv, bits2)
    if with_scale:
        out["scale"] = scales(rng(wid, layer, copy, T_SCALE), n)
    if with_bias:
        out["bias"] = f16_bits(rng(wid, layer, copy, T_BIAS).standard_normal(n).astype(np.float32) * 0.1)
    return out


def workload_layer(key: str, layer: int = 0, copy: int = 0) -> dict:
    w = WORKLOADS[key]
    n, in_features = w.layers[layer]
    return make_layer(n, in_features, w.v, w.bits1, w.bits2, wid=w.wid, layer=layer, copy=copy,
                      sigma1=w.sigma1, sigma2=w.sigma2)


def workload_x(key: str, layer: int, m: int) -> np.ndarray:
    w = WORKLOADS[key]
    _, in_features = w.layers[layer]
    return activations(rng(w.wid, layer, 0, T_X), m, in_features, w.x_dtype)


def lattice(g: np.random.Generator, step: float = SVQ_STEP):
    """Affine-grid parameters as fp16 bits: A [4, 4] = step * a Haar-random orthogonal
    matrix (QR of a Gaussian matrix, signs fixed by R's diagonal), and B [4] = -1.5 * (row
    sums of the rounded A), which centres the 256 grid points A q + B (q in {0..3}^4) on 0."""
    z = g.standard_normal((4, 4))
    qm, r = np.linalg.qr(z)
    qm = qm * np.sign(np.diag(r))
    a = f16_bits((qm * step).astype(np.float32))
    b = -1.5 * a.view(np.float16).astype(np.float64).sum(axis=1)
    return a, f16_bits(b.astype(np.float32))


def make_svq_layer(n: int, in_features: int, *, wid: int = 98, layer: int = 0, copy: int = 0,
                   step: float = SVQ_STEP, with_scale: bool = False, with_bias: bool = False) -> dict:
    """One synthetic affine-lattice layer: codes (uint32 [n, ceil(in/4)], values 0..255, four
    2-bit codes each), A / B fp16 bits, optional scale and bias."""
    nv = num_vectors(in_features, 4)
    a, b = lattice(rng(wid, layer, copy, T_LATTICE), step)
    out = {
        "n": n, "in_features": in_features, "v": 4, "bits1": 8, "bits2": 0,
        "codes": indices(rng(wid, layer, copy, T_IDX1), n, nv, 8),
        "a": a, "b": b, "scale": None, "bias": None,
    }
    if with_scale:
        out["scale"] = scales(rng(wid, layer, copy, T_SCALE), n)
    if with_bias:
        out["bias"] = f16_bits(rng(wid, layer, copy, T_BIAS).standard_normal(n).astype(np.float32) * 0.1)
    return out


def svq_workload_layer(key: str, layer: int = 0, copy: int = 0) -> dict:
    w = SVQ_WORKLOADS[key]
    n, in_features = w.layers[layer]
    return make_svq_layer(n, in_features, wid=w.wid, layer=layer, copy=copy)


def svq_workload_x(key: str, layer: int, m: int) -> np.ndarray:
    w = SVQ_WORKLOADS[key]
    _, in_features = w.layers[layer]
    return activations(rng(w.wid, layer, 0, T_X), m, in_features, w.x_dtype)


def make_encode_problem(n: int, in_features: int, v: int, bits1: int, bits2: int, *, wid: int = 96, layer: int = 0,
                        w_dtype: str = "f16", sigma: float = 0.02, sigma2: float = 0.005) -> dict:
    """Inputs of the residual VQ encode.  w: [n, in] fp16 / bf16 bits (uint16) or float32
    values; w_f32: the same weights as float32; cb1 fp16 bits [2^bits1, v]; cb2 fp16 bits
    [2^bits2, v] or None."""
    a = rng(wid, layer, 0, T_W).standard_normal((n, in_features), dtype=np.float32) * np.float32(sigma)
    if w_dtype == "f16":
        w = f16_bits(a)
        w32 = w.view(np.float16).astype(np.float32)
    elif w_dtype == "bf16":
        w = f32_to_bf16_bits(a)
        w32 = (w.astype(np.uint32) << 16).view(np.float32)
    else:
        w = np.ascontiguousarray(a)
        w32 = w
    k1 = 1 << bits1
    vecs = w32.reshape(-1, v) if in_features % v == 0 else np.zeros((0, v), np.float32)
    take = min(k1, vecs.shape[0])
    pos = rng(wid, layer, 0, T_PICK).choice(vecs.shape[0], size=take, replace=False) if take else np.zeros(0, int)
    cb1 = np.empty((k1, v), dtype=np.uint16)
    cb1[:take] = f16_bits(vecs[pos])
    if take < k1:
        cb1[take:] = codebook(rng(wid, layer, 0, T_C1), k1 - take, v, sigma)
    cb2 = codebook(rng(wid, layer, 0, T_C2), 1 << bits2, v, sigma2) if bits2 else None
    return {"n": n, "in_features": in_features, "v": v, "bits1": bits1, "bits2": bits2, "w_dtype": w_dtype,
            "w": w, "w_f32": w32, "cb1": cb1, "cb2": cb2}
