"""Encode problems whose nearest centroid is decided by a gap far below fp64 rounding.

The nearest centroid is q(w) = argmin_k |w - c_k|^2 (VPTQ guide, "The Information-Theoretic
Superiority of Vector Quantization"; its "Step 2" quantizer takes the first index among
equal minima).  Each case built here has two centroids a and b that agree everywhere except
one small coordinate, where they are adjacent fp16 values, and a weight vector w whose other
coordinates are huge.  The exact squared distances of a and b then differ by about 2^-40
(fp32 weights) or 3 * 2^-36 (fp16 weights), while any fp64 evaluation of a distance rounds
at 2^-7 or 2^-22: an implementation that ranks rounded distances is deciding on noise.

`fp64_chain_pick` evaluates the ranking |c|^2 - 2 w.c the way an fp64 implementation would
(fused multiply-add chains in ascending coordinate order, emulated exactly with fractions and
rounded once per operation) so the tests can keep only the cases where that ranking and the
exact one disagree.  `exact_pick` is the definition, in rational arithmetic.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _fma(a: float, b: float, c: float) -> float:
    return float(Fraction(a) * Fraction(b) + Fraction(c))  # one correctly rounded operation


def fp64_chain_pick(w, book) -> int:
    """Lowest index minimising fl64(|c|^2 - 2 w.c) evaluated as fma chains."""
    best, bi = None, 0
    for k, c in enumerate(book):
        nc, dot = 0.0, 0.0
        for wt, ct in zip(w, c):
            nc = _fma(float(ct), float(ct), nc)
            dot = _fma(float(wt), float(ct), dot)
        d = _fma(-2.0, dot, nc)
        if best is None or d < best:
            best, bi = d, k
    return bi


def exact_pick(w, book) -> int:
    """Lowest index minimising the exact |w - c|^2."""
    d = [sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(w, c)) for c in book]
    return d.index(min(d))


def _bf16(x: float) -> np.float32:
    """x rounded to bfloat16 (nearest, ties to even), as a float32."""
    u = np.array([x], np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)[0]


def _next_f16(x: np.float16) -> np.float16:
    return (np.array([x], np.float16).view(np.uint16) + 1).view(np.float16)[0]


def near_tie_case(rng, v: int, w_dtype: str, k: int):
    """One vector w (float32 values representable in w_dtype: "f16", "bf16" or "f32") and a
    fp16 book [k][v]
    holding the pair a, b at two random rows; every other row is far away.  Returns
    (w [v] float32, book [k][v] float16, rows (ia, ib))."""
    assert v >= 3 and k >= 2
    big_c = np.float16(rng.uniform(32768, 65504))
    if w_dtype == "f16":
        w0 = big_c  # (w0 - c0) = 0 for the pair; w0 c0 ~ 2^31
        ca2 = np.float16(rng.uniform(2.0 ** -8, 2.0 ** -7))
        cb2 = _next_f16(ca2)
        # one fp16 step outside the pair: the nearer of the two wins by 3 ulp^2
        lo = (np.array([ca2], np.float16).view(np.uint16) - 1).view(np.float16)[0]
        w2 = lo if rng.integers(2) else _next_f16(cb2)
        w = np.zeros(v, np.float32)
        w[0], w[2] = np.float32(w0), np.float32(w2)
    elif w_dtype == "bf16":
        w0 = _bf16(rng.uniform(2.0 ** 29, 2.0 ** 30))  # w0 c0 ~ 2^45
        ca2 = np.float16(rng.uniform(2.0 ** -4, 2.0 ** -3))
        cb2 = _next_f16(ca2)
        # a bf16 value near the pair (bf16 steps there are 2^-11, the pair 2^-14 apart)
        w2 = _bf16(rng.uniform(float(ca2) - 2.0 ** -12, float(cb2) + 2.0 ** -12))
        w = np.zeros(v, np.float32)
        w[0], w[2] = w0, w2
    else:
        w0 = np.float32(rng.uniform(2.0 ** 29, 2.0 ** 30))  # w0 c0 ~ 2^45
        ca2 = np.float16(rng.uniform(2.0 ** -4, 2.0 ** -3))
        cb2 = _next_f16(ca2)
        mid = (np.float64(ca2) + np.float64(cb2)) / 2  # exact in fp32
        w2 = np.float32(mid + (2.0 ** -27 if rng.integers(2) else -(2.0 ** -27)))
        w = np.zeros(v, np.float32)
        w[0], w[2] = w0, w2
    for t in range(3, v):
        w[t] = np.float32(np.float16(rng.standard_normal() * 0.02))
    w[1] = np.float32(np.float16(rng.standard_normal() * 0.02))
    pair = np.zeros((2, v), np.float16)
    pair[:, 0] = big_c
    pair[:, 1] = np.float16(rng.standard_normal() * 0.02)
    pair[0, 2], pair[1, 2] = ca2, cb2
    for t in range(3, v):
        pair[:, t] = np.float16(rng.standard_normal() * 0.02)
    book = (rng.standard_normal((k, v)) * 0.02).astype(np.float16)
    book[:, 0] = np.float16(0.0)  # far: (w0 - 0)^2 dwarfs every other term
    ia, ib = rng.choice(k, size=2, replace=False)
    book[ia], book[ib] = pair[0], pair[1]
    return w, book, (int(ia), int(ib))


def disagreeing_cases(seed: int, count: int, v: int, w_dtype: str, k: int):
    """`count` cases (deterministic for a seed) where the fp64 chain and the exact minimum
    pick different rows; each is (w, book, exact row)."""
    rng = np.random.default_rng(seed)
    out = []
    tries = 0
    while len(out) < count:
        tries += 1
        assert tries < 200 * count, "no disagreeing cases found"
        w, book, (ia, ib) = near_tie_case(rng, v, w_dtype, k)
        pair = book[[ia, ib]].astype(np.float64)
        ex = exact_pick(w.astype(np.float64), pair)
        ch = fp64_chain_pick(w.astype(np.float64), pair)
        if ex != ch:
            out.append((w, book, (ia, ib)[ex]))
    return out
