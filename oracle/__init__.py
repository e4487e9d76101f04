"""CPU oracle for the VQ dequantize-and-multiply path.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code with
the HIP library in ``gemv_bit_unpack_amd``: the arithmetic lives in the plain C file
``vq_oracle.c`` (built here with gcc, ``-O2 -fno-fast-math -ffp-contract=off``), and
this module only marshals numpy arrays into it.

What it computes follows the VPTQ guide (aifetchly): the residual-decode formula of
"2. Multi-Stage Residual Vector Quantization (RVQ)", the ``dequantize`` of "Step 2" and
the forward of "Step 3: Fused Low-Bit VPTQ Linear Layer"; the per-output-channel scale
follows the QuIP# "per-channel scaling" of the production-VQ post (llms.blog).  The
bit layout of the packed indices is a reading (the pages are silent on it): per row,
LSB-first fields of B bits, rows padded to 16 bytes, main stream then residual stream.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off", "-fPIC"]

_lock = threading.Lock()
_lib = None

OK = 0
BAD_ARGS = -1
BUFFER_SMALL = -2
INDEX_RANGE = -3
PAD_NONZERO = 1


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc.  Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_CFLAGS, "-shared", "-pthread", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # VQ_ORACLE_LIB names another build of vq_oracle.c (the sanitizer build of the tests)
        path = os.environ.get("VQ_ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            path = _LIB_PATH
        lib = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_f32_to_f16_rne_array.argtypes = [vp, vp, i64]
        lib.oracle_f32_to_f16_rne_array.restype = None
        lib.oracle_f32_to_bf16_rne_array.argtypes = [vp, vp, i64]
        lib.oracle_f32_to_bf16_rne_array.restype = None
        lib.oracle_row_stride.argtypes = [i64, i32, i32]
        lib.oracle_row_stride.restype = i64
        lib.oracle_packed_bytes.argtypes = [i64, i64, i32, i32, i32]
        lib.oracle_packed_bytes.restype = i64
        lib.oracle_pack.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, i64]
        lib.oracle_pack.restype = i32
        lib.oracle_unpack.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp]
        lib.oracle_unpack.restype = i32
        lib.oracle_dequant_rows.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, i32]
        lib.oracle_dequant_rows.restype = i32
        lib.oracle_forward_rows.argtypes = [i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i64, vp, i64,
                                            vp, i32]
        lib.oracle_forward_rows.restype = i32
        lib.oracle_svq_dequant_rows.argtypes = [i64, i64, vp, vp, vp, vp, vp, i64, vp, i32]
        lib.oracle_svq_dequant_rows.restype = i32
        lib.oracle_svq_forward_rows.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, i32, i64, vp, i64, vp, i32]
        lib.oracle_svq_forward_rows.restype = i32
        lib.oracle_rht_block.argtypes = [i64]
        lib.oracle_rht_block.restype = i64
        lib.oracle_rht.argtypes = [i64, i64, vp, vp, i32, vp]
        lib.oracle_rht.restype = i32
        lib.oracle_rvq_assign.argtypes = [i64, i64, i32, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_rvq_assign.restype = i32
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    """fp16 / bf16 / uint16 numpy array -> contiguous uint16 bit view (None passes)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 bit patterns, got %s" % a.dtype)
    return a


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc < 0:
        raise OracleError("%s failed with code %d" % (what, rc))
    return rc


# ------------------------------------------------------------------ number formats

def f16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_f16_to_f64(int(v)) for v in b], dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.oracle_bf16_to_f64(int(v)) for v in b], dtype=np.float64)


def f64_to_f16_rne(vals) -> np.ndarray:
    lib = _load()
    v = np.asarray(vals, dtype=np.float64).ravel()
    return np.array([lib.oracle_f64_to_f16_rne(float(x)) for x in v], dtype=np.uint16)


def f64_to_bf16_rne(vals) -> np.ndarray:
    lib = _load()
    v = np.asarray(vals, dtype=np.float64).ravel()
    return np.array([lib.oracle_f64_to_bf16_rne(float(x)) for x in v], dtype=np.uint16)


def f32_array_to_f16_rne(a) -> np.ndarray:
    """RNE of an fp32 array to binary16 bits (same rounding as f64_to_f16_rne)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.zeros(a.shape, dtype=np.uint16)
    _load().oracle_f32_to_f16_rne_array(_ptr(a), _ptr(out), a.size)
    return out


def f32_array_to_bf16_rne(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.zeros(a.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16_rne_array(_ptr(a), _ptr(out), a.size)
    return out


# ------------------------------------------------------------------ layout

def num_vectors(in_features: int, v: int) -> int:
    return (in_features + v - 1) // v


def row_stride(in_features: int, v: int, bits: int) -> int:
    return int(_load().oracle_row_stride(in_features, v, bits))


def packed_bytes(n: int, in_features: int, v: int, bits1: int, bits2: int) -> int:
    r = int(_load().oracle_packed_bytes(n, in_features, v, bits1, bits2))
    if r < 0:
        raise OracleError("invalid descriptor")
    return r


def pack(n, in_features, v, bits1, bits2, idx1, idx2=None) -> np.ndarray:
    nv = num_vectors(in_features, v)
    i1 = np.ascontiguousarray(idx1, dtype=np.uint32).reshape(n, nv)
    i2 = None if bits2 == 0 else np.ascontiguousarray(idx2, dtype=np.uint32).reshape(n, nv)
    nb = packed_bytes(n, in_features, v, bits1, bits2)
    out = np.zeros(max(nb, 1), dtype=np.uint8)
    _check(_load().oracle_pack(n, in_features, v, bits1, bits2, _ptr(i1), _ptr(i2), _ptr(out), nb), "oracle_pack")
    return out[:nb]


def unpack(n, in_features, v, bits1, bits2, packed):
    """Returns (idx1, idx2 or None, pad_bits_were_zero)."""
    nv = num_vectors(in_features, v)
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    if p.size < packed_bytes(n, in_features, v, bits1, bits2):
        raise OracleError("packed buffer too small")
    i1 = np.zeros((n, nv), dtype=np.uint32)
    i2 = np.zeros((n, nv), dtype=np.uint32) if bits2 else None
    rc = _check(_load().oracle_unpack(n, in_features, v, bits1, bits2, _ptr(p), _ptr(i1), _ptr(i2)), "oracle_unpack")
    return i1, i2, rc == OK


# ------------------------------------------------------------------ dequant and product

def dequant(n, in_features, v, bits1, bits2, packed, cb1, cb2=None, scale=None, rows=None, nthreads=0):
    """fp32 W rows [len(rows) or n, in_features] exactly as the decode defines them."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.size
    w = np.zeros((nrows, in_features), dtype=np.float32)
    _check(_load().oracle_dequant_rows(n, in_features, v, bits1, bits2, _ptr(p), _ptr(_u16(cb1)),
                                       _ptr(_u16(cb2) if bits2 else None), _ptr(_u16(scale)), _ptr(r), nrows,
                                       _ptr(w), nthreads), "oracle_dequant_rows")
    return w


def forward(n, in_features, v, bits1, bits2, packed, cb1, cb2, scale, bias, x_bits, x_is_bf16, M, rows=None,
            nthreads=0):
    """y64 [M, len(rows) or n]: fp64 sum over columns of x * fp32 W (+ bias)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    xb = _u16(x_bits) if M * in_features > 0 else None
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.size
    y = np.zeros((M, nrows), dtype=np.float64)
    _check(_load().oracle_forward_rows(n, in_features, v, bits1, bits2, _ptr(p), _ptr(_u16(cb1)),
                                       _ptr(_u16(cb2) if bits2 else None), _ptr(_u16(scale)), _ptr(_u16(bias)),
                                       _ptr(xb), int(bool(x_is_bf16)), M, _ptr(r), nrows, _ptr(y), nthreads),
           "oracle_forward_rows")
    return y


# ------------------------------------------------------------------ affine lattice (UniSVQ)

def svq_dequant(n, in_features, packed, a, b, scale=None, rows=None, nthreads=0):
    """fp32 W rows of an affine-lattice layer: coordinate t of a vector is
    fl32(B[t] + sum_u A[t][u] q_u) (times the channel scale in fp32)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.size
    w = np.zeros((nrows, in_features), dtype=np.float32)
    _check(_load().oracle_svq_dequant_rows(n, in_features, _ptr(p), _ptr(_u16(np.ravel(a))), _ptr(_u16(np.ravel(b))),
                                           _ptr(_u16(scale)), _ptr(r), nrows, _ptr(w), nthreads),
           "oracle_svq_dequant_rows")
    return w


def svq_forward(n, in_features, packed, a, b, scale, bias, x_bits, x_is_bf16, M, rows=None, nthreads=0):
    """y64 [M, len(rows) or n] of an affine-lattice layer: fp64 sum of x times fp32 W (+ bias)."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    xb = _u16(x_bits) if M * in_features > 0 else None
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.size
    y = np.zeros((M, nrows), dtype=np.float64)
    _check(_load().oracle_svq_forward_rows(n, in_features, _ptr(p), _ptr(_u16(np.ravel(a))), _ptr(_u16(np.ravel(b))),
                                           _ptr(_u16(scale)), _ptr(_u16(bias)), _ptr(xb), int(bool(x_is_bf16)), M,
                                           _ptr(r), nrows, _ptr(y), nthreads),
           "oracle_svq_forward_rows")
    return y


# ------------------------------------------------------------------ randomized Hadamard transform

def rht_block(n: int) -> int:
    """Block size of the transform: the largest power of two dividing n, at most 16384."""
    return int(_load().oracle_rht_block(n))


def rht(x, signs, transpose=False):
    """Randomized Walsh-Hadamard transform of the rows of x (any float array [M, n]),
    computed in fp64 as the matrix product.  signs: uint8 bit array (bit j set: s_j = -1)."""
    xd = np.ascontiguousarray(np.atleast_2d(np.asarray(x, dtype=np.float64)))
    m, n = xd.shape
    sg = np.ascontiguousarray(signs, dtype=np.uint8)
    if sg.size * 8 < n:
        raise OracleError("sign bits too short")
    y = np.zeros_like(xd)
    _check(_load().oracle_rht(m, n, _ptr(xd), _ptr(sg), int(bool(transpose)), _ptr(y)), "oracle_rht")
    return y


# ------------------------------------------------------------------ residual VQ encode

def rvq_assign(w, v, cb1, cb2=None):
    """(idx1, idx2 or None) [n, in / v]: nearest main centroid, then nearest residual centroid of
    the fp32 residual; nearest = the exact minimum of |w - c|^2 (decided in exact arithmetic),
    ties to the lowest index; non-finite values as described in vq_oracle.h.  w: any float
    array [n, in] whose values are fp32-representable (fp16 / bf16 / fp32 weights)."""
    wd = np.ascontiguousarray(np.atleast_2d(np.asarray(w, dtype=np.float64)))
    n, i = wd.shape
    c1 = np.ascontiguousarray(_u16(cb1)).reshape(-1)
    k1 = c1.size // v
    c2 = None if cb2 is None else np.ascontiguousarray(_u16(cb2)).reshape(-1)
    k2 = 0 if c2 is None else c2.size // v
    nv = i // v if v > 0 else 0
    idx1 = np.zeros((n, nv), dtype=np.uint32)
    idx2 = np.zeros((n, nv), dtype=np.uint32) if k2 else None
    _check(_load().oracle_rvq_assign(n, i, v, k1, k2, _ptr(wd), _ptr(c1), _ptr(c2), _ptr(idx1), _ptr(idx2)),
           "oracle_rvq_assign")
    return idx1, idx2
