"""Python binding of libvq, the gfx950 VQ dequantize-and-multiply library.

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libvq.so`` behind the C ABI of ``include/vq.h``.  PyTorch provides device memory and
streams.  If the library is not built, the first call raises: there is no fallback
path, and nothing here computes.

Calls (same names as the C ABI):
    packed_bytes(desc) -> int
    pack(desc, idx1, idx2=None) -> numpy uint8 (host packing in desc.layout, vq.h)
    dequant(desc, packed, cb1, cb2, scale, w_dtype=torch.float32, out=None) -> W^ [N, IN]
    gemv(desc, packed, cb1, cb2, scale, bias, x, y_dtype=None, out=None)  # 1 <= M <= 16
    gemv_workspace_bytes(desc, m, x_dtype) -> int
    gemv_ws(desc, packed, cb1, cb2, scale, bias, x, workspace, y_dtype=None, out=None)
    gemm(desc, packed, cb1, cb2, scale, bias, x, y_dtype=None, out=None)  # any M, MFMA
    gemm_workspace_bytes(desc, m, x_dtype) -> int
    gemm_ws(desc, packed, cb1, cb2, scale, bias, x, workspace, y_dtype=None, out=None)
plus ``workspace(desc, m, x_dtype, device)`` and ``gemm_workspace(...)``, zero-filled
device buffers for gemv_ws / gemm_ws, and ``VQLinear``, a layer object holding the packed
weights that picks gemv_ws or gemm_ws by batch size, the analogue of the VPTQ guide's
``VPTQLinear`` module.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvq.so")

VQ_OK = 0
VQ_ERR_NULL = -1
VQ_ERR_SHAPE = -2
VQ_ERR_BITS = -3
VQ_ERR_UNSUPPORTED = -4
VQ_ERR_ALIGN = -5
VQ_ERR_INDEX_RANGE = -6
VQ_ERR_BUFFER_SIZE = -7
VQ_ERR_HIP = -8

VQ_F16, VQ_BF16, VQ_F32 = 0, 1, 2
LAYOUT_ROWSTREAM = 1
LAYOUT_BUCKETED = 2  # slice-bucketed: the batch-1 decode layout of gemv_ws (v = 8, bits1 = 16)

EXPORTED = ("vq_abi_version", "vq_status_string", "vq_packed_bytes", "vq_pack", "vq_dequant", "vq_gemv",
            "vq_gemv_workspace_bytes", "vq_gemv_ws", "vq_gemm", "vq_svq_dequant", "vq_svq_gemv", "vq_rht", "vq_rht_block",
            "vq_assign_workspace_bytes", "vq_assign", "vq_svq_gemm", "vq_gemv_noalloc", "vq_svq_pack",
            "vq_gemm_workspace_bytes", "vq_gemm_ws", "vq_rht_product_workspace_bytes", "vq_gemv_ws_rht",
            "vq_gemm_ws_rht")


class Desc(ctypes.Structure):
    _fields_ = [("out_features", ctypes.c_int32), ("in_features", ctypes.c_int32), ("v", ctypes.c_int32),
                ("bits1", ctypes.c_int32), ("bits2", ctypes.c_int32), ("layout", ctypes.c_int32)]

    def __repr__(self):
        return "Desc(N=%d, IN=%d, v=%d, bits1=%d, bits2=%d, layout=%d)" % (
            self.out_features, self.in_features, self.v, self.bits1, self.bits2, self.layout)


def make_desc(out_features, in_features, v, bits1, bits2=0, layout=LAYOUT_ROWSTREAM) -> Desc:
    return Desc(out_features, in_features, v, bits1, bits2, layout)


class VQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, _status_string(status)))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libvq.so is not built (%s); run `python -m gemv_bit_unpack_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    lib.vq_abi_version.argtypes = []
    lib.vq_abi_version.restype = i32
    lib.vq_status_string.argtypes = [ctypes.c_int]
    lib.vq_status_string.restype = ctypes.c_char_p
    lib.vq_packed_bytes.argtypes = [dp, ctypes.POINTER(sz)]
    lib.vq_packed_bytes.restype = ctypes.c_int
    lib.vq_pack.argtypes = [dp, vp, vp, vp, sz]
    lib.vq_svq_pack.argtypes = [dp, vp, vp, sz]
    lib.vq_svq_pack.restype = ctypes.c_int
    lib.vq_pack.restype = ctypes.c_int
    lib.vq_dequant.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.vq_dequant.restype = ctypes.c_int
    for name in ("vq_gemv", "vq_gemm"):
        f = getattr(lib, name)
        f.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp]
        f.restype = ctypes.c_int
    lib.vq_gemv_workspace_bytes.argtypes = [dp, i32, ctypes.c_int, ctypes.POINTER(sz)]
    lib.vq_gemv_workspace_bytes.restype = ctypes.c_int
    lib.vq_gemv_ws.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp, sz, vp]
    lib.vq_gemv_ws.restype = ctypes.c_int
    lib.vq_gemm_workspace_bytes.argtypes = [dp, i32, ctypes.c_int, ctypes.POINTER(sz)]
    lib.vq_gemm_workspace_bytes.restype = ctypes.c_int
    lib.vq_gemm_ws.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp, sz, vp]
    lib.vq_gemm_ws.restype = ctypes.c_int
    lib.vq_rht_product_workspace_bytes.argtypes = [dp, i32, ctypes.c_int, i32, ctypes.POINTER(sz)]
    lib.vq_rht_product_workspace_bytes.restype = ctypes.c_int
    for name in ("vq_gemv_ws_rht", "vq_gemm_ws_rht"):
        getattr(lib, name).argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, vp, ctypes.c_int, vp, sz, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.vq_gemv_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp]
    lib.vq_gemv_noalloc.restype = ctypes.c_int
    lib.vq_svq_dequant.argtypes = [dp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
    lib.vq_svq_dequant.restype = ctypes.c_int
    lib.vq_svq_gemv.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp]
    lib.vq_svq_gemv.restype = ctypes.c_int
    lib.vq_svq_gemm.argtypes = [dp, vp, vp, vp, vp, vp, vp, ctypes.c_int, i32, vp, ctypes.c_int, vp]
    lib.vq_svq_gemm.restype = ctypes.c_int
    lib.vq_rht.argtypes = [i32, i32, vp, ctypes.c_int, vp, i32, vp, ctypes.c_int, vp]
    lib.vq_rht.restype = ctypes.c_int
    lib.vq_rht_block.argtypes = [i32]
    lib.vq_rht_block.restype = i32
    lib.vq_assign_workspace_bytes.argtypes = [dp, ctypes.POINTER(sz)]
    lib.vq_assign_workspace_bytes.restype = ctypes.c_int
    lib.vq_assign.argtypes = [dp, vp, ctypes.c_int, vp, vp, vp, vp, vp, sz, vp]
    lib.vq_assign.restype = ctypes.c_int
    return lib


_lib = None


def lib():
    """The loaded ctypes handle of libvq.so (raw C ABI); raises if it is not built."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _status_string(status) -> str:
    s = lib().vq_status_string(int(status))
    return s.decode() if s else "unknown"


def _check(status, where):
    if status != VQ_OK:
        raise VQError(status, where)


def abi_version() -> int:
    return int(lib().vq_abi_version())


def packed_bytes(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().vq_packed_bytes(ctypes.byref(desc), ctypes.byref(n)), "vq_packed_bytes")
    return int(n.value)


def pack(desc: Desc, idx1, idx2=None) -> np.ndarray:
    """Host packing of uint32 indices [N, nv] into desc.layout (row stream or slice-bucketed)."""
    nv = (desc.in_features + desc.v - 1) // desc.v
    i1 = np.ascontiguousarray(np.asarray(idx1, dtype=np.uint32).reshape(desc.out_features, nv))
    i2 = None
    if desc.bits2:
        i2 = np.ascontiguousarray(np.asarray(idx2, dtype=np.uint32).reshape(desc.out_features, nv))
    nb = packed_bytes(desc)
    out = np.zeros(max(nb, 1), dtype=np.uint8)
    _check(lib().vq_pack(ctypes.byref(desc), i1.ctypes.data_as(ctypes.c_void_p),
                        None if i2 is None else i2.ctypes.data_as(ctypes.c_void_p),
                        out.ctypes.data_as(ctypes.c_void_p), nb), "vq_pack")
    return out[:nb]


# ------------------------------------------------------------------ torch marshalling

def _torch():
    import torch

    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float16:
        return VQ_F16
    if dt == torch.bfloat16:
        return VQ_BF16
    if dt == torch.float32:
        return VQ_F32
    raise TypeError("unsupported dtype %s" % dt)


def _dev_ptr(t, what, dtypes=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (what, t.dtype, dtypes))
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def dequant(desc: Desc, packed, cb1, cb2, scale, w_dtype=None, out=None):
    torch = _torch()
    w_dtype = w_dtype or torch.float32
    if out is None:
        out = torch.empty((desc.out_features, desc.in_features), dtype=w_dtype, device=packed.device)
    f16 = (torch.float16,)
    st = lib().vq_dequant(ctypes.byref(desc), _dev_ptr(packed, "packed"), _dev_ptr(cb1, "cb1", f16),
                         _dev_ptr(cb2, "cb2", f16) if desc.bits2 else None, _dev_ptr(scale, "scale", f16),
                         _dev_ptr(out, "out"), _dtype_code(out.dtype), _stream_ptr(packed.device))
    _check(st, "vq_dequant")
    return out


def _product(fn, name, desc, packed, cb1, cb2, scale, bias, x, y_dtype, out, extra=()):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != desc.in_features:
        raise ValueError("x must be [M, %d], got %s" % (desc.in_features, tuple(x.shape)))
    m = x.shape[0]
    y_dtype = y_dtype or x.dtype
    if out is None:
        out = torch.empty((m, desc.out_features), dtype=y_dtype, device=x.device)
    f16 = (torch.float16,)
    st = fn(ctypes.byref(desc), _dev_ptr(packed, "packed"), _dev_ptr(cb1, "cb1", f16),
            _dev_ptr(cb2, "cb2", f16) if desc.bits2 else None, _dev_ptr(scale, "scale", f16),
            _dev_ptr(bias, "bias", f16), _dev_ptr(x, "x", (torch.float16, torch.bfloat16)), _dtype_code(x.dtype),
            m, _dev_ptr(out, "out"), _dtype_code(out.dtype), *extra, _stream_ptr(x.device))
    _check(st, name)
    return out


def gemv(desc, packed, cb1, cb2, scale, bias, x, y_dtype=None, out=None):
    return _product(lib().vq_gemv, "vq_gemv", desc, packed, cb1, cb2, scale, bias, x, y_dtype, out)


def gemv_workspace_bytes(desc: Desc, m: int, x_dtype) -> int:
    """Workspace bytes for gemv_ws at batch m with activations of torch dtype x_dtype (0: none used)."""
    n = ctypes.c_size_t(0)
    _check(lib().vq_gemv_workspace_bytes(ctypes.byref(desc), int(m), _dtype_code(x_dtype), ctypes.byref(n)),
           "vq_gemv_workspace_bytes")
    return int(n.value)


def workspace(desc: Desc, m: int, x_dtype, device="cuda"):
    """A zero-filled device workspace for gemv_ws (None when the shape needs none)."""
    nbytes = gemv_workspace_bytes(desc, m, x_dtype)
    if nbytes == 0:
        return None
    return _torch().zeros(nbytes, dtype=_torch().uint8, device=device)


def gemv_ws(desc, packed, cb1, cb2, scale, bias, x, ws, y_dtype=None, out=None):
    """gemv with a caller-owned workspace (from ``workspace``; None: plain gemv).

    Calls that share a workspace must be ordered (one stream)."""
    extra = (None, 0) if ws is None else (_dev_ptr(ws, "workspace"), ws.numel() * ws.element_size())
    return _product(lib().vq_gemv_ws, "vq_gemv_ws", desc, packed, cb1, cb2, scale, bias, x, y_dtype, out, extra)


def gemv_noalloc(desc, packed, cb1, cb2, scale, bias, x, y_dtype=None, out=None):
    """gemv_ws with the library's fixed per-GPU workspace: allocates nothing (``out`` given).

    Calls on one GPU share that workspace and must not overlap."""
    return _product(lib().vq_gemv_noalloc, "vq_gemv_noalloc", desc, packed, cb1, cb2, scale, bias, x, y_dtype, out)


def gemm(desc, packed, cb1, cb2, scale, bias, x, y_dtype=None, out=None):
    return _product(lib().vq_gemm, "vq_gemm", desc, packed, cb1, cb2, scale, bias, x, y_dtype, out)


def gemm_workspace_bytes(desc: Desc, m: int, x_dtype) -> int:
    """Workspace bytes for gemm_ws at batch m with activations of torch dtype x_dtype (0: none used)."""
    n = ctypes.c_size_t(0)
    _check(lib().vq_gemm_workspace_bytes(ctypes.byref(desc), int(m), _dtype_code(x_dtype), ctypes.byref(n)),
           "vq_gemm_workspace_bytes")
    return int(n.value)


def gemm_workspace(desc: Desc, m: int, x_dtype, device="cuda"):
    """A zero-filled device workspace for gemm_ws (None when the shape needs none)."""
    nbytes = gemm_workspace_bytes(desc, m, x_dtype)
    if nbytes == 0:
        return None
    return _torch().zeros(nbytes, dtype=_torch().uint8, device=device)


def gemm_ws(desc, packed, cb1, cb2, scale, bias, x, ws, y_dtype=None, out=None):
    """gemm with a caller-owned workspace (from ``gemm_workspace``; None where none is needed).

    Calls that share a workspace must be ordered (one stream)."""
    extra = (None, 0) if ws is None else (_dev_ptr(ws, "workspace"), ws.numel() * ws.element_size())
    return _product(lib().vq_gemm_ws, "vq_gemm_ws", desc, packed, cb1, cb2, scale, bias, x, y_dtype, out, extra)


def svq_desc(out_features, in_features) -> Desc:
    """Descriptor of an affine-lattice layer: one 8-bit field of four 2-bit codes per 4-vector."""
    return make_desc(out_features, in_features, 4, 8, 0)


def svq_pack(desc: Desc, q) -> np.ndarray:
    """Integer grid coordinates q [N, nv, 4] (values 0..3) of an affine-lattice layer -> its
    packed row stream (host bytes), through vq_svq_pack."""
    qa = np.ascontiguousarray(q, dtype=np.uint8)
    nv = (desc.in_features + 3) // 4
    if qa.shape != (desc.out_features, nv, 4):
        raise ValueError("q must be [%d, %d, 4], got %s" % (desc.out_features, nv, qa.shape))
    out = np.zeros(max(packed_bytes(desc), 1), dtype=np.uint8)
    st = lib().vq_svq_pack(ctypes.byref(desc), qa.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p),
                           out.size)
    _check(st, "vq_svq_pack")
    return out[:packed_bytes(desc)]


def svq_dequant(desc: Desc, packed, a, b, scale, w_dtype=None, out=None):
    """W^ of an affine-lattice layer (a: fp16 [4, 4], b: fp16 [4] device tensors)."""
    torch = _torch()
    w_dtype = w_dtype or torch.float32
    if out is None:
        out = torch.empty((desc.out_features, desc.in_features), dtype=w_dtype, device=packed.device)
    f16 = (torch.float16,)
    st = lib().vq_svq_dequant(ctypes.byref(desc), _dev_ptr(packed, "packed"), _dev_ptr(a, "a", f16),
                             _dev_ptr(b, "b", f16), _dev_ptr(scale, "scale", f16), _dev_ptr(out, "out"),
                             _dtype_code(out.dtype), _stream_ptr(packed.device))
    _check(st, "vq_svq_dequant")
    return out


def svq_gemv(desc: Desc, packed, a, b, scale, bias, x, y_dtype=None, out=None):
    """y [M, N] = x W^T (+ bias) of an affine-lattice layer, 1 <= M <= 16."""
    return _svq_product(lib().vq_svq_gemv, "vq_svq_gemv", desc, packed, a, b, scale, bias, x, y_dtype, out)


def svq_gemm(desc: Desc, packed, a, b, scale, bias, x, y_dtype=None, out=None):
    """y [M, N] = x W^T (+ bias) of an affine-lattice layer on the matrix cores, any M."""
    return _svq_product(lib().vq_svq_gemm, "vq_svq_gemm", desc, packed, a, b, scale, bias, x, y_dtype, out)


def _svq_product(fn, name, desc, packed, a, b, scale, bias, x, y_dtype, out):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != desc.in_features:
        raise ValueError("x must be [M, %d], got %s" % (desc.in_features, tuple(x.shape)))
    m = x.shape[0]
    y_dtype = y_dtype or x.dtype
    if out is None:
        out = torch.empty((m, desc.out_features), dtype=y_dtype, device=x.device)
    f16 = (torch.float16,)
    st = fn(ctypes.byref(desc), _dev_ptr(packed, "packed"), _dev_ptr(a, "a", f16), _dev_ptr(b, "b", f16),
            _dev_ptr(scale, "scale", f16), _dev_ptr(bias, "bias", f16),
            _dev_ptr(x, "x", (torch.float16, torch.bfloat16)), _dtype_code(x.dtype), m, _dev_ptr(out, "out"),
            _dtype_code(out.dtype), _stream_ptr(x.device))
    _check(st, name)
    return out


def rht_block(n: int) -> int:
    """Block size of vq_rht for rows of n columns."""
    return int(lib().vq_rht_block(int(n)))


def rht(x, signs, transpose=False, y_dtype=None, out=None):
    """Randomized Hadamard transform of the rows of x [M, n] (device tensor); signs: uint8
    device tensor of ceil(n / 8) bytes.  ``transpose=True`` applies the inverse."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M, n]")
    m, n = x.shape
    if signs.dtype != torch.uint8 or signs.numel() * 8 < n:
        raise ValueError("signs must be a uint8 tensor of at least ceil(n / 8) bytes")
    y_dtype = y_dtype or x.dtype
    if out is None:
        out = torch.empty((m, n), dtype=y_dtype, device=x.device)
    st = lib().vq_rht(m, n, _dev_ptr(x, "x", (torch.float16, torch.bfloat16, torch.float32)), _dtype_code(x.dtype),
                      _dev_ptr(signs, "signs"), int(bool(transpose)), _dev_ptr(out, "out"), _dtype_code(out.dtype),
                      _stream_ptr(x.device))
    _check(st, "vq_rht")
    return out


def assign_workspace_bytes(desc: Desc) -> int:
    """Device workspace bytes that vq_assign needs for desc's codebooks."""
    n = ctypes.c_size_t(0)
    _check(lib().vq_assign_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "vq_assign_workspace_bytes")
    return int(n.value)


def assign(desc: Desc, w, cb1, cb2=None, ws=None, out1=None, out2=None):
    """Residual VQ encode of W [N, IN] (fp16 / bf16 / fp32 device tensor) against fp16
    codebooks: (idx1, idx2) as int32 tensors [N, IN / v] holding the uint32 indices
    (idx2 None when desc.bits2 == 0).  ws: a uint8 device tensor of at least
    assign_workspace_bytes(desc) bytes (allocated here when None)."""
    torch = _torch()
    if w.dim() != 2 or tuple(w.shape) != (desc.out_features, desc.in_features):
        raise ValueError("w must be [%d, %d], got %s" % (desc.out_features, desc.in_features, tuple(w.shape)))
    nv = desc.in_features // desc.v if desc.v > 0 else 0
    if out1 is None:
        out1 = torch.empty((desc.out_features, nv), dtype=torch.int32, device=w.device)
    if desc.bits2 and out2 is None:
        out2 = torch.empty((desc.out_features, nv), dtype=torch.int32, device=w.device)
    if ws is None:
        ws = torch.empty(max(assign_workspace_bytes(desc), 256), dtype=torch.uint8, device=w.device)
    f16 = (torch.float16,)
    st = lib().vq_assign(ctypes.byref(desc), _dev_ptr(w, "w", (torch.float16, torch.bfloat16, torch.float32)),
                         _dtype_code(w.dtype), _dev_ptr(cb1, "cb1", f16),
                         _dev_ptr(cb2, "cb2", f16) if desc.bits2 else None, _dev_ptr(out1, "idx1", (torch.int32,)),
                         _dev_ptr(out2, "idx2", (torch.int32,)) if desc.bits2 else None, _dev_ptr(ws, "workspace"),
                         ws.numel() * ws.element_size(), _stream_ptr(w.device))
    _check(st, "vq_assign")
    return out1, (out2 if desc.bits2 else None)


_stream_ws = {}


def rht_product_workspace_bytes(desc: Desc, m: int, x_dtype, gemm: bool) -> int:
    """Workspace bytes for gemv_ws_rht (gemm False) or gemm_ws_rht (gemm True)."""
    n = ctypes.c_size_t(0)
    _check(lib().vq_rht_product_workspace_bytes(ctypes.byref(desc), int(m), _dtype_code(x_dtype), int(bool(gemm)),
                                                ctypes.byref(n)), "vq_rht_product_workspace_bytes")
    return int(n.value)


def rht_workspace(desc: Desc, m: int, x_dtype, gemm: bool, device="cuda"):
    """A zero-filled device workspace for gemv_ws_rht / gemm_ws_rht (None when none is needed)."""
    nbytes = rht_product_workspace_bytes(desc, m, x_dtype, gemm)
    if nbytes == 0:
        return None
    return _torch().zeros(nbytes, dtype=_torch().uint8, device=device)


def _rht_product(gemm, desc, packed, cb1, cb2, scale, bias, x, signs, ws, y_dtype=None, out=None):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != desc.in_features:
        raise ValueError("x must be [M, %d], got %s" % (desc.in_features, tuple(x.shape)))
    m = x.shape[0]
    y_dtype = y_dtype or x.dtype
    if out is None:
        out = torch.empty((m, desc.out_features), dtype=y_dtype, device=x.device)
    f16 = (torch.float16,)
    name = "vq_gemm_ws_rht" if gemm else "vq_gemv_ws_rht"
    wsp, wsb = (None, 0) if ws is None else (_dev_ptr(ws, "workspace"), ws.numel() * ws.element_size())
    st = getattr(lib(), name)(ctypes.byref(desc), _dev_ptr(packed, "packed"), _dev_ptr(cb1, "cb1", f16),
                              _dev_ptr(cb2, "cb2", f16) if desc.bits2 else None, _dev_ptr(scale, "scale", f16),
                              _dev_ptr(bias, "bias", f16), _dev_ptr(x, "x", (torch.float16, torch.bfloat16)),
                              _dtype_code(x.dtype), m, _dev_ptr(signs, "signs", (torch.uint8,)), _dev_ptr(out, "out"),
                              _dtype_code(out.dtype), wsp, wsb, _stream_ptr(x.device))
    _check(st, name)
    return out


def gemv_ws_rht(desc, packed, cb1, cb2, scale, bias, x, signs, ws, y_dtype=None, out=None):
    """gemv_ws on the randomized Hadamard transform of x (vq_rht forward, `signs` uint8 bits),
    the transform fused into the x pass where the shape has the workspace path."""
    return _rht_product(False, desc, packed, cb1, cb2, scale, bias, x, signs, ws, y_dtype, out)


def gemm_ws_rht(desc, packed, cb1, cb2, scale, bias, x, signs, ws, y_dtype=None, out=None):
    """gemm_ws on the randomized Hadamard transform of x, as gemv_ws_rht."""
    return _rht_product(True, desc, packed, cb1, cb2, scale, bias, x, signs, ws, y_dtype, out)


def stream_workspace(desc: Desc, m: int, x_dtype, device, gemm_path: bool = False):
    """A workspace kept per (device, current stream), grown on demand, for layers that run
    their calls in stream order (gemv_ws, or gemm_ws with ``gemm_path``).  None when the
    shape needs none."""
    torch = _torch()
    nbytes = (gemm_workspace_bytes if gemm_path else gemv_workspace_bytes)(desc, m, x_dtype)
    if nbytes == 0:
        return None
    dev = torch.device(device)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(),
           torch.cuda.current_stream(dev).cuda_stream)
    ws = _stream_ws.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        _stream_ws[key] = ws
    return ws


class VQLinear:
    """A quantized linear layer: packed indices, fp16 codebooks, per-channel scale, bias.

    ``forward(x)`` computes x W^T (+ bias) for x of shape [..., in_features]; batches of
    up to ``gemv_max_m`` rows take gemv_ws (the codebook-sliced kernel where the shape has
    it), larger ones gemm_ws (the matrix-core product fed by the gathering lanes where the
    shape has it); both with a workspace kept per device and stream.  With
    ``decode_packed`` (the same indices in the slice-bucketed layout, ``decode_desc``) a
    batch of one row takes the bucketed decode product instead.
    """

    def __init__(self, desc: Desc, packed, cb1, cb2=None, scale=None, bias=None, gemv_max_m: int = 16,
                 decode_desc: Desc | None = None, decode_packed=None):
        self.desc = desc
        self.packed, self.cb1, self.cb2, self.scale, self.bias = packed, cb1, cb2, scale, bias
        self.gemv_max_m = min(int(gemv_max_m), 16)
        self.decode_desc, self.decode_packed = decode_desc, decode_packed

    @classmethod
    def from_indices(cls, desc: Desc, idx1, idx2, cb1, cb2=None, scale=None, bias=None, device="cuda",
                     decode_layout: bool = False):
        """Packs the indices (and, with ``decode_layout``, their slice-bucketed copy for
        batch-1 decode: 32 bits per vector) and uploads them."""
        torch = _torch()
        packed = torch.from_numpy(pack(desc, idx1, idx2)).to(device)
        ddesc = dpacked = None
        if decode_layout:
            ddesc = make_desc(desc.out_features, desc.in_features, desc.v, desc.bits1, desc.bits2, LAYOUT_BUCKETED)
            dpacked = torch.from_numpy(pack(ddesc, idx1, idx2)).to(device)
        return cls(desc, packed, cb1, cb2, scale, bias, decode_desc=ddesc, decode_packed=dpacked)

    def forward(self, x, y_dtype=None):
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        args = (self.desc, self.packed, self.cb1, self.cb2, self.scale, self.bias, x2)
        if x2.shape[0] == 1 and self.decode_packed is not None:
            dargs = (self.decode_desc, self.decode_packed, self.cb1, self.cb2, self.scale, self.bias, x2)
            ws = stream_workspace(self.decode_desc, 1, x2.dtype, x2.device)
            y = gemv_ws(*dargs, ws, y_dtype)
        elif x2.shape[0] <= self.gemv_max_m:
            ws = stream_workspace(self.desc, x2.shape[0], x2.dtype, x2.device)
            y = gemv_ws(*args, ws, y_dtype)
        else:
            ws = stream_workspace(self.desc, x2.shape[0], x2.dtype, x2.device, gemm_path=True)
            y = gemm_ws(*args, ws, y_dtype)
        return y.reshape(*lead, self.desc.out_features)

    __call__ = forward
