"""Benchmark of the VQ dequantize-and-multiply path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one decode pass over the 70B-class MLP layer pair: vq_gemv_ws (vq_gemv with a
caller-owned workspace, the call VQLinear makes for decode batches) at M = 1 on the
28672 x 8192 "up" layer, then on the 8192 x 28672 "down" layer; v = 8, a 65536-entry main
codebook plus a 256-entry residual codebook (3 index bits per weight), bf16 x and y.  Steps
rotate through a ring of distinct layer copies (own indices, codebooks and scales each)
totalling more than 1 GiB per layer, so the 256 MB Infinity Cache cannot hold the stream
and every step reads its indices from HBM.  W warm-up steps run first; exactly K steps are
captured in one HIP graph, replayed once untimed, then timed in 5 trials (median reported,
minimum beside it).

Printed: ONE JSON line with the throughput on algorithmic bytes (packed indices + each
codebook once + scales + x + y), the roofline of the call, the cold single-call latency,
the GEMV / GEMM crossover on the same layers, the prefill GEMM at M = 128 (vq_gemm_ws,
with vq_gemm beside it), the GEMV at M = 1 on every workload, the other legs, and the CPU
oracle timed on the host's cores on every workload.

Inputs are synthetic: uniform indices (a packed stream of uniform random bits),
centroids 0.02*N(0,1) main and 0.005*N(0,1) residual in fp16, scales U(0.5, 1.5),
x ~ N(0,1); all seeded.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
import zlib

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16
RING_BYTES = 1 << 30         # > 4x the 256 MB Infinity Cache
MAX_COPIES = 512             # tiny layers: the ring stays cache-resident, said in the output

WORKLOADS = {
    # key: (layers [(N, IN)], v, bits1, bits2, x dtype)
    "tiny": ([(256, 256)], 8, 8, 0, "f16"),
    "dec4k": ([(4096, 4096)], 8, 16, 0, "f16"),
    "dec4k_res": ([(4096, 4096)], 8, 16, 8, "f16"),
    "mlp8b": ([(14336, 4096), (4096, 14336)], 6, 12, 12, "f16"),
    "l70b": ([(28672, 8192), (8192, 28672)], 8, 16, 8, "bf16"),
    "aqlm4k": ([(4096, 4096)], 8, 16, 16, "f16"),
    "v16_4k": ([(4096, 4096)], 16, 16, 8, "f16"),
}
DESCRIBE = {
    "tiny": "256x256 v8 K1=256 (1 bit/weight)",
    "dec4k": "4096x4096 v8 K1=65536 (2 bits/weight)",
    "dec4k_res": "4096x4096 v8 K1=65536+K2=256 (3 bits/weight)",
    "mlp8b": "MLP pair 14336x4096 + 4096x14336 v6 K1=K2=4096 (4 bits/weight)",
    "l70b": "70B-class pair 28672x8192 + 8192x28672 v8 K1=65536+K2=256 (3 bits/weight)",
    "aqlm4k": "4096x4096 v8 two additive books K1=K2=65536 (4 bits/weight)",
    "v16_4k": "4096x4096 v16 K1=65536+K2=256 (1.5 bits/weight)",
}
SVQ_WORKLOADS = {
    # affine-lattice layers: one 8-bit field of four 2-bit codes per 4-vector (2 bits/weight)
    "svq4k": ([(4096, 4096)], "f16"),
    "svq70b": ([(28672, 8192), (8192, 28672)], "bf16"),
}
SVQ_DESCRIBE = {
    "svq4k": "4096x4096 affine lattice d=4 (2 bits/weight)",
    "svq70b": "70B-class pair 28672x8192 + 8192x28672 affine lattice d=4 (2 bits/weight)",
}
GEMV_SOURCES = ["gemv_bit_unpack_amd/csrc/vq_gemv_bucket.hip", "gemv_bit_unpack_amd/csrc/vq_gemv_sliced.hip",
                "gemv_bit_unpack_amd/csrc/vq_device.h", "gemv_bit_unpack_amd/csrc/vq_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_vq_gemv_ws_bucketed_l70b_m1.json")
TRIALS = 5
HEADLINE_KEY = "l70b"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ byte and flop counts

def layer_bytes(vq, desc, m, y_bytes=2):
    """Algorithmic bytes of one call: packed indices + each codebook once + scale + x + y."""
    n, i, v = desc.out_features, desc.in_features, desc.v
    books = (1 << desc.bits1) * v * 2 + ((1 << desc.bits2) * v * 2 if desc.bits2 else 0)
    return vq.packed_bytes(desc) + books + 2 * n + 2 * m * i + y_bytes * m * n


def gathered_bytes(desc):
    """Centroid bytes gathered from books that are not staged in LDS (K > 4096)."""
    nv = (desc.in_features + desc.v - 1) // desc.v
    g = 0
    for bits in (desc.bits1, desc.bits2):
        if bits > 12:
            g += desc.out_features * nv * desc.v * 2
    return g


# ------------------------------------------------------------------ device rings

class Ring:
    """Distinct copies of one workload layer on the device, plus ctypes argument tuples."""

    def __init__(self, vq, torch, key, layer, m, copies=None, fn="vq_gemv_ws", y_dtype=None, shared_book=False,
                 layout=1):
        layers, v, b1, b2, xd = WORKLOADS[key]
        n, i = layers[layer]
        self.desc = vq.make_desc(n, i, v, b1, b2, layout)
        rs_desc = vq.make_desc(n, i, v, b1, b2)  # algorithmic bytes: the row stream's log2(K) bits per index
        self.m = m
        self.layout = layout
        dev = torch.device("cuda")
        per = layer_bytes(vq, self.desc, m)
        self.copies = copies or min(MAX_COPIES, max(1, -(-RING_BYTES // per)))
        g = torch.Generator(device=dev)
        g.manual_seed(zlib.crc32(("%d/%s/%d" % (42, key, layer)).encode()))
        nb = vq.packed_bytes(self.desc)
        bucketed = None
        if layout == vq.LAYOUT_BUCKETED:
            # a valid bucketed buffer needs real indices: pack seeded ones once on the host, and
            # give every copy its own device copy of it (the caches see distinct addresses)
            import numpy as np

            hr = np.random.default_rng(zlib.crc32(("%d/%s/%d/bucketed" % (42, key, layer)).encode()))
            nvec = (i + v - 1) // v
            idx1 = hr.integers(0, 1 << b1, (n, nvec), dtype=np.uint32)
            idx2 = hr.integers(0, 1 << b2, (n, nvec), dtype=np.uint32) if b2 else None
            bucketed = torch.from_numpy(vq.pack(self.desc, idx1, idx2)).to(dev)
        xdt = torch.bfloat16 if xd == "bf16" else torch.float16
        self.x = torch.randn((m, i), generator=g, device=dev, dtype=torch.float32).to(xdt)
        self.y_dtype = y_dtype or xdt
        self.items = []
        lib = vq.lib()
        self.fn = getattr(lib, fn)
        # one workspace for the whole ring: its calls run in order on one stream
        self.ws = None
        if fn == "vq_gemv_ws":
            self.ws = vq.workspace(self.desc, m, xdt, dev)
        elif fn == "vq_gemm_ws":
            self.ws = vq.gemm_workspace(self.desc, m, xdt, dev)
        self.sliced = fn == "vq_gemv_ws" and self.ws is not None
        extra = ()
        if fn in ("vq_gemv_ws", "vq_gemm_ws"):
            extra = (None, 0) if self.ws is None else (ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel())
        code = {torch.float16: vq.VQ_F16, torch.bfloat16: vq.VQ_BF16, torch.float32: vq.VQ_F32}
        self.tensors = []
        for c in range(self.copies):
            if bucketed is not None:
                packed = bucketed.clone()
            else:
                packed = torch.randint(0, 256, (nb,), generator=g, device=dev, dtype=torch.uint8)
            if shared_book and c > 0:
                cb1, cb2 = self.tensors[0][1], self.tensors[0][2]
            else:
                cb1 = (torch.randn((1 << b1, v), generator=g, device=dev) * 0.02).half()
                cb2 = (torch.randn((1 << b2, v), generator=g, device=dev) * 0.005).half() if b2 else None
            scale = (torch.rand((n,), generator=g, device=dev) + 0.5).half()
            y = torch.empty((m, n), device=dev, dtype=self.y_dtype)
            self.tensors.append((packed, cb1, cb2, scale, y))
            p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
            self.items.append((ctypes.byref(self.desc), p(packed), p(cb1), p(cb2), p(scale), None, p(self.x),
                               code[xdt], m, p(y), code[self.y_dtype]) + extra)
        yb = 4 if self.y_dtype == torch.float32 else 2
        self.bytes_per_call = layer_bytes(vq, rs_desc, m, yb)
        self.stored_bytes_per_call = layer_bytes(vq, self.desc, m, yb)  # what the layout actually holds
        self.flops_per_call = 2.0 * m * n * i

    def call(self, k, stream_ptr):
        st = self.fn(*self.items[k % self.copies], stream_ptr)
        if st != 0:
            raise RuntimeError("%s failed with status %d" % (self.fn.__name__, st))


class SvqRing:
    """Distinct copies of an affine-lattice layer (own codes and A, B; shared x) for vq_svq_gemv."""

    def __init__(self, vq, torch, key, layer, m, copies=None, fn="vq_svq_gemv"):
        layers, xd = SVQ_WORKLOADS[key]
        n, i = layers[layer]
        self.desc = vq.svq_desc(n, i)
        self.m = m
        self.flops_per_call = 2 * m * n * i
        dev = torch.device("cuda")
        nb = vq.packed_bytes(self.desc)
        xdt = torch.bfloat16 if xd == "bf16" else torch.float16
        self.bytes_per_call = nb + 40 + 2 * m * i + 2 * m * n   # codes + A, B + x + y
        self.copies = copies or min(MAX_COPIES, max(1, -(-RING_BYTES // self.bytes_per_call)))
        g = torch.Generator(device=dev)
        g.manual_seed(zlib.crc32(("%d/%s/%d/svq" % (42, key, layer)).encode()))
        self.x = torch.randn((m, i), generator=g, device=dev, dtype=torch.float32).to(xdt)
        code = {torch.float16: vq.VQ_F16, torch.bfloat16: vq.VQ_BF16}
        self.name = fn
        self.fn = getattr(vq.lib(), fn)
        self.items, self.tensors = [], []
        p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        for _ in range(self.copies):
            packed = torch.randint(0, 256, (nb,), generator=g, device=dev, dtype=torch.uint8)
            a = (torch.randn((4, 4), generator=g, device=dev) * 0.018).half()
            b = (torch.randn((4,), generator=g, device=dev) * 0.03).half()
            y = torch.empty((m, n), device=dev, dtype=xdt)
            self.tensors.append((packed, a, b, y))
            self.items.append((ctypes.byref(self.desc), p(packed), p(a), p(b), None, None, p(self.x), code[xdt], m,
                               p(y), code[xdt]))
        self.sliced = False

    def call(self, k, stream_ptr):
        st = self.fn(*self.items[k % self.copies], stream_ptr)
        if st != 0:
            raise RuntimeError("%s failed with status %d" % (self.name, st))


def svq_leg(vq, torch, use_graph, steps=None):
    """vq_svq_gemv on the affine-lattice workloads: M = 1 on both, M = 16 on the 4096^2 layer."""
    out = {}
    for key, m in (("svq4k", 1), ("svq70b", 1), ("svq4k", 16), ("svq70b", 8)):
        rings = [SvqRing(vq, torch, key, li, m) for li in range(len(SVQ_WORKLOADS[key][0]))]
        n_steps = steps or max(400, 2 * sum(r.copies for r in rings))
        sec, calls, _, launch = time_ring(torch, rings, n_steps, 20, use_graph)
        b = sum(r.bytes_per_call for r in rings) / len(rings)
        out["%s_m%d" % (key, m)] = {
            "workload": SVQ_DESCRIBE[key] + ", M=%d" % m, "us_per_call": round(sec * 1e6, 3),
            "GBps": round(b / sec / 1e9, 1), "pct_hbm": round(100 * b / sec / 1e9 / HBM_PEAK_GBPS, 2),
            "bytes_per_call": int(b), "copies": rings[0].copies, "calls": calls, "launch": launch}
        del rings
        torch.cuda.empty_cache()
    # the matrix-core product: prefill batches, and M = 16 against the VALU kernel above
    for key, m in (("svq70b", 128), ("svq4k", 16), ("svq70b", 16)):
        rings = [SvqRing(vq, torch, key, li, m, copies=4, fn="vq_svq_gemm")
                 for li in range(len(SVQ_WORKLOADS[key][0]))]
        sec, calls, _, launch = time_ring(torch, rings, 40, 4, use_graph)
        fl = sum(r.flops_per_call for r in rings) / len(rings)
        b = sum(r.bytes_per_call for r in rings) / len(rings)
        out["%s_m%d_gemm" % (key, m)] = {
            "workload": SVQ_DESCRIBE[key] + ", M=%d, vq_svq_gemm" % m, "us_per_call": round(sec * 1e6, 3),
            "tflops": round(fl / sec / 1e12, 1), "pct_mfma_peak": round(100 * fl / sec / 1e12 / MFMA_F16_PEAK_TFLOPS, 2),
            "GBps": round(b / sec / 1e9, 1), "calls": calls, "launch": launch}
        del rings
        torch.cuda.empty_cache()
    return out


class RhtRing:
    """Distinct activation rows for vq_rht (fresh inputs per call, outputs in place of new buffers)."""

    def __init__(self, vq, torch, m, n, dtype, copies=64):
        dev = torch.device("cuda")
        g = torch.Generator(device=dev)
        g.manual_seed(zlib.crc32(("%d/rht/%d/%d" % (42, m, n)).encode()))
        self.copies = copies
        self.bytes_per_call = 2 * 2 * m * n + (n + 7) // 8
        self.fn = vq.lib().vq_rht
        code = vq.VQ_BF16 if dtype == torch.bfloat16 else vq.VQ_F16
        self.signs = torch.randint(0, 256, ((n + 7) // 8,), generator=g, device=dev, dtype=torch.uint8)
        self.tensors, self.items = [], []
        for _ in range(copies):
            x = torch.randn((m, n), generator=g, device=dev).to(dtype)
            y = torch.empty_like(x)
            self.tensors.append((x, y))
            self.items.append((m, n, ctypes.c_void_p(x.data_ptr()), code, ctypes.c_void_p(self.signs.data_ptr()), 0,
                               ctypes.c_void_p(y.data_ptr()), code))

    def call(self, k, stream_ptr):
        st = self.fn(*self.items[k % self.copies], stream_ptr)
        if st != 0:
            raise RuntimeError("vq_rht failed with status %d" % st)


def rht_leg(vq, torch, use_graph):
    """vq_rht at decode batches on the row lengths of the workloads."""
    out = {}
    for m, n in ((1, 4096), (1, 8192), (1, 14336), (1, 28672), (16, 4096)):
        ring = RhtRing(vq, torch, m, n, torch.bfloat16 if n in (8192, 28672) else torch.float16)
        sec, _, _, launch = time_ring(torch, [ring], 640, 20, use_graph)
        out["m%d_n%d" % (m, n)] = {"us_per_call": round(sec * 1e6, 3), "block": vq.rht_block(n),
                                   "GBps": round(ring.bytes_per_call / sec / 1e9, 1), "launch": launch}
        del ring
        torch.cuda.empty_cache()
    return out


class RhtProductRing:
    """A layer ring whose calls take the randomized Hadamard transform of x first: fused
    (vq_gemv_ws_rht / vq_gemm_ws_rht) or separate (vq_rht into a buffer, then vq_gemv_ws /
    vq_gemm_ws on it)."""

    def __init__(self, vq, torch, key, layer, m, gemm, fused):
        self.ring = Ring(vq, torch, key, layer, m, copies=6, fn="vq_gemm_ws" if gemm else "vq_gemv_ws")
        self.copies = self.ring.copies
        dev = torch.device("cuda")
        n_in = self.ring.desc.in_features
        g = torch.Generator(device=dev)
        g.manual_seed(zlib.crc32(("%d/rhtp/%s/%d" % (42, key, layer)).encode()))
        self.signs = torch.randint(0, 256, ((n_in + 7) // 8,), generator=g, device=dev, dtype=torch.uint8)
        sp = ctypes.c_void_p(self.signs.data_ptr())
        lib = vq.lib()
        self.fused = fused
        if fused:
            self.fn = lib.vq_gemm_ws_rht if gemm else lib.vq_gemv_ws_rht
            self.ws = torch.zeros(vq.rht_product_workspace_bytes(self.ring.desc, m, self.ring.x.dtype, gemm),
                                  dtype=torch.uint8, device=dev)
            wp = (ctypes.c_void_p(self.ws.data_ptr()), self.ws.numel())
            self.items = [it[:9] + (sp,) + it[9:11] + wp for it in self.ring.items]
        else:
            self.fn = self.ring.fn
            self.xt = torch.empty_like(self.ring.x)
            xtp = ctypes.c_void_p(self.xt.data_ptr())
            self.items = [it[:6] + (xtp,) + it[7:] for it in self.ring.items]
            self.rht_args = (m, n_in, self.ring.items[0][6], self.ring.items[0][7], sp, 0, xtp, self.ring.items[0][7])
            self.rht = lib.vq_rht

    def call(self, k, stream_ptr):
        if not self.fused:
            st = self.rht(*self.rht_args, stream_ptr)
            if st != 0:
                raise RuntimeError("vq_rht failed with status %d" % st)
        st = self.fn(*self.items[k % self.copies], stream_ptr)
        if st != 0:
            raise RuntimeError("%s failed with status %d" % (self.fn.__name__, st))


def rht_fused_leg(vq, torch, use_graph):
    """The 70B-class pair with the input transform: fused into the x pass against vq_rht
    followed by the workspace product, per call (average of the two layers)."""
    out = {}
    for m, gemm in ((1, False), (8, False), (128, True)):
        entry = {}
        for fused in (True, False):
            rings = [RhtProductRing(vq, torch, "l70b", li, m, gemm, fused) for li in (0, 1)]
            sec, _, _, launch = time_ring(torch, rings, 240 if m < 128 else 48, 6, use_graph)
            entry["fused_us_per_call" if fused else "separate_us_per_call"] = round(sec * 1e6, 3)
            entry["launch"] = launch
            del rings
            torch.cuda.empty_cache()
        out["l70b_m%d_%s" % (m, "vq_gemm_ws_rht" if gemm else "vq_gemv_ws_rht")] = entry
    return out


FP64_PEAK_TFLOPS = 78.6  # MI355X vector fp64 (FMA = 2 flops)


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix


def encode_leg(vq, torch, calls=5):
    """vq_assign on a 4096 x 4096 layer, v = 8, K1 = 65536 + K2 = 256 (the books of the
    3-bit layer): main book = fp16 copies of W's vectors at random positions, residual book
    0.005 N(0,1), as the seeded generators draw them.  fp16 weights take the matrix-core
    main stage; the same weights in bf16 take the fp64 walk (timed with fewer calls)."""
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(zlib.crc32(b"42/encode/4096/4096"))
    n, inf, v, b1, b2 = 4096, 4096, 8, 16, 8
    w = (torch.randn((n, inf), generator=g, device=dev) * 0.02).to(torch.float16)
    pick = torch.randperm(n * inf // v, generator=g, device=dev)[: 1 << b1]
    cb1 = w.view(-1, v)[pick].contiguous()
    cb2 = (torch.randn((1 << b2, v), generator=g, device=dev) * 0.005).to(torch.float16)
    d = vq.make_desc(n, inf, v, b1, b2)
    ws = torch.empty(vq.assign_workspace_bytes(d), dtype=torch.uint8, device=dev)
    i1 = torch.empty((n, inf // v), dtype=torch.int32, device=dev)
    i2 = torch.empty_like(i1)
    stream = torch.cuda.current_stream()

    def timed(wt, k):
        vq.assign(d, wt, cb1, cb2, ws=ws, out1=i1, out2=i2)  # warm-up
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(k):
            vq.assign(d, wt, cb1, cb2, ws=ws, out1=i1, out2=i2)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1e-3 / k

    sec = timed(w, calls)
    sec64 = timed(w.to(torch.bfloat16), 2)
    nvec = n * inf // v
    dists = nvec * ((1 << b1) + (1 << b2))
    mfma_flops = nvec * (1 << b1) * 2 * v  # the products the distances need (K = v of the 16 slots)
    fp64_flops = dists * (2 * v + 2)
    return {"workload": "4096x4096 W, v=8, K1=65536 + K2=256", "ms_per_call": round(sec * 1e3, 3),
            "vectors_per_s": round(nvec / sec), "weights_per_s": round(n * inf / sec),
            "distances_per_s": round(dists / sec),
            "mfma_tflops": round(mfma_flops / sec / 1e12, 1),
            "pct_mfma_f16_peak": round(100 * mfma_flops / sec / 1e12 / MFMA_F16_PEAK_TFLOPS, 1),
            "fp64_walk_ms_per_call": round(sec64 * 1e3, 3),
            "fp64_walk_tflops": round(fp64_flops / sec64 / 1e12, 2),
            "fp64_walk_pct_fp64_peak": round(100 * fp64_flops / sec64 / 1e12 / FP64_PEAK_TFLOPS, 1),
            "calls": calls}


def time_ring(torch, rings, steps, warmup, use_graph=True):
    """Average seconds per call over `steps` calls rotating through the ring(s)."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    seq = [(r, k) for k in range(max(r.copies for r in rings)) for r in rings]
    for s in range(max(warmup, 1)):
        r, k = seq[s % len(seq)]
        r.call(k, sp)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            # warm up on the capture stream too
            ssp = ctypes.c_void_p(side.cuda_stream)
            for r, k in seq[:2]:
                r.call(k, ssp)
            side.synchronize()
            with torch.cuda.graph(graph, stream=side):
                gsp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for r, k in seq:
                    r.call(k, gsp)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: time eager launches
            log("graph capture failed (%s); timing eager launches" % e)
            graph = None
    reps = max(1, -(-steps // len(seq)))
    n_calls = reps * len(seq) if graph is not None else steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    if graph is not None:
        for _ in range(reps):
            graph.replay()
    else:
        for s in range(steps):
            r, k = seq[s % len(seq)]
            r.call(k, sp)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = start.elapsed_time(end) * 1e-3
    return gpu_s / n_calls, n_calls, wall, ("hipgraph" if graph is not None else "eager")


# ------------------------------------------------------------------ exact-step timing

def time_steps(torch, rings, steps, warmup, trials=TRIALS):
    """Time exactly `steps` steps, one call per ring per step (ring copy = step mod copies).

    `warmup` eager steps first; the `steps` steps are then captured in one HIP graph,
    replayed once untimed, and replayed `trials` times, each between two device
    synchronisations and timed with events on the replay stream.  Returns per-step seconds
    for every trial."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    for k in range(warmup):
        for r in rings:
            r.call(k, sp)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    ssp = ctypes.c_void_p(side.cuda_stream)
    for r in rings:  # warm-up on the capture stream too
        r.call(0, ssp)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        gsp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for k in range(steps):
            for r in rings:
                r.call(k, gsp)
    torch.cuda.synchronize()
    graph.replay()  # untimed: uploads the graph
    torch.cuda.synchronize()
    out = []
    for _ in range(trials):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        out.append(start.elapsed_time(end) * 1e-3 / steps)
    del graph
    return out


def cold_call_us(torch, ring, reps=5):
    """One call after streaming a 1 GiB buffer through the caches (L2 and Infinity Cache
    flushed of the layer), timed with events; median over `reps` different copies."""
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for k in range(reps):
        flush.add_(1.0)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        ring.call(k, sp)
        end.record(stream)
        torch.cuda.synchronize()
        times.append(start.elapsed_time(end) * 1e3)
    del flush
    return round(sorted(times)[len(times) // 2], 3)


def stream_ceiling_gbps():
    """HBM streaming-read rate measured by the ceiling microbenchmark (a separate process)."""
    import subprocess

    exe = os.path.join(ROOT, "gemv_bit_unpack_amd", "micro", "vq_ceilings")
    try:
        r = subprocess.run([exe, "--stream"], capture_output=True, text=True, timeout=120)
        return float(json.loads(r.stdout)["stream_read_GBps"])
    except Exception as e:  # the ratio is reported only when the measurement ran
        log("stream ceiling not measured: %s" % e)
        return None


# ------------------------------------------------------------------ CPU baseline

CPU_CONFIGS = [("tiny", 1), ("dec4k", 1), ("dec4k_res", 1), ("mlp8b", 1), ("l70b", 1)]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(budget_s=30.0):
    """The oracle (bit-by-bit unpack + fp32 dequant + fp64 product) on all host cores, on
    every workload at M = 1 (both layers of a pair): wall-clock median of 3 per workload.
    Workloads are taken smallest first and stop once `budget_s` of timed work has run."""
    import numpy as np

    import oracle
    import synth

    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    per, spent = {}, 0.0
    for key, m in CPU_CONFIGS:
        w = synth.WORKLOADS[key]
        layers = []
        for li, (n, i) in enumerate(w.layers):
            lay = synth.workload_layer(key, li)
            packed = oracle.pack(n, i, w.v, w.bits1, w.bits2, lay["idx1"], lay["idx2"])
            layers.append((lay, packed, synth.workload_x(key, li, m)))
        t_runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            for lay, packed, xb in layers:
                oracle.forward(lay["n"], lay["in_features"], w.v, w.bits1, w.bits2, packed, lay["cb1"], lay["cb2"],
                               lay["scale"], None, xb, w.x_dtype == "bf16", m, nthreads=threads)
            t_runs.append(time.perf_counter() - t0)
        t = sorted(t_runs)[1]
        spent += sum(t_runs)
        nbytes = sum(packed.size + ((1 << w.bits1) + ((1 << w.bits2) if w.bits2 else 0)) * w.v * 2
                     + 2 * lay["n"] + 2 * m * lay["in_features"] + 2 * m * lay["n"] for lay, packed, _ in layers)
        per[key] = {"ms_per_step": round(t * 1e3, 3), "GBps": round(nbytes / t / 1e9, 4), "layers": len(layers)}
        del layers
        if spent > budget_s:
            break
    head = per.get(HEADLINE_KEY)
    return {"value": head["GBps"] if head else None, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": "one copy of each workload's layer(s) at M = 1, the whole layer (bit-by-bit unpack, fp32 "
                      "dequant, fp64 product over all rows), wall-clock median of 3 on %d threads; value = the "
                      "70B-class pair, the headline workload, on the same algorithmic bytes" % threads,
            "per_workload": per}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps (layer pairs) per trial")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--only-headline", action="store_true", help="skip the GEMM, per-workload and CPU legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-gemm", action="store_true", help="run only the M=128 prefill GEMM leg (for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--ceilings", action="store_true",
                    help="run only the hardware-ceiling microbenchmark (stream read, global and LDS gathers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy (known bytes) to scale rocprofv3 counters")
    ap.add_argument("--shared-book", action="store_true",
                    help="diagnostic: every ring copy shares one codebook (warm in L2), headline only")
    ap.add_argument("--only-rht", action="store_true", help="run only the Hadamard-transform leg (for profiling)")
    ap.add_argument("--only-encode", action="store_true", help="run only the residual VQ encode leg (for profiling)")
    ap.add_argument("--only-svq", action="store_true",
                    help="run only the affine-lattice (vq_svq_gemv) leg (for profiling)")
    ap.add_argument("--m", type=int, default=1, help="batch rows for --only-workload (1..16)")
    ap.add_argument("--layout", type=int, default=1, choices=(1, 2),
                    help="packed layout for --only-workload: 1 row stream, 2 slice-bucketed (M = 1)")
    ap.add_argument("--only-workload", default=None, choices=sorted(WORKLOADS),
                    help="run only one workload's M=1 leg through vq_gemv_ws (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.ceilings:
        import subprocess

        exe = os.path.join(ROOT, "gemv_bit_unpack_amd", "micro", "vq_ceilings")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        sys.stderr.write(r.stderr)
        print(r.stdout.strip(), flush=True)
        sys.exit(r.returncode)

    import torch

    import gemv_bit_unpack_amd as vq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    vq.lib()
    use_graph = not args.no_graph
    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel(), "bytes_written": dst.numel(), "copies": 5}))
        return

    if args.only_gemm:
        res = {}
        for fn in ("vq_gemm_ws", "vq_gemm"):
            up = Ring(vq, torch, "l70b", 0, 128, copies=6, fn=fn)
            down = Ring(vq, torch, "l70b", 1, 128, copies=6, fn=fn)
            gsec, gcalls, _, glaunch = time_ring(torch, [up, down], args.steps, args.warmup, use_graph)
            flops = (up.flops_per_call + down.flops_per_call) / 2
            res[fn] = {"gemm_tflops": round(flops / gsec / 1e12, 2), "ms_per_call": round(gsec * 1e3, 4),
                       "calls": gcalls, "launch": glaunch}
            del up, down
            torch.cuda.empty_cache()
        print(json.dumps(res))
        return
    if args.only_rht:
        print(json.dumps({"rht": rht_leg(vq, torch, use_graph), "rht_fused": rht_fused_leg(vq, torch, use_graph)}))
        return
    if args.only_encode:
        print(json.dumps({"encode": encode_leg(vq, torch)}))
        return
    if args.only_svq:
        print(json.dumps({"affine_lattice": svq_leg(vq, torch, use_graph, steps=args.steps)}))
        return
    if args.only_workload:
        key = args.only_workload
        rings = [Ring(vq, torch, key, li, args.m, layout=args.layout) for li in range(len(WORKLOADS[key][0]))]
        sec, calls, _, launch = time_ring(torch, rings, args.steps, args.warmup, use_graph)
        b = sum(r.bytes_per_call for r in rings) / len(rings)
        kern = "slice-bucketed" if args.layout == 2 else (
            "codebook-sliced" if any(r.sliced for r in rings) else "gather")
        print(json.dumps({"workload": key, "m": args.m, "us_per_call": round(sec * 1e6, 3), "GBps": round(b / sec / 1e9, 1),
                          "kernel": kern, "calls": calls, "launch": launch}))
        return
    # Headline: vq_gemv_ws at M = 1 on the 70B-class pair (up, then down, per step), over the
    # slice-bucketed decode layout; the row-stream (codebook-sliced) call is timed beside it.
    stream_gbps = stream_ceiling_gbps()
    rs_up = Ring(vq, torch, HEADLINE_KEY, 0, 1, shared_book=args.shared_book)
    rs_down = Ring(vq, torch, HEADLINE_KEY, 1, 1, shared_book=args.shared_book)
    rs_steps = time_steps(torch, [rs_up, rs_down], args.steps, args.warmup)
    rs_sec = sorted(rs_steps)[len(rs_steps) // 2]
    rowstream = {"call": "vq_gemv_ws over the row-stream layout (codebook-sliced kernel)",
                 "ms_per_step": round(rs_sec * 1e3, 6),
                 "trials_ms_per_step": [round(t * 1e3, 6) for t in rs_steps],
                 "GBps": round((rs_up.bytes_per_call + rs_down.bytes_per_call) / rs_sec / 1e9, 2)}
    del rs_up, rs_down
    torch.cuda.empty_cache()
    up = Ring(vq, torch, HEADLINE_KEY, 0, 1, shared_book=args.shared_book, layout=vq.LAYOUT_BUCKETED)
    down = Ring(vq, torch, HEADLINE_KEY, 1, 1, shared_book=args.shared_book, layout=vq.LAYOUT_BUCKETED)
    rings = [up, down]
    log("headline: %d + %d copies of %s, %.2f MB per step" % (up.copies, down.copies, DESCRIBE[HEADLINE_KEY],
                                                           (up.bytes_per_call + down.bytes_per_call) / 1e6))
    t0 = time.perf_counter()
    per_step = time_steps(torch, rings, args.steps, args.warmup)
    wall = time.perf_counter() - t0
    sec = sorted(per_step)[len(per_step) // 2]
    step_bytes = up.bytes_per_call + down.bytes_per_call
    gbps = step_bytes / sec / 1e9
    nv = lambda r: (r.desc.in_features + 7) // 8
    gathers = sum(r.desc.out_features * nv(r) for r in rings)
    g_cb = (step_bytes + sum(gathered_bytes(r.desc) for r in rings)) / sec / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash(GEMV_SOURCES):
            traffic = tr.get("hbm_bytes_per_step")
    out = {
        "metric": "vq_gemv effective GB/s & % HBM peak at M=1; vq_gemm TFLOP/s at M=128",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV (vq_gemv_ws) over the 70B-class MLP layer pair, "
                               + DESCRIBE[HEADLINE_KEY] + ", M=1, bf16 x and y; one step = the up then the down layer",
                   "global_batch": 1, "layer_copies_in_ring": [up.copies, down.copies],
                   "launch": "hipgraph of exactly `steps` steps", "trials": TRIALS,
                   "bytes_per_step": step_bytes,
                   "stored_bytes_per_step": up.stored_bytes_per_call + down.stored_bytes_per_call,
                   "bytes_note": "value counts the row-stream bytes (16 + 8 bits per vector, 3 bits/weight); "
                                 "the slice-bucketed layout the call reads stores 32 bits per vector "
                                 "(stored_bytes_per_step)",
                   "path": "slice-bucketed"},
        "rowstream_codebook_sliced": rowstream,
        "trials_ms_per_step": [round(t * 1e3, 6) for t in per_step],
        "ms_per_step_min": round(min(per_step) * 1e3, 6),
        "value_at_min": round(step_bytes / min(per_step) / 1e9, 2),
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "pct_measured_stream_ceiling": round(100.0 * gbps / stream_gbps, 2) if stream_gbps else None,
        "measured_stream_ceiling_GBps": stream_gbps,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "vq_gemv_ws call over the slice-bucketed layout, timed whole: "
                               "gemv_bucket_kernel<true> (the dominant kernel, which also converts the bf16 x) "
                               "+ gemv_sliced_finalize",
                     "units": "algorithmic bytes of the pair per step / event-timed step"},
        "cold_single_call_us": {"up": cold_call_us(torch, up), "down": cold_call_us(torch, down),
                                "note": "one call after a 1 GiB buffer has been streamed through the caches"},
        "gather": {"gathers_per_s": round(gathers / sec, 1),
                   "effective_incl_gathered_centroids_GBps": round(g_cb, 2),
                   "note": "every 16-byte main-book centroid lookup counted once, from the 128 KiB LDS "
                           "slices"},
        "wall_s_timed": round(wall, 4),
    }
    del up, down, rings
    torch.cuda.empty_cache()
    if args.shared_book:
        out["config"]["diagnostic"] = "shared codebook across the ring (not the headline protocol)"
    if not args.only_headline and not args.shared_book:
        # Prefill GEMM at M = 128 on the 70B-class pair: vq_gemm_ws (the gather-fed matrix-core
        # product) and, for comparison, vq_gemm (LDS weight tiles, no workspace).
        gemm = {"workload": "prefill GEMM, " + DESCRIBE[HEADLINE_KEY] + ", M=128, bf16 x and y",
                "launch": "hipgraph, 8 steps (up + down) per trial"}
        for fn in ("vq_gemm_ws", "vq_gemm"):
            up = Ring(vq, torch, HEADLINE_KEY, 0, 128, copies=4, fn=fn)
            down = Ring(vq, torch, HEADLINE_KEY, 1, 128, copies=4, fn=fn)
            gt = time_steps(torch, [up, down], 8, 2)
            gsec = sorted(gt)[len(gt) // 2] / 2  # per layer call
            flops = (up.flops_per_call + down.flops_per_call) / 2
            tflops = flops / gsec / 1e12
            entry = {"tflops": round(tflops, 2), "frac_mfma_peak": round(tflops / MFMA_PEAK_TFLOPS, 4),
                     "ms_per_call": round(gsec * 1e3, 4), "trials_ms_per_call": [round(t * 500, 4) for t in gt]}
            if fn == "vq_gemm_ws":
                gemm.update(entry)
                gemm["call"] = fn
            else:
                gemm["vq_gemm"] = entry
            del up, down
            torch.cuda.empty_cache()
        out["gemm"] = gemm
        # GEMV / GEMM crossover on the same pair: vq_gemv_ws (M <= 16) against vq_gemm_ws.
        cross = {}
        for m in (1, 8, 16, 32):
            entry = {}
            for fn in ("vq_gemv_ws", "vq_gemm_ws"):
                if fn == "vq_gemv_ws" and m > 16:
                    entry[fn + "_us_per_call"] = None  # the GEMV takes M <= 16
                    continue
                rr = [Ring(vq, torch, HEADLINE_KEY, li, m, copies=6, fn=fn) for li in (0, 1)]
                tt = time_steps(torch, rr, 12, 2)
                entry[fn + "_us_per_call"] = round(sorted(tt)[len(tt) // 2] / 2 * 1e6, 3)
                del rr
                torch.cuda.empty_cache()
            if m == 1:  # the batch-1 decode product over the slice-bucketed layout
                rr = [Ring(vq, torch, HEADLINE_KEY, li, 1, copies=6, layout=vq.LAYOUT_BUCKETED) for li in (0, 1)]
                tt = time_steps(torch, rr, 12, 2)
                entry["vq_gemv_ws_bucketed_us_per_call"] = round(sorted(tt)[len(tt) // 2] / 2 * 1e6, 3)
                del rr
                torch.cuda.empty_cache()
            g_us, m_us = entry.get("vq_gemv_ws_us_per_call"), entry["vq_gemm_ws_us_per_call"]
            entry["faster"] = "vq_gemm_ws" if g_us is None or m_us < g_us else "vq_gemv_ws"
            cross["m%d" % m] = entry
        out["gemv_gemm_crossover_l70b"] = cross
        per = {}

        def measure(rings):
            s, _, _, _ = time_ring(torch, rings, max(200, 2 * sum(r.copies for r in rings)), 20, use_graph)
            b = sum(r.bytes_per_call for r in rings) / len(rings)
            bcb = sum(r.bytes_per_call + gathered_bytes(r.desc) for r in rings) / len(rings)
            return {"us_per_call": round(s * 1e6, 3), "GBps": round(b / s / 1e9, 1),
                    "pct_hbm": round(100 * b / s / 1e9 / HBM_PEAK_GBPS, 2),
                    "GBps_incl_gathered": round(bcb / s / 1e9, 1)}

        for key in WORKLOADS:
            n_layers = len(WORKLOADS[key][0])
            rings = [Ring(vq, torch, key, li, 1) for li in range(n_layers)]
            sliced = any(r.sliced for r in rings)
            entry = measure(rings)
            entry["kernel"] = "codebook-sliced" if sliced else "gather"
            del rings
            torch.cuda.empty_cache()
            if sliced:  # the same layers through vq_gemv (no workspace): the L2-gather kernel
                rings = [Ring(vq, torch, key, li, 1, fn="vq_gemv") for li in range(n_layers)]
                entry["gather_kernel_us_per_call"] = measure(rings)["us_per_call"]
                del rings
                torch.cuda.empty_cache()
            _, v_, b1_, b2_, _ = WORKLOADS[key]
            if v_ == 8 and b1_ == 16 and b2_ in (0, 8):  # the slice-bucketed decode layout
                rings = [Ring(vq, torch, key, li, 1, layout=vq.LAYOUT_BUCKETED) for li in range(n_layers)]
                bk = measure(rings)
                entry["bucketed_us_per_call"] = bk["us_per_call"]
                entry["bucketed_GBps"] = bk["GBps"]
                del rings
                torch.cuda.empty_cache()
            per[key] = entry
        out["gemv_m1_per_workload"] = per
        # Decode batches: the 65536-entry book (vq_gemv_ws against vq_gemv) and the v = 6
        # LDS books (vq_gemv: the matrix-core kernel at 2..16 rows).
        batch = {}
        for key, m in (("dec4k_res", 4), ("dec4k_res", 16), ("l70b", 8), ("mlp8b", 2), ("mlp8b", 4), ("mlp8b", 16)):
            n_layers = len(WORKLOADS[key][0])
            entry = {}
            for fn in (("vq_gemv",) if key == "mlp8b" else ("vq_gemv_ws", "vq_gemv")):
                rings = [Ring(vq, torch, key, li, m, fn=fn, copies=8) for li in range(n_layers)]
                s, _, _, _ = time_ring(torch, rings, 64, 8, use_graph)
                entry[fn + "_us_per_call"] = round(s * 1e6, 3)
                if fn == "vq_gemv_ws":
                    entry["kernel"] = "codebook-sliced" if any(r.sliced for r in rings) else "gather"
                elif key == "mlp8b":
                    entry["kernel"] = "v6 matrix-core"
                del rings
                torch.cuda.empty_cache()
            batch["%s_m%d" % (key, m)] = entry
        out["gemv_batched"] = batch
        out["affine_lattice"] = svq_leg(vq, torch, use_graph)
        out["rht"] = rht_leg(vq, torch, use_graph)
        out["rht_fused"] = rht_fused_leg(vq, torch, use_graph)
        out["encode"] = encode_leg(vq, torch)
    if not args.no_cpu_baseline and not args.shared_book and not args.only_headline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
