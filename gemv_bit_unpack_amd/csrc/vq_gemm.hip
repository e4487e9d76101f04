// vq_gemm: prefill-batch product y[M][N] = x[M][IN] * W^T (+ bias) on the matrix cores.
//
// At large batches the product is a dense contraction: the tensor-core formats win
// there (production-VQ post, "Prefill vs. Decode Bottlenecks" and "Throughput and
// Concurrency Trade-Offs"), so here the rebuilt weights are fed to MFMA instead of the
// VALU.  Each workgroup owns 32 output rows and the whole batch chunk (up to 256 rows
// of x), so every weight vector is gathered and rebuilt exactly once per call.  Per
// K-tile (8 or 16 vectors per row):
//   1. every thread rebuilds its vector slot(s): unpack the indices, gather the main
//      centroid (LDS when it fits, else global memory through L2), gather the
//      residual centroid, add in fp32, and write the sum to the LDS weight tile in the
//      activation's 16-bit type.  bf16 activations get a hi + lo pair of bf16 tiles
//      (hi = RNE(w), lo = RNE(w - hi)), which carries ~16 significant bits of w;
//   2. the x tile [chunk rows][K-tile] is copied to LDS;
//   3. each wavefront runs v_mfma_f32_32x32x16 over its 32-row batch blocks: A = the
//      32 x 16 weight fragment (eight consecutive k of one output row per lane),
//      B = the matching x fragment, fp32 accumulators in registers.
// The channel scale and bias are applied once per output in the epilogue.
// LDS rows are padded by 16 bytes so the fragment reads of a wavefront hit distinct banks.
#include <mutex>

#include "vq_device.h"

namespace {

using vqi::ProductArgs;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 32;       // output rows per workgroup
constexpr int kThreads = 256;  // 4 wavefronts

struct GemmCfg {
  int32_t vpt;     // vectors per row per K-tile
  int32_t bk;      // K-tile width in columns (v * vpt, a multiple of 16)
  int32_t ld;      // LDS row stride of the tiles, in halves (bk + 8)
  int32_t lds1;    // main book staged in LDS
  int32_t lds2;    // residual book staged in LDS
  int32_t x_vec;   // x rows allow 16-byte loads
  int32_t book_off;  // byte offset of the staged books in LDS
};

// Centroid k (fp16 bits) of a book with V halves per entry -> fp32.  V == 0: runtime v.
template <int V>
__device__ __forceinline__ void gather_centroid(const uint16_t* __restrict__ book, uint32_t k, int v, float* c) {
  if constexpr (V == 8) {
    const uint4 q = *(const uint4*)(book + (size_t)k * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = vqd::f16_to_f32(w[i]);
      c[2 * i + 1] = vqd::f16_to_f32(w[i] >> 16);
    }
  } else if constexpr (V == 6) {
    const uint32_t* p = (const uint32_t*)(book + (size_t)k * 6);
    const uint32_t w[3] = {p[0], p[1], p[2]};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      c[2 * i] = vqd::f16_to_f32(w[i]);
      c[2 * i + 1] = vqd::f16_to_f32(w[i] >> 16);
    }
  } else {
    for (int t = 0; t < v; ++t) c[t] = vqd::f16_to_f32(book[(size_t)k * v + t]);
  }
}

template <int V, int MB, int XT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(ProductArgs a, GemmCfg g) {
  constexpr int kMaxV = V == 0 ? 16 : V;
  constexpr int kTiles = XT == 1 ? 2 : 1;          // bf16: hi + lo weight tiles
  constexpr int kAcc = (MB + 3) / 4;               // batch blocks per wavefront
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* wt = smem;                             // [kTiles][kBN][ld]
  uint16_t* xt = smem + kTiles * kBN * g.ld;       // [32*MB][ld]
  const uint16_t* book1 = a.cb1;
  const uint16_t* book2 = a.cb2;
  const int v = V == 0 ? a.v : V;
  {
    uint16_t* lb = (uint16_t*)((uint8_t*)smem + g.book_off);
    const int n1 = g.lds1 ? (v << a.bits1) : 0;
    const int n2 = g.lds2 ? (v << a.bits2) : 0;
    for (int e = threadIdx.x; e < n1; e += kThreads) lb[e] = a.cb1[e];
    uint16_t* lb2 = lb + ((n1 + 7) & ~7);
    for (int e = threadIdx.x; e < n2; e += kThreads) lb2[e] = a.cb2[e];
    if (g.lds1) book1 = lb;
    if (g.lds2) book2 = lb2;
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * kBN;
  const int slots = kBN * g.vpt;

  float16_t acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  for (int k0 = 0; k0 < a.in_features; k0 += g.bk) {
    const int j0 = k0 / v;
    // 1. rebuild the weight tile
    for (int slot = threadIdx.x; slot < slots; slot += kThreads) {
      const int r = slot / g.vpt;
      const int jl = slot - r * g.vpt;
      const int row = row0 + r;
      const int j = j0 + jl;
      float c[kMaxV];
      const bool live = row < a.n && j < a.nv;
      if (live) {
        const uint32_t i1 = vqd::extract_index(a.packed1 + (size_t)row * a.s1_words, a.s1_words, (uint32_t)j, a.bits1);
        gather_centroid<V>(book1, i1, v, c);
        if (a.bits2) {
          const uint32_t i2 =
              vqd::extract_index(a.packed2 + (size_t)row * a.s2_words, a.s2_words, (uint32_t)j, a.bits2);
          float c2[kMaxV];
          gather_centroid<V>(book2, i2, v, c2);
#pragma unroll
          for (int t = 0; t < kMaxV; ++t)
            if (t < v) c[t] = c[t] + c2[t];
        }
      }
#pragma unroll
      for (int t = 0; t < kMaxV; ++t) {
        if (t < v) {
          const int col = jl * v + t;
          const float w = (live && k0 + col < a.in_features) ? c[t] : 0.0f;
          if constexpr (XT == 0) {
            wt[r * g.ld + col] = vqd::f32_to_f16_rne(w);
          } else {
            const uint16_t hi = vqd::f32_to_bf16_rne(w);
            const float rest = w - vqd::bf16_to_f32(hi);
            wt[r * g.ld + col] = hi;
            wt[kBN * g.ld + r * g.ld + col] = vqd::f32_to_bf16_rne(rest);
          }
        }
      }
    }
    // 2. x tile [32*MB][bk], zero outside [M, IN)
    {
      const int chunks = 32 * MB * (g.bk / 8);
      for (int ch = threadIdx.x; ch < chunks; ch += kThreads) {
        const int m = ch / (g.bk / 8);
        const int c8 = ch - m * (g.bk / 8);
        const int k = k0 + c8 * 8;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (m < a.m) {
          const uint16_t* xr = a.x + (size_t)m * a.in_features;
          if (g.x_vec && k + 8 <= a.in_features) {
            q = *(const uint4*)(xr + k);
          } else {
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (k + e < a.in_features) ? xr[k + e] : (uint16_t)0;
            q.x = h[0] | ((uint32_t)h[1] << 16);
            q.y = h[2] | ((uint32_t)h[3] << 16);
            q.z = h[4] | ((uint32_t)h[5] << 16);
            q.w = h[6] | ((uint32_t)h[7] << 16);
          }
        }
        *(uint4*)(xt + m * g.ld + c8 * 8) = q;
      }
    }
    __syncthreads();
    // 3. MFMA over the tile
    const int ar = lane & 31;
    const int kh = (lane >> 5) * 8;
    for (int ks = 0; ks < g.bk; ks += 16) {
      const uint4 aw = *(const uint4*)(wt + ar * g.ld + ks + kh);
      uint4 aw_lo = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (XT == 1) aw_lo = *(const uint4*)(wt + kBN * g.ld + ar * g.ld + ks + kh);
#pragma unroll
      for (int i = 0; i < kAcc; ++i) {
        const int mb = wave + 4 * i;
        if (mb < MB) {
          const uint4 bw = *(const uint4*)(xt + (mb * 32 + ar) * g.ld + ks + kh);
          if constexpr (XT == 0) {
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, aw),
                                                            __builtin_bit_cast(half8_t, bw), acc[i], 0, 0, 0);
          } else {
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                             __builtin_bit_cast(bf16x8_t, bw), acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, aw_lo),
                                                             __builtin_bit_cast(bf16x8_t, bw), acc[i], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }
  // Epilogue: accumulator register r of lane l holds output row 8*(r/4) + 4*(l/32) + r%4
  // of the wavefront's 32 and batch row l%32 of the block.
#pragma unroll
  for (int i = 0; i < kAcc; ++i) {
    const int mb = wave + 4 * i;
    if (mb >= MB) continue;
    const int m = mb * 32 + (lane & 31);
    if (m >= a.m) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = row0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (n < a.n) {
        float out = acc[i][r];
        if (a.scale) out = out * vqd::f16_to_f32(a.scale[n]);
        if (a.bias) out = out + vqd::f16_to_f32(a.bias[n]);
        vqd::store_out(a.y, (size_t)m * a.n + n, out, a.y_dtype);
      }
    }
  }
}

template <int V, int MB, int XT>
vq_status launch_one(const ProductArgs& a, const GemmCfg& g, size_t lds, hipStream_t s) {
  auto kern = gemm_kernel<V, MB, XT>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return VQ_ERR_HIP;
  const unsigned grid = (unsigned)((a.n + kBN - 1) / kBN);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, s, a, g);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int V, int XT>
vq_status dispatch_mb(const ProductArgs& a, const GemmCfg& g, int mb, size_t lds, hipStream_t s) {
  if (mb <= 1) return launch_one<V, 1, XT>(a, g, lds, s);
  if (mb <= 2) return launch_one<V, 2, XT>(a, g, lds, s);
  if (mb <= 4) return launch_one<V, 4, XT>(a, g, lds, s);
  return launch_one<V, 8, XT>(a, g, lds, s);
}

template <int V>
vq_status dispatch_xt(const ProductArgs& a, const GemmCfg& g, int mb, size_t lds, hipStream_t s) {
  return a.x_dtype == VQ_BF16 ? dispatch_mb<V, 1>(a, g, mb, lds, s) : dispatch_mb<V, 0>(a, g, mb, lds, s);
}

constexpr size_t kLdsMax = 160 * 1024;

}  // namespace

namespace vqi {

vq_status launch_gemm(const ProductArgs& a0, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a0.in_features == 0) {
    // y = bias (or 0): the kernel's K loop is empty and the epilogue writes it.
  }
  const int v = a0.v;
  GemmCfg g;
  g.vpt = (v % 2 == 0) ? 8 : 16;
  g.bk = v * g.vpt;
  g.ld = g.bk + 8;
  const int fast_v = (v == 8 && aligned(a0.cb1, 16) && (!a0.cb2 || aligned(a0.cb2, 16)))   ? 8
                     : (v == 6 && aligned(a0.cb1, 4) && (!a0.cb2 || aligned(a0.cb2, 4))) ? 6
                                                                                          : 0;
  g.x_vec = (aligned(a0.x, 16) && a0.in_features % 8 == 0) ? 1 : 0;
  const int tiles = a0.x_dtype == VQ_BF16 ? 2 : 1;
  for (int32_t m0 = 0; m0 < a0.m; m0 += 256) {
    ProductArgs a = a0;
    a.m = a0.m - m0 < 256 ? a0.m - m0 : 256;
    a.x = a0.x + (size_t)m0 * a0.in_features;
    a.y = (uint8_t*)a0.y + (size_t)m0 * a0.n * (a0.y_dtype == VQ_F32 ? 4 : 2);
    const int mb = (a.m + 31) / 32;
    const int mb_pow = mb <= 1 ? 1 : mb <= 2 ? 2 : mb <= 4 ? 4 : 8;
    size_t lds = (size_t)(tiles * kBN + 32 * mb_pow) * g.ld * 2;
    lds = (lds + 15) & ~(size_t)15;
    g.book_off = (int32_t)lds;
    const size_t b1 = (size_t)v * ((size_t)1 << a.bits1) * 2;
    const size_t b2 = a.bits2 ? (size_t)v * ((size_t)1 << a.bits2) * 2 : 0;
    size_t used = lds;
    g.lds2 = (a.bits2 && used + ((b2 + 15) & ~(size_t)15) <= kLdsMax) ? 1 : 0;
    // the main book goes before the residual book in LDS
    g.lds1 = (used + ((b1 + 15) & ~(size_t)15) + (g.lds2 ? b2 : 0) <= kLdsMax && b1 <= 96 * 1024) ? 1 : 0;
    if (g.lds1) used += (b1 + 15) & ~(size_t)15;
    if (g.lds2) used += (b2 + 15) & ~(size_t)15;
    vq_status st;
    if (fast_v == 8) {
      st = dispatch_xt<8>(a, g, mb, used, s);
    } else if (fast_v == 6) {
      st = dispatch_xt<6>(a, g, mb, used, s);
    } else {
      st = dispatch_xt<0>(a, g, mb, used, s);
    }
    if (st != VQ_OK) return st;
  }
  return VQ_OK;
}

}  // namespace vqi
