// vq_gemv: decode-batch product y[M][N] = x[M][IN] * W^T (+ bias), 1 <= M <= 16.
//
// The weight vectors are rebuilt on the fly, never stored (VPTQ guide, "Step 3: Fused
// Low-Bit VPTQ Linear Layer": one fused kernel per linear layer, indices read from
// device memory, looked up in an on-chip codebook, dot product in registers; the
// production-VQ post's "Dequantization Kernels and Inference Dynamics": small books in
// on-chip memory, K >= 65536 books served from L2).
//
// gfx950 mapping.  One wavefront owns one output row at a time and walks its index
// stream 64 vectors per step, lane l taking vector j0 + l, so the index words, the x
// slices and the output of a step are contiguous across the wavefront.  Per vector a
// lane unpacks its indices (one funnel shift), gathers the main centroid (LDS when
// K1 <= 4096, else global memory through L2/MALL: a 1 MiB book stays cache-resident),
// gathers the residual centroid from LDS, adds them in fp32 and multiply-accumulates
// with x in fp32.  At the end of the row the 64 partial sums are reduced across the
// wavefront and lane 0 applies the channel scale and bias.  Small codebooks are staged
// once per workgroup (16 B per centroid, v <= 8); workgroups are persistent and
// grid-stride over rows so the staging is amortised.
#include <mutex>

#include "vq_device.h"

namespace {

using vqi::ProductArgs;

constexpr int kUnroll = 4;  // vectors in flight per lane

// v halves of a centroid (fp16 bits) -> fp32.  Fast path for v = 6 and v = 8.
template <int V>
__device__ __forceinline__ void load_centroid_global(const uint16_t* __restrict__ cb, uint32_t k, float (&c)[V]) {
  if constexpr (V == 8) {
    const uint4 q = *(const uint4*)(cb + (size_t)k * 8);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = vqd::f16_to_f32(w[i]);
      c[2 * i + 1] = vqd::f16_to_f32(w[i] >> 16);
    }
  } else {
    static_assert(V == 6, "fast path covers v = 6 and v = 8");
    const uint32_t* p = (const uint32_t*)(cb + (size_t)k * 6);
    const uint32_t w[3] = {p[0], p[1], p[2]};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      c[2 * i] = vqd::f16_to_f32(w[i]);
      c[2 * i + 1] = vqd::f16_to_f32(w[i] >> 16);
    }
  }
}

template <int V>
__device__ __forceinline__ void load_centroid_lds(const uint4* lds, uint32_t k, float (&c)[V]) {
  const uint4 q = lds[k];
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < V; ++t) c[t] = vqd::f16_to_f32(w[t >> 1] >> (16 * (t & 1)));
}

// x[m][col0 .. col0 + V) as fp32; lanes past IN read as 0 without touching memory.
template <int V, int XT>
__device__ __forceinline__ void load_x(const uint16_t* __restrict__ xrow, int32_t col0, int32_t in_features,
                                       float (&xv)[V]) {
  if (col0 + V <= in_features) {
    uint32_t w[V / 2];
    if constexpr (V == 8) {
      const uint4 q = *(const uint4*)(xrow + col0);
      w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
    } else {
      const uint32_t* p = (const uint32_t*)(xrow + col0);
#pragma unroll
      for (int i = 0; i < V / 2; ++i) w[i] = p[i];
    }
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      xv[2 * i] = vqd::x_to_f32<XT>(w[i] & 0xFFFFu);
      xv[2 * i + 1] = vqd::x_to_f32<XT>(w[i] >> 16);
    }
  } else {
#pragma unroll
    for (int t = 0; t < V; ++t) xv[t] = (col0 + t < in_features) ? vqd::x_to_f32<XT>(xrow[col0 + t]) : 0.0f;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, vqd::kWave);
  return v;
}

// Fast path: v in {6, 8}, books staged as 16-byte LDS entries when small.
template <int V, int MT, int XT, bool RES>
__global__ __launch_bounds__(1024) void gemv_kernel(ProductArgs a, int lds1, int lds2) {
  extern __shared__ uint4 lds_books[];
  const uint4* book1 = lds_books;
  const uint4* book2 = lds_books + (lds1 ? (1 << a.bits1) : 0);
  // Stage small codebooks: entry k = v halves padded to 16 bytes.
  {
    const int k1 = lds1 ? (1 << a.bits1) : 0;
    const int k2 = (RES && lds2) ? (1 << a.bits2) : 0;
    for (int e = threadIdx.x; e < k1 + k2; e += blockDim.x) {
      const uint16_t* src = e < k1 ? a.cb1 + (size_t)e * V : a.cb2 + (size_t)(e - k1) * V;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < V / 2; ++i) w[i] = ((const uint32_t*)src)[i];
      lds_books[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    __syncthreads();
  }
  const int lane = threadIdx.x & (vqd::kWave - 1);
  const int waves_per_block = blockDim.x / vqd::kWave;
  const int wave = blockIdx.x * waves_per_block + (threadIdx.x / vqd::kWave);
  const int total_waves = gridDim.x * waves_per_block;
  const int m_count = a.m;
  for (int row = wave; row < a.n; row += total_waves) {
    const uint32_t* r1 = a.packed1 + (size_t)row * a.s1_words;
    const uint32_t* r2 = RES ? a.packed2 + (size_t)row * a.s2_words : nullptr;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    for (int j0 = 0; j0 < a.nv; j0 += vqd::kWave * kUnroll) {
      uint32_t i1[kUnroll], i2[kUnroll];
      bool live[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t j = (uint32_t)(j0 + u * vqd::kWave + lane);
        live[u] = (int)j < a.nv;
        i1[u] = live[u] ? vqd::extract_index(r1, a.s1_words, j, a.bits1) : 0u;
        if constexpr (RES) i2[u] = live[u] ? vqd::extract_index(r2, a.s2_words, j, a.bits2) : 0u;
      }
      float w[kUnroll][V];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (lds1) {
          load_centroid_lds<V>(book1, i1[u], w[u]);
        } else {
          load_centroid_global<V>(a.cb1, i1[u], w[u]);
        }
        if constexpr (RES) {
          float c2[V];
          if (lds2) {
            load_centroid_lds<V>(book2, i2[u], c2);
          } else {
            load_centroid_global<V>(a.cb2, i2[u], c2);
          }
#pragma unroll
          for (int t = 0; t < V; ++t) w[u][t] = w[u][t] + c2[t];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (!live[u]) continue;
        const int32_t col0 = (j0 + u * vqd::kWave + lane) * V;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < m_count) {
            float xv[V];
            load_x<V, XT>(a.x + (size_t)m * a.in_features, col0, a.in_features, xv);
#pragma unroll
            for (int t = 0; t < V; ++t) acc[m] = __builtin_fmaf(xv[t], w[u][t], acc[m]);
          }
        }
      }
    }
    const float s = a.scale ? vqd::f16_to_f32(a.scale[row]) : 1.0f;
    const float b = a.bias ? vqd::f16_to_f32(a.bias[row]) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < m_count) {
        float r = wave_sum(acc[m]);
        if (lane == 0) {
          if (a.scale) r = r * s;
          if (a.bias) r = r + b;
          vqd::store_out(a.y, (size_t)m * a.n + row, r, a.y_dtype);
        }
      }
    }
  }
}

// Generic path: any v in 1..16, centroids and x read element by element from global
// memory.  Used for shapes the fast path does not cover (and for test layouts).
template <int XT>
__global__ __launch_bounds__(256) void gemv_generic_kernel(ProductArgs a) {
  const int lane = threadIdx.x & (vqd::kWave - 1);
  const int waves_per_block = blockDim.x / vqd::kWave;
  const int wave = blockIdx.x * waves_per_block + (threadIdx.x / vqd::kWave);
  const int total_waves = gridDim.x * waves_per_block;
  for (int row = wave; row < a.n; row += total_waves) {
    const uint32_t* r1 = a.packed1 + (size_t)row * a.s1_words;
    const uint32_t* r2 = a.bits2 ? a.packed2 + (size_t)row * a.s2_words : nullptr;
    float acc[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
    for (int j = lane; j < a.nv; j += vqd::kWave) {
      const uint32_t i1 = vqd::extract_index(r1, a.s1_words, (uint32_t)j, a.bits1);
      const uint32_t i2 = a.bits2 ? vqd::extract_index(r2, a.s2_words, (uint32_t)j, a.bits2) : 0u;
      const int32_t col0 = j * a.v;
      const int32_t nt = min(a.v, a.in_features - col0);
      for (int t = 0; t < nt; ++t) {
        float w = vqd::f16_to_f32(a.cb1[(size_t)i1 * a.v + t]);
        if (a.bits2) w = w + vqd::f16_to_f32(a.cb2[(size_t)i2 * a.v + t]);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (m < a.m) acc[m] = __builtin_fmaf(vqd::x_to_f32<XT>(a.x[(size_t)m * a.in_features + col0 + t]), w, acc[m]);
        }
      }
    }
    const float s = a.scale ? vqd::f16_to_f32(a.scale[row]) : 1.0f;
    const float b = a.bias ? vqd::f16_to_f32(a.bias[row]) : 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if (m < a.m) {
        float r = wave_sum(acc[m]);
        if (lane == 0) {
          if (a.scale) r = r * s;
          if (a.bias) r = r + b;
          vqd::store_out(a.y, (size_t)m * a.n + row, r, a.y_dtype);
        }
      }
    }
  }
}

constexpr int kNumCU = 256;

template <int V, int MT, int XT, bool RES>
vq_status launch_fast(const ProductArgs& a, hipStream_t s) {
  const int lds1 = a.bits1 <= 12 ? 1 : 0;
  const int lds2 = (RES && a.bits2 <= 12) ? 1 : 0;
  const size_t lds_bytes = 16u * ((lds1 ? (1u << a.bits1) : 0u) + (lds2 ? (1u << a.bits2) : 0u));
  auto kern = gemv_kernel<V, MT, XT, RES>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return VQ_ERR_HIP;
  // Big LDS footprint: one 1024-thread workgroup per CU; otherwise 256-thread groups.
  const int block = lds_bytes > 32 * 1024 ? 1024 : 256;
  const int per_cu = lds_bytes > 32 * 1024 ? 1 : (lds_bytes > 0 ? 8 : 8);
  const int waves_per_block = block / vqd::kWave;
  const long want = (a.n + waves_per_block - 1) / waves_per_block;
  const long cap = (long)kNumCU * per_cu;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds_bytes, s, a, lds1, lds2);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int V, int XT, bool RES>
vq_status dispatch_m(const ProductArgs& a, hipStream_t s) {
  if (a.m <= 1) return launch_fast<V, 1, XT, RES>(a, s);
  if (a.m <= 2) return launch_fast<V, 2, XT, RES>(a, s);
  if (a.m <= 4) return launch_fast<V, 4, XT, RES>(a, s);
  if (a.m <= 8) return launch_fast<V, 8, XT, RES>(a, s);
  return launch_fast<V, 16, XT, RES>(a, s);
}

template <int V, int XT>
vq_status dispatch_res(const ProductArgs& a, hipStream_t s) {
  return a.bits2 ? dispatch_m<V, XT, true>(a, s) : dispatch_m<V, XT, false>(a, s);
}

template <int V>
vq_status dispatch_x(const ProductArgs& a, hipStream_t s) {
  return a.x_dtype == VQ_BF16 ? dispatch_res<V, 1>(a, s) : dispatch_res<V, 0>(a, s);
}

}  // namespace

namespace vqi {

vq_status launch_gemv(const ProductArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // The fast path needs vector-aligned codebooks and x rows.
  const size_t vb = (size_t)a.v * 2;
  const size_t align = (a.v == 8) ? 16 : 4;
  const bool fast_shape = (a.v == 8 || a.v == 6);
  const bool fast_align = aligned(a.cb1, align) && (!a.cb2 || aligned(a.cb2, align)) && aligned(a.x, align) &&
                          (((size_t)a.in_features * 2) % align == 0);
  (void)vb;
  if (a.in_features > 0 && fast_shape && fast_align) {
    return a.v == 8 ? dispatch_x<8>(a, s) : dispatch_x<6>(a, s);
  }
  const int block = 256;
  const long want = (a.n + 3) / 4;
  const long cap = (long)kNumCU * 8;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  if (a.x_dtype == VQ_BF16) {
    hipLaunchKernelGGL(gemv_generic_kernel<1>, dim3(grid), dim3(block), 0, s, a);
  } else {
    hipLaunchKernelGGL(gemv_generic_kernel<0>, dim3(grid), dim3(block), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
