// vq_assign: two-stage residual VQ encode with given codebooks (VPTQ guide, "Step 2:
// Multi-Stage Residual Vector Quantizer (RVQ)"; the distance and argmin of "1. Vector
// Quantization Fundamentals"; the residual of "2. Multi-Stage Residual Vector
// Quantization").  Each v-vector w of W takes
//
//   idx1 = the lowest k minimising |C1[k]|^2 - 2 w . C1[k]
//   idx2 = the lowest k minimising |C2[k]|^2 - 2 r . C2[k],   r = fp32(w - C1[idx1])
//
// which ranks centroids as the squared Euclidean distance does (|w|^2 is common to all).
// The ranking is evaluated in fp64 with one fused multiply-add per term, in ascending
// coordinate order: the products of fp16 centroids with fp16 / bf16 / fp32 weights are
// exact in fp64, and the index taken is the same on every conforming implementation of
// that sequence of operations.
//
// Kernels:
//   assign_table_kernel  one thread per centroid: the fp64 record {|c|^2, c_0 .. c_{v-1}}
//                        of each fp16 centroid into the workspace.
//   assign_kernel<V, R>  one lane per R vectors (consecutive lanes on consecutive vectors),
//                        the vectors held in fp64 registers; every wave walks the whole
//                        record table in index order with uniform (scalar-unit) loads, so
//                        each centroid costs V + 1 fp64 FMAs and one compare per vector,
//                        and the rare improvements take a branch that the wave skips
//                        when none of its lanes improves.
#include "vq_device.h"

namespace {

constexpr int kThreads = 256;

template <int WT>  // VQ_F16, VQ_BF16, VQ_F32
__device__ __forceinline__ double weight_at(const void* w, int64_t i) {
  if constexpr (WT == VQ_F16) {
    return (double)vqd::f16_to_f32(((const uint16_t*)w)[i]);
  } else if constexpr (WT == VQ_BF16) {
    return (double)vqd::bf16_to_f32(((const uint16_t*)w)[i]);
  } else {
    return (double)((const float*)w)[i];
  }
}

__global__ __launch_bounds__(kThreads) void assign_table_kernel(const uint16_t* __restrict__ cb, int32_t k, int32_t v,
                                                                double* __restrict__ tab) {
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= k) return;
  double* rec = tab + (size_t)c * (size_t)(v + 1);
  double nc = 0.0;
  for (int t = 0; t < v; ++t) {
    const double ct = (double)vqd::f16_to_f32(cb[(size_t)c * v + t]);
    nc = fma(ct, ct, nc);
    rec[1 + t] = ct;
  }
  rec[0] = nc;
}

// Lowest index minimising the ranking distance, for each of the lane's R vectors.  The
// record of centroid c + 1 is loaded while centroid c is ranked.
template <int V, int R>
__device__ __forceinline__ void nearest(const double (&w)[R][V], const double* __restrict__ tab, int32_t k,
                                        uint32_t (&best_i)[R]) {
  double best[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    best[r] = __builtin_inf();
    best_i[r] = 0;
  }
  double cur[V + 1];
#pragma unroll
  for (int t = 0; t <= V; ++t) cur[t] = tab[t];  // uniform: the same record for every lane
  for (int32_t c = 0; c < k; ++c) {
    const double* nrec = tab + (size_t)min(c + 1, k - 1) * (V + 1);
    double nxt[V + 1];
#pragma unroll
    for (int t = 0; t <= V; ++t) nxt[t] = nrec[t];
    double d[R];
    bool better = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double dot = fma(w[r][0], cur[1], 0.0);
#pragma unroll
      for (int t = 1; t < V; ++t) dot = fma(w[r][t], cur[1 + t], dot);
      d[r] = fma(-2.0, dot, cur[0]);
      better |= d[r] < best[r];
    }
    if (__any(better)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (d[r] < best[r]) {
          best[r] = d[r];
          best_i[r] = (uint32_t)c;
        }
      }
    }
#pragma unroll
    for (int t = 0; t <= V; ++t) cur[t] = nxt[t];
  }
}

template <int V, int R, int WT>
__global__ __launch_bounds__(kThreads) void assign_kernel(const void* __restrict__ w, int64_t nvec,
                                                          const double* __restrict__ tab1, int32_t k1,
                                                          const double* __restrict__ tab2, int32_t k2,
                                                          uint32_t* __restrict__ idx1, uint32_t* __restrict__ idx2) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * R) + threadIdx.x;
  double wv[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = min(base + (int64_t)r * kThreads, nvec - 1);  // lanes past the end rank a copy
#pragma unroll
    for (int t = 0; t < V; ++t) wv[r][t] = weight_at<WT>(w, g * V + t);
  }
  uint32_t i1[R];
  nearest<V, R>(wv, tab1, k1, i1);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = base + (int64_t)r * kThreads;
    if (g < nvec) idx1[g] = i1[r];
  }
  if (k2 == 0) return;
  // residual in fp32, held exactly in fp64
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double* rec = tab1 + (size_t)i1[r] * (V + 1);
#pragma unroll
    for (int t = 0; t < V; ++t) wv[r][t] = (double)((float)wv[r][t] - (float)rec[1 + t]);
  }
  uint32_t i2[R];
  nearest<V, R>(wv, tab2, k2, i2);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = base + (int64_t)r * kThreads;
    if (g < nvec) idx2[g] = i2[r];
  }
}

template <int V>
vq_status launch_v(const void* w, vq_dtype w_dtype, int64_t nvec, const double* tab1, int32_t k1, const double* tab2,
                   int32_t k2, uint32_t* idx1, uint32_t* idx2, hipStream_t s) {
  constexpr int R = V <= 4 ? 4 : 2;
  const int64_t blocks = (nvec + (int64_t)kThreads * R - 1) / ((int64_t)kThreads * R);
  if (blocks > 0x7FFFFFFF) return VQ_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (w_dtype == VQ_F16) {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_F16>), grid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  } else if (w_dtype == VQ_BF16) {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_BF16>), grid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  } else {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_F32>), grid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  }
  return VQ_OK;
}

}  // namespace

namespace vqi {

size_t assign_workspace(const vq_desc& d) {
  const size_t k = ((size_t)1 << d.bits1) + (d.bits2 ? ((size_t)1 << d.bits2) : 0);
  const size_t bytes = k * (size_t)(d.v + 1) * sizeof(double);
  return (bytes + 255) & ~(size_t)255;
}

vq_status launch_assign(const vq_desc& d, const void* w, vq_dtype w_dtype, const uint16_t* cb1, const uint16_t* cb2,
                        uint32_t* idx1, uint32_t* idx2, void* workspace, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int32_t k1 = 1 << d.bits1, k2 = d.bits2 ? 1 << d.bits2 : 0;
  double* tab1 = (double*)workspace;
  double* tab2 = tab1 + (size_t)k1 * (d.v + 1);
  hipLaunchKernelGGL(assign_table_kernel, dim3((k1 + kThreads - 1) / kThreads), dim3(kThreads), 0, s, cb1, k1, d.v,
                     tab1);
  if (k2) {
    hipLaunchKernelGGL(assign_table_kernel, dim3((k2 + kThreads - 1) / kThreads), dim3(kThreads), 0, s, cb2, k2, d.v,
                       tab2);
  }
  const int64_t nvec = (int64_t)d.out_features * (d.in_features / d.v);
  vq_status st = VQ_OK;
  switch (d.v) {
#define VQ_ASSIGN_CASE(V)                                                             \
  case V:                                                                             \
    st = launch_v<V>(w, w_dtype, nvec, tab1, k1, tab2, k2, idx1, idx2, s); \
    break;
    VQ_ASSIGN_CASE(1)
    VQ_ASSIGN_CASE(2)
    VQ_ASSIGN_CASE(3)
    VQ_ASSIGN_CASE(4)
    VQ_ASSIGN_CASE(5)
    VQ_ASSIGN_CASE(6)
    VQ_ASSIGN_CASE(7)
    VQ_ASSIGN_CASE(8)
    VQ_ASSIGN_CASE(9)
    VQ_ASSIGN_CASE(10)
    VQ_ASSIGN_CASE(11)
    VQ_ASSIGN_CASE(12)
    VQ_ASSIGN_CASE(13)
    VQ_ASSIGN_CASE(14)
    VQ_ASSIGN_CASE(15)
    VQ_ASSIGN_CASE(16)
#undef VQ_ASSIGN_CASE
    default:
      return VQ_ERR_UNSUPPORTED;
  }
  if (st != VQ_OK) return st;
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
