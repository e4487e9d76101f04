// vq_rht: randomized Walsh-Hadamard transform of the activations, the incoherence step
// that runs ahead of a product with incoherence-processed weights (production-VQ post,
// QuIP#: randomized orthogonal Hadamard transforms on the layer's inputs and outputs; the
// sub-4-bit lecture, "QuIP#: Incoherence Processing": Hadamard plus random signs at
// O(d log d); UniSVQ summary, "Preprocessing (Randomized Hadamard Transform - RHT)").
//
// For each row of x [M][n] and each block of b columns (b: the largest power of two that
// divides n, at most 16384):
//   forward    y = H_b (s . x) / sqrt(b)
//   transpose  y = s . (H_b x) / sqrt(b)          (the inverse of forward)
// with H_b[i][j] = (-1)^popcount(i & j) and s_j = -1 where sign bit j is set.
//
// One workgroup per (row, block), b / 16 threads, 16 values per thread in registers.  The
// fast transform is a butterfly on every bit of the index; a thread's 16 values differ in
// a window of 4 index bits, so 4 butterfly stages run in registers, then the values go
// through LDS (padded so that neither the contiguous nor the strided pattern shares banks)
// to the next window: at most 4 register phases for b = 16384.  The first phase reads 16
// contiguous inputs per thread, the last writes with consecutive threads on consecutive
// columns.  Arithmetic in fp32.
#include "vq_device.h"

namespace {

constexpr int kMaxLog = 14;  // b <= 16384: at most 1024 threads of 16 values

__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 5); }

// Index of value k of thread t when the register window starts at bit w.
__device__ __forceinline__ int win_index(int t, int k, int w) {
  return ((t >> w) << (w + 4)) | (k << w) | (t & ((1 << w) - 1));
}

template <int Q>
__device__ __forceinline__ void butterfly(float (&v)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (!(k & (1 << Q))) {
      const float a = v[k], c = v[k | (1 << Q)];
      v[k] = a + c;
      v[k | (1 << Q)] = a - c;
    }
  }
}

template <int T>  // 0 fp16, 1 bf16, 2 fp32
__device__ __forceinline__ void load16(const void* p, size_t i, float (&v)[16]) {
  if constexpr (T == 2) {
    const float4* q = (const float4*)((const float*)p + i);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 f = q[h];
      v[4 * h] = f.x;
      v[4 * h + 1] = f.y;
      v[4 * h + 2] = f.z;
      v[4 * h + 3] = f.w;
    }
  } else {
    const uint4* q = (const uint4*)((const uint16_t*)p + i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 u = q[h];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        v[8 * h + 2 * d] = vqd::x_to_f32<T>(w[d] & 0xFFFFu);
        v[8 * h + 2 * d + 1] = vqd::x_to_f32<T>(w[d] >> 16);
      }
    }
  }
}

template <int XT>
__global__ __launch_bounds__(1024) void rht_kernel(const void* __restrict__ x, const uint8_t* __restrict__ signs,
                                                   void* __restrict__ y, vq_dtype y_dtype, int n, int L, float inv,
                                                   int transpose) {
  extern __shared__ float buf[];
  const int t = threadIdx.x;  // blockDim.x == 2^(L - 4)
  const int nblk = n >> L;
  const int m = blockIdx.x / nblk;
  const int base = (blockIdx.x - m * nblk) << L;
  const size_t row = (size_t)m * (size_t)n + (size_t)base;

  float v[16];
  load16<XT>(x, row + 16 * (size_t)t, v);  // window 0: value k is column 16 t + k
  if (!transpose) {
    const int c0 = base + 16 * t;  // a multiple of 16: two whole sign bytes
    const uint32_t bits = (uint32_t)signs[c0 >> 3] | ((uint32_t)signs[(c0 >> 3) + 1] << 8);
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = ((bits >> k) & 1u) ? -v[k] : v[k];
  }
  const int P = (L + 3) / 4;
  int w = 0;
  for (int p = 0; p < P; ++p) {
    w = min(4 * p, L - 4);
    if (p > 0) {
      __syncthreads();  // the previous phase's values are all in LDS
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = buf[lds_pad(win_index(t, k, w))];
    }
    // index bits 4p .. min(4p + 4, L) - 1, i.e. register bits q0 .. q1 - 1 of the window
    const int q0 = 4 * p - w, q1 = min(4 * p + 4, L) - w;
    if (q0 <= 0 && 0 < q1) butterfly<0>(v);
    if (q0 <= 1 && 1 < q1) butterfly<1>(v);
    if (q0 <= 2 && 2 < q1) butterfly<2>(v);
    if (q0 <= 3 && 3 < q1) butterfly<3>(v);
    if (p + 1 < P) {
      __syncthreads();  // every thread has read this phase's inputs
#pragma unroll
      for (int k = 0; k < 16; ++k) buf[lds_pad(win_index(t, k, w))] = v[k];
    }
  }
  // last window starts at bit L - 4: value k is column (k << w) | t
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = (k << w) | t;
    float r = v[k] * inv;
    if (transpose && ((signs[(base + i) >> 3] >> ((base + i) & 7)) & 1)) r = -r;
    vqd::store_out(y, row + (size_t)i, r, y_dtype);
  }
}

}  // namespace

namespace vqi {

int32_t rht_block(int32_t n) {
  if (n <= 0) return 0;
  int32_t b = 1;
  while (b < (1 << kMaxLog) && n % (2 * b) == 0) b *= 2;
  return b;
}

vq_status launch_rht(int32_t m, int32_t n, const void* x, vq_dtype x_dtype, const uint8_t* signs, int32_t transpose,
                     void* y, vq_dtype y_dtype, void* stream) {
  const int32_t b = rht_block(n);
  int L = 0;
  while ((1 << L) < b) ++L;
  const unsigned grid = (unsigned)((int64_t)m * (n / b));
  const size_t lds = (size_t)(b + (b >> 5)) * sizeof(float);
  const float inv = (float)(1.0 / __builtin_sqrt((double)b));
  hipStream_t s = (hipStream_t)stream;
  const int threads = b / 16;
  if (x_dtype == VQ_F16) {
    hipLaunchKernelGGL(rht_kernel<0>, dim3(grid), dim3(threads), lds, s, x, signs, y, y_dtype, n, L, inv, transpose);
  } else if (x_dtype == VQ_BF16) {
    hipLaunchKernelGGL(rht_kernel<1>, dim3(grid), dim3(threads), lds, s, x, signs, y, y_dtype, n, L, inv, transpose);
  } else {
    hipLaunchKernelGGL(rht_kernel<2>, dim3(grid), dim3(threads), lds, s, x, signs, y, y_dtype, n, L, inv, transpose);
  }
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
