// vq_svq: layers whose weight vectors lie on an affine integer grid (UniSVQ summary,
// "Mathematical Formulation": a d = 4 vector is A q + B over integer coordinates q;
// "Efficiency": 2 bits per coordinate, 20 parameters per matrix, and the affine map can
// be moved onto the activations, which leaves a plain low-bit scalar product).
//
// Storage: one 8-bit field per 4-vector, code u (the integer coordinate q_u, 0..3) in bits
// [2u, 2u + 2); rows are packed like a v = 4, bits1 = 8 index stream, so the weights of a
// row are consecutive 2-bit codes and a row takes 16 * ceil(nv / 16) bytes.
//
// svq_gemv_kernel computes y[m][o] = s_o (sum_j q_oj . (A^T x_mj) + B . sum_j x_mj) + bias_o
// over the 4-vectors j of a row.  Mapping on gfx950:
//   - a workgroup (8 wavefronts) owns 8R consecutive rows, R per wavefront; the columns
//     are walked in slices of 256 L weights, L code bytes per lane per row, so one load
//     instruction of a wavefront reads 64 L contiguous bytes of a row;
//   - per slice the workgroup first issues the loads of its code bytes, then writes the
//     pre-applied activations of the slice to LDS, xh[m][col] = (A^T x_mj)_u * 4^-u for
//     col = 4 j + u, and adds B . x_mj to a per-thread partial of the constant term;
//   - each lane copies the activations of its 4 L columns into registers and runs its R
//     rows through them.  For a 32-bit code word, AND with 0x03030303 << 2u leaves code u
//     of the word's four vectors as bytes q_u * 4^u; v_cvt_f32_ubyte turns each byte into
//     a float, and the 4^-u folded into xh makes the product exact again.  Per word: 4
//     ANDs, 16 conversions and 16 M FMAs, no lookups;
//   - the row sums are reduced across the wavefront once at the end; the constant term is
//     reduced over the workgroup once and added to every row.
// L falls with M so that the activations of a lane stay in registers: L = 16 at M = 1,
// 8 at M = 2, 4 up to M = 8, 2 up to M = 16.
//
// svq_dequant_kernel writes W itself: coordinate t of a vector is B_t + sum_u A_tu q_u,
// summed in double (every term, an fp16 value times an integer below 4, and every partial
// sum is exact there) and rounded once to fp32, then times the channel scale in fp32.
#include "vq_device.h"

namespace {

using vqi::SvqArgs;

constexpr int kSvqThreads = 512;
constexpr int kSvqWaves = kSvqThreads / vqd::kWave;

template <int L>
struct CodeWord;
template <>
struct CodeWord<16> {
  using T = uint4;
};
template <>
struct CodeWord<8> {
  using T = uint2;
};
template <>
struct CodeWord<4> {
  using T = uint32_t;
};
template <>
struct CodeWord<2> {
  using T = uint16_t;
};

template <int L>
__device__ __forceinline__ uint32_t code_dword(const typename CodeWord<L>::T& c, int d) {
  if constexpr (L == 16) {
    return d == 0 ? c.x : d == 1 ? c.y : d == 2 ? c.z : c.w;
  } else if constexpr (L == 8) {
    return d == 0 ? c.x : c.y;
  } else {
    return (uint32_t)c;
  }
}

// Byte b of w as a float: v_cvt_f32_ubyte{b} reads the byte in place.  (Written out because
// the compiler otherwise extracts each byte with a separate instruction first.)
template <int B>
__device__ __forceinline__ float ubyte_to_f32(uint32_t w) {
  float f;
  if constexpr (B == 0) {
    asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(w));
  } else if constexpr (B == 1) {
    asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(w));
  } else if constexpr (B == 2) {
    asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(w));
  } else {
    asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(w));
  }
  return f;
}

template <int NB>
__device__ __forceinline__ void bytes_to_f32(uint32_t w, float (&q)[4]) {
  q[0] = ubyte_to_f32<0>(w);
  if constexpr (NB > 1) q[1] = ubyte_to_f32<1>(w);
  if constexpr (NB > 2) q[2] = ubyte_to_f32<2>(w);
  if constexpr (NB > 3) q[3] = ubyte_to_f32<3>(w);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, vqd::kWave);
  return v;
}

template <int MT, int XT, int L, int R>
__global__ __launch_bounds__(kSvqThreads) void svq_gemv_kernel(SvqArgs p) {
  constexpr int SW = 256 * L;               // columns per slice
  constexpr int SG = SW / 4;                // 4-vectors (code bytes) per slice
  constexpr int NB = L < 4 ? L : 4;         // code bytes per 32-bit word
  constexpr int ND = L < 4 ? 1 : L / 4;     // 32-bit words per lane and row
  using CT = typename CodeWord<L>::T;
  __shared__ float xh[MT * SW];
  __shared__ float cred[kSvqWaves * MT];

  const int tid = threadIdx.x;
  const int lane = tid & (vqd::kWave - 1);
  const int wave = tid / vqd::kWave;
  const int M = p.m, IN = p.in_features, N = p.n;
  float A[4][4], B[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    B[t] = vqd::f16_to_f32(p.b[t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) A[t][u] = vqd::f16_to_f32(p.a[t * 4 + u]);
  }
  const float quarter_pow[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};

  const int row0 = blockIdx.x * (kSvqWaves * R) + wave * R;
  const uint8_t* prow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) prow[r] = p.packed + (size_t)min(row0 + r, N - 1) * (size_t)p.stride;
  const int nsl = (p.nv + SG - 1) / SG;

  float acc[R][MT];
  float cpart[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    cpart[m] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][m] = 0.0f;
  }

  for (int s = 0; s < nsl; ++s) {
    // code bytes of the lane's 4L columns in each of its rows; a lane past the row end
    // reads the row start instead (its activations below are zero)
    const uint32_t boff = (uint32_t)s * SG + (uint32_t)lane * L;
    const uint32_t off = boff < (uint32_t)p.stride ? boff : 0u;
    CT cw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = *(const CT*)(prow[r] + off);

    // pre-applied activations of the slice (zero past the row end).  Vector g of the slice
    // belongs to lane g / L as its (g % L)-th vector; xh keeps [g % L][lane][4] so that the
    // lanes' float4 reads below, and these writes (lane fastest), do not share banks.
    for (int idx = tid; idx < SG; idx += kSvqThreads) {
      const int g = (idx % vqd::kWave) * L + idx / vqd::kWave;
      const int j = s * SG + g;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float xv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (m < M) {
          const uint16_t* xrow = p.x + (size_t)m * IN;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int col = 4 * j + t;
            if (col < IN) xv[t] = vqd::x_to_f32<XT>(xrow[col]);
          }
        }
        float h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          h[u] = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) h[u] = __builtin_fmaf(A[t][u], xv[t], h[u]);
          h[u] = h[u] * quarter_pow[u];
        }
        *(float4*)&xh[m * SW + 4 * idx] = make_float4(h[0], h[1], h[2], h[3]);
        float cb = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) cb = __builtin_fmaf(B[t], xv[t], cb);
        cpart[m] += cb;
      }
    }
    __syncthreads();

    float xr[MT][4 * L];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const float4 v = *(const float4*)&xh[m * SW + 4 * (i * vqd::kWave + lane)];
        xr[m][4 * i] = v.x;
        xr[m][4 * i + 1] = v.y;
        xr[m][4 * i + 2] = v.z;
        xr[m][4 * i + 3] = v.w;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const uint32_t w = code_dword<L>(cw[r], d);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float q[4];
          bytes_to_f32<NB>(w & (0x03030303u << (2 * k)), q);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            // rows m >= M have zero activations: their sums stay zero and are not stored
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = __builtin_fmaf(q[b], xr[m][16 * d + 4 * b + k], acc[r][m]);
          }
        }
      }
    }
    __syncthreads();  // xh is rewritten by the next slice
  }

  // constant term B . sum_j x_mj, over the whole workgroup in a fixed order
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float v = wave_sum(cpart[m]);
    if (lane == 0) cred[wave * MT + m] = v;
  }
  __syncthreads();
  float c[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    c[m] = 0.0f;
#pragma unroll
    for (int w = 0; w < kSvqWaves; ++w) c[m] += cred[w * MT + m];
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    const int rc = min(row, N - 1);
    const float sc = p.scale ? vqd::f16_to_f32(p.scale[rc]) : 1.0f;
    const float bi = p.bias ? vqd::f16_to_f32(p.bias[rc]) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        float v = wave_sum(acc[r][m]) + c[m];
        if (lane == 0 && row < N) {
          if (p.scale) v = v * sc;
          if (p.bias) v = v + bi;
          vqd::store_out(p.y, (size_t)m * N + row, v, p.y_dtype);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void svq_dequant_kernel(SvqArgs p, void* w, vq_dtype w_dtype) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4-vector index over the layer
  if (i >= (int64_t)p.n * p.nv) return;
  const int64_t o = i / p.nv;
  const int64_t j = i - o * p.nv;
  const uint32_t field = p.packed[(size_t)o * p.stride + (size_t)j];
  const float sc = p.scale ? vqd::f16_to_f32(p.scale[o]) : 1.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t col = 4 * j + t;
    if (col >= p.in_features) break;
    double v = (double)vqd::f16_to_f32(p.b[t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) v += (double)vqd::f16_to_f32(p.a[t * 4 + u]) * (double)((field >> (2 * u)) & 3u);
    float f = (float)v;
    if (p.scale) f = f * sc;
    vqd::store_out(w, (size_t)o * p.in_features + (size_t)col, f, w_dtype);
  }
}

template <int MT, int XT, int L, int R>
vq_status launch_rows(const SvqArgs& p, hipStream_t s) {
  const int rows_per_group = kSvqWaves * R;
  const unsigned grid = (unsigned)((p.n + rows_per_group - 1) / rows_per_group);
  hipLaunchKernelGGL((svq_gemv_kernel<MT, XT, L, R>), dim3(grid), dim3(kSvqThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int MT, int XT>
vq_status launch_m(const SvqArgs& p, hipStream_t s) {
  constexpr int L = MT == 1 ? 16 : MT == 2 ? 8 : MT <= 8 ? 4 : 2;
  // four rows per wavefront once there are enough rows to fill the chip with 512-row
  // steps of 32 rows; one row per wavefront below that
  if (p.n >= 16384) return launch_rows<MT, XT, L, 4>(p, s);
  return launch_rows<MT, XT, L, 1>(p, s);
}

template <int XT>
vq_status launch_x(const SvqArgs& p, hipStream_t s) {
  if (p.m <= 1) return launch_m<1, XT>(p, s);
  if (p.m <= 2) return launch_m<2, XT>(p, s);
  if (p.m <= 4) return launch_m<4, XT>(p, s);
  if (p.m <= 8) return launch_m<8, XT>(p, s);
  return launch_m<16, XT>(p, s);
}

}  // namespace

namespace vqi {

vq_status launch_svq_gemv(const SvqArgs& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  return p.x_dtype == VQ_BF16 ? launch_x<1>(p, s) : launch_x<0>(p, s);
}

vq_status launch_svq_dequant(const SvqArgs& p, void* w, vq_dtype w_dtype, void* stream) {
  const int64_t total = (int64_t)p.n * p.nv;
  const unsigned grid = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(svq_dequant_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, p, w, w_dtype);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
