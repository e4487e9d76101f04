// vq_svq_gemm: prefill-batch product of an affine-lattice layer (UniSVQ summary,
// "Mathematical Formulation"; the prefill regime of the production-VQ post, "Prefill vs.
// Decode Bottlenecks"), y[M][N] = x[M][IN] * W^T (+ bias) with
//
//   W^[o, 4j + t] = scale[o] * fp32(B[t] + sum_u A[t][u] * q_u(o, j)),
//
// on the matrix cores.  A lattice vector is one code byte, so the layer's weights take at
// most 256 distinct 4-vectors: each workgroup first writes that table (byte -> the four
// weights in the activation's 16-bit type; bf16 activations get a hi + lo pair,
// hi = RNE(w), lo = RNE(w - hi), ~16 significant bits of w) into LDS, and the MFMA
// A fragments are then read from it directly, two table entries per fragment, with no
// weight tile at all.  Work split: a workgroup owns 128 output rows (wavefront w the 32
// rows 32w .. 32w + 31) and a chunk of 32 * MB batch rows; per K-tile of 64 columns
// (16 lattice vectors per row) each lane holds its row's 16 code bytes, the x tile
// [32 * MB][64] sits in LDS (double-buffered), and each wavefront runs 4 x MB
// v_mfma_f32_32x32x16 (twice for bf16) into fp32 accumulators.  The next tile's codes and
// x are loaded into registers while the current tile is multiplied.  Columns past IN
// meet zero activations, so the padding codes of the last tile contribute nothing.  The
// channel scale and bias are applied once per output in the epilogue.
#include "vq_device.h"

namespace {

using vqi::SvqArgs;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kNumCUs = 256;
constexpr int kBK = 64;          // K-tile width in columns (16 lattice vectors)
constexpr int kLd = kBK + 8;     // LDS row stride of the x tile in halves (16 bytes of padding)

template <int XT>
__device__ __forceinline__ void build_entry(const SvqArgs& p, uint4* lut, int e) {
  // entry e: the four weights of code byte e (table of 16-byte entries: fp16 uses the
  // first 8 bytes, bf16 holds hi in the first 8 and lo in the last 8)
  uint16_t hv[4], lv[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float w = vqd::f16_to_f32(p.b[t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) w = fmaf(vqd::f16_to_f32(p.a[t * 4 + u]), (float)((e >> (2 * u)) & 3), w);
    if constexpr (XT == 0) {
      hv[t] = vqd::f32_to_f16_rne(w);
      lv[t] = 0;
    } else {
      hv[t] = vqd::f32_to_bf16_rne(w);
      lv[t] = vqd::f32_to_bf16_rne(w - vqd::bf16_to_f32(hv[t]));
    }
  }
  lut[e] = make_uint4(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16),
                      lv[0] | ((uint32_t)lv[1] << 16), lv[2] | ((uint32_t)lv[3] << 16));
}

// x tile [32 * MB][64] of one K-stream of T threads: 256 * MB chunks of 8 columns, thread
// tg takes chunks tg, tg + T, ...
template <int MB, int T>
__device__ __forceinline__ void load_x(const SvqArgs& p, int m0, int k0, bool x_vec, int tg,
                                       uint4 (&xr)[256 * MB / T]) {
#pragma unroll
  for (int i = 0; i < 256 * MB / T; ++i) {
    const int ch = tg + i * T;
    const int m = m0 + (ch >> 3);
    const int k = k0 + (ch & 7) * 8;
    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    if (m < p.m) {
      const uint16_t* row = p.x + (size_t)m * p.in_features;
      if (x_vec && k + 8 <= p.in_features) {
        q = *(const uint4*)(row + k);
      } else {
        uint16_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (k + e < p.in_features) ? row[k + e] : (uint16_t)0;
        q.x = h[0] | ((uint32_t)h[1] << 16);
        q.y = h[2] | ((uint32_t)h[3] << 16);
        q.z = h[4] | ((uint32_t)h[5] << 16);
        q.w = h[6] | ((uint32_t)h[7] << 16);
      }
    }
    xr[i] = q;
  }
}

template <int MB, int T>
__device__ __forceinline__ void store_x(uint16_t* xt, int tg, const uint4 (&xr)[256 * MB / T]) {
#pragma unroll
  for (int i = 0; i < 256 * MB / T; ++i) {
    const int ch = tg + i * T;
    *(uint4*)(xt + (ch >> 3) * kLd + (ch & 7) * 8) = xr[i];
  }
}

// A workgroup runs KS K-streams of RW wavefronts: wavefront w of a stream owns the 32 output
// rows 32 w .. 32 w + 31 of the workgroup's 32 RW, stream g takes the K-tiles g, g + KS, ...
// with its own x buffers, and streams 1 .. KS-1 hand their sums to stream 0 through LDS at
// the end (added in stream order).  More streams serve layers with few row blocks.
template <int MB, int XT, int RW, int KS>  // XT: 0 fp16 activations, 1 bf16
__global__ __launch_bounds__(64 * RW * KS) void svq_gemm_kernel(SvqArgs p) {
  constexpr int T = 64 * RW;  // threads per stream
  __shared__ uint4 lut[256];
  __shared__ __attribute__((aligned(16))) uint16_t xt[KS][2][32 * MB * kLd];
  static_assert(KS == 1 || sizeof(xt) >= (size_t)(KS - 1) * RW * MB * 16 * 64 * sizeof(float), "reduction area");
  const int tg = threadIdx.x % T;  // thread within its stream
  const int grp = threadIdx.x / T; // K-stream
  const int lane = tg & 63;
  const int wave = tg >> 6;     // row block of the stream
  const int ar = lane & 31;     // A row / B column of this lane
  const int kh = lane >> 5;     // which 8 of the 16 k of a step
  const int m0 = blockIdx.y * 32 * MB;
  const int row = blockIdx.x * (32 * RW) + wave * 32 + ar;
  const int nkt = (p.in_features + kBK - 1) / kBK;
  const int nit = (nkt + KS - 1) / KS;  // iterations, the same for every stream
  const bool x_vec = p.in_features % 8 == 0 && ((uintptr_t)p.x & 15) == 0;

  float16_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  if (nkt > 0) {
    for (int e = threadIdx.x; e < 256; e += T * KS) build_entry<XT>(p, lut, e);
    const uint8_t* crow = p.packed + (size_t)min(row, p.n - 1) * p.stride;  // rows past N read a copy
    const int kt0 = min(grp, nkt - 1);
    uint4 code = *(const uint4*)(crow + 16 * kt0);  // 16 code bytes of the stream's first K-tile
    uint4 xr[256 * MB / T];
    load_x<MB, T>(p, m0, kt0 * kBK, x_vec, tg, xr);
    store_x<MB, T>(xt[grp][0], tg, xr);
    __syncthreads();
    for (int it = 0; it < nit; ++it) {
      const int buf = it & 1;
      const int kt = it * KS + grp;
      // next tile of this stream into registers while this one is multiplied
      const int nt = min(kt + KS, nkt - 1);
      const uint4 ncode = *(const uint4*)(crow + 16 * nt);
      load_x<MB, T>(p, m0, nt * kBK, x_vec, tg, xr);
      if (KS == 1 || kt < nkt) {
        const uint32_t cw[4] = {code.x, code.y, code.z, code.w};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          // this lane's 8 k of step ks: lattice vectors 4 ks + 2 kh and + 1 of its row
          const uint32_t pair = cw[ks] >> (16 * kh);
          const uint4 e0 = lut[pair & 0xFFu];
          const uint4 e1 = lut[(pair >> 8) & 0xFFu];
          const uint4 ahi = make_uint4(e0.x, e0.y, e1.x, e1.y);
#pragma unroll
          for (int i = 0; i < MB; ++i) {
            const uint4 bw = *(const uint4*)(xt[grp][buf] + (i * 32 + ar) * kLd + ks * 16 + kh * 8);
            if constexpr (XT == 0) {
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, ahi),
                                                              __builtin_bit_cast(half8_t, bw), acc[i], 0, 0, 0);
            } else {
              const uint4 alo = make_uint4(e0.z, e0.w, e1.z, e1.w);
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ahi),
                                                               __builtin_bit_cast(bf16x8_t, bw), acc[i], 0, 0, 0);
              acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, alo),
                                                               __builtin_bit_cast(bf16x8_t, bw), acc[i], 0, 0, 0);
            }
          }
        }
      }
      store_x<MB, T>(xt[grp][buf ^ 1], tg, xr);  // the other buffer: last read before the previous barrier
      code = ncode;
      __syncthreads();
    }
    if constexpr (KS > 1) {
      // streams 1 .. KS-1 hand their sums to stream 0 (the x buffers are free after the last barrier)
      float* red = (float*)&xt[0][0][0];
      if (grp > 0) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((((grp - 1) * RW + wave) * MB + i) * 16 + r) * 64 + lane] = acc[i][r];
      }
      __syncthreads();
      if (grp == 0) {
        for (int g = 1; g < KS; ++g) {
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] += red[((((g - 1) * RW + wave) * MB + i) * 16 + r) * 64 + lane];
        }
      }
    }
  }
  if (grp != 0) return;
  // Epilogue: accumulator register r of lane l holds output row 8*(r/4) + 4*(l/32) + r%4
  // of the wavefront's 32 and batch row l%32 of block i.
  const int rbase = blockIdx.x * (32 * RW) + wave * 32;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + i * 32 + ar;
    if (m >= p.m) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = rbase + 8 * (r >> 2) + 4 * kh + (r & 3);
      if (n < p.n) {
        float out = acc[i][r];
        if (p.scale) out = out * vqd::f16_to_f32(p.scale[n]);
        if (p.bias) out = out + vqd::f16_to_f32(p.bias[n]);
        vqd::store_out(p.y, (size_t)m * p.n + n, out, p.y_dtype);
      }
    }
  }
}

template <int MB, int RW, int KS>
void launch_cfg(const SvqArgs& p, hipStream_t s) {
  const int chunk = 32 * MB;
  const dim3 grid((unsigned)((p.n + 32 * RW - 1) / (32 * RW)), (unsigned)((p.m + chunk - 1) / chunk));
  if (p.x_dtype == VQ_BF16) {
    hipLaunchKernelGGL((svq_gemm_kernel<MB, 1, RW, KS>), grid, dim3(64 * RW * KS), 0, s, p);
  } else {
    hipLaunchKernelGGL((svq_gemm_kernel<MB, 0, RW, KS>), grid, dim3(64 * RW * KS), 0, s, p);
  }
}

// cfg: 0 = 4 row blocks x 1 stream, 1 = 4 x 2, 2 = 2 x 4, 3 = 1 x 8 (MB <= 2 for 2 and 3)
template <int MB>
void launch_mb(const SvqArgs& p, hipStream_t s, int cfg) {
  if (cfg == 0) {
    launch_cfg<MB, 4, 1>(p, s);
  } else if (cfg == 1) {
    launch_cfg<MB, 4, 2>(p, s);
  } else if constexpr (MB <= 2) {
    if (cfg == 2) {
      launch_cfg<MB, 2, 4>(p, s);
    } else {
      launch_cfg<MB, 1, 8>(p, s);
    }
  } else {
    launch_cfg<MB, 4, 2>(p, s);
  }
}

// Workgroup shape from the number of 128-row workgroups the layer and batch chunk give:
// fewer row blocks, more K-streams.  Measured per layer (us, shapes 4x1 / 4x2 / 2x4 / 1x8):
// 8192 x 28672 at M = 16 209 / 145 / 85 / 60 (64 workgroups); 4096^2 at M = 16
// 27 / 21 / 14 / 12 (32); 14336 x 4096 at M = 16 27 / 21 / 15 / 17 (112); 8192 x 28672 at
// M = 128 220 / 164 / 162 / 201 (256); 28672 x 8192 at M = 128 134 / 123 / 145 / 250 (448).
int svq_gemm_cfg(int64_t wgs, int mb, int in_features) {
  if (in_features <= kBK) return 0;
  if (wgs < 96 && mb <= 2) return 3;    // 1 row block, eight K-streams
  if (wgs < 384 && mb <= 2) return 2;   // 2 row blocks, four K-streams
  if (wgs < 1024) return 1;             // 4 row blocks, two K-streams
  return 0;                             // 4 row blocks, one K-stream
}

}  // namespace

namespace vqi {

vq_status launch_svq_gemm(const SvqArgs& p, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // batch chunk: the largest of 128 / 64 / 32 rows that still gives at least 384 workgroups
  // of 128 output rows (1.5 per CU); layers with few rows take 32-row chunks and read
  // their codes once per chunk.  (70B-class pair, M = 128: 64-row chunks for the
  // 28672-row layer, 139 us against 174 us with 128-row chunks; 32-row chunks for the
  // 8192-row layer, 240 us against 495 us.)
  const int64_t row_blocks = (p.n + 127) / 128;
  auto wgs = [&](int mb) { return row_blocks * ((p.m + 32 * mb - 1) / (32 * mb)); };
  const bool tall = (p.m + 31) / 32 > 65535;  // too many 32-row chunks for the grid: 128-row ones
  const int mb = (tall || (p.m > 64 && wgs(4) >= 384)) ? 4
                 : (p.m > 32 && (wgs(2) >= 384 || (p.m + 31) / 32 > 65535)) ? 2
                                                                             : 1;
  const int cfg = svq_gemm_cfg(wgs(mb), mb, p.in_features);
  if (mb == 4) {
    launch_mb<4>(p, s, cfg);
  } else if (mb == 2) {
    launch_mb<2>(p, s, cfg);
  } else {
    launch_mb<1>(p, s, cfg);
  }
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
