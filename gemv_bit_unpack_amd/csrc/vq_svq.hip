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

template <int CTRL>
__device__ __forceinline__ float dpp_shuffle(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, the same value in every lane, in a fixed order: within each row
// of 16 lanes by DPP (quad_perm [1,0,3,2], [2,3,0,1], row_ror 4, row_ror 8), then the four
// row sums read from lanes 0, 16, 32, 48.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_shuffle<0xB1>(v);
  v += dpp_shuffle<0x4E>(v);
  v += dpp_shuffle<0x124>(v);
  v += dpp_shuffle<0x128>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum over the lanes that agree with this one modulo S (S a power of two up to 64).
template <int S>
__device__ __forceinline__ float wave_sum_stride(float v) {
#pragma unroll
  for (int off = 32; off >= S; off >>= 1) v += __shfl_xor(v, off, vqd::kWave);
  return v;
}

template <int MT, int XT, int L, int R>
__global__ __launch_bounds__(kSvqThreads) void svq_gemv_kernel(SvqArgs p) {
  constexpr int SW = 256 * L;               // columns per slice
  constexpr int SG = SW / 4;                // 4-vectors (code bytes) per slice
  constexpr int XS = SW + 4;                // xh row pitch: batch rows start in different banks
  constexpr int NB = L < 4 ? L : 4;         // code bytes per 32-bit word
  constexpr int ND = L < 4 ? 1 : L / 4;     // 32-bit words per lane and row
  constexpr int PSTEP = kSvqThreads / MT;   // pre-pass: threads per batch row
  constexpr int PI = SG / PSTEP;            // pre-pass: 4-vectors per thread and slice
  static_assert(PI * PSTEP == SG && PI >= 1, "the pre-pass covers the slice exactly");
  constexpr int PB = PI < 2 ? PI : 2;       // pre-pass: activation loads in flight per batch
  using CT = typename CodeWord<L>::T;
  __shared__ float4 xh[MT * XS / 4];
  __shared__ float cbuf[kSvqWaves * MT];
  __shared__ float cfin[MT];

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

  // code bytes of the lane's 4L columns of slice s in each of its rows; a lane past the
  // row end reads the row start instead (its activations are zero)
  auto load_codes = [&](int s, CT (&cw)[R]) __attribute__((always_inline)) {
    const uint32_t boff = (uint32_t)s * SG + (uint32_t)lane * L;
    const uint32_t off = boff < (uint32_t)p.stride ? boff : 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = *(const CT*)(prow[r] + off);
  };

  // pre-pass: thread tid serves batch row pm (rows >= M write zeros) for 4-vectors
  // pi0, pi0 + PSTEP, ...; its loads are clamped into the row and zeroed afterwards, so
  // they issue back to back
  const int pm = tid % MT;
  const int pi0 = tid / MT;
  const bool pm_live = pm < M;
  const uint16_t* xrow = p.x + (size_t)min(pm, M - 1) * (size_t)IN;
  float cpart = 0.0f;

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
  }

  CT cw[R], cn[R];
  for (int s = 0; s < nsl; ++s) {
    // pre-applied activations of the slice (zero past the row end).  Vector g of the slice
    // belongs to lane g / L as its (g % L)-th vector; xh keeps [g % L][lane][4] per batch
    // row so that the lanes' float4 reads below do not share banks.  The thread's PI
    // activation loads go out PB at a time, without branches (and for the first slice
    // ahead of the first code loads), so the pre-pass waits on L2 only.
#pragma unroll
    for (int e0 = 0; e0 < PI; e0 += PB) {
      uint2 xw[PB];  // the 4 activations of each 4-vector, two 16-bit values per word
#pragma unroll
      for (int e = 0; e < PB; ++e) {
        const int pi = pi0 + (e0 + e) * PSTEP;
        const int g = (pi % vqd::kWave) * L + pi / vqd::kWave;
        const int c0 = 4 * (s * SG + g);
        if (p.x_vec4) {  // IN % 4 == 0 and x 8-byte aligned: one load per vector
          xw[e] = *(const uint2*)(xrow + min(c0, IN - 4));
        } else {
          uint32_t raw[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) raw[t] = xrow[min(c0 + t, IN - 1)];
          xw[e] = make_uint2(raw[0] | (raw[1] << 16), raw[2] | (raw[3] << 16));
        }
      }
      if (s == 0 && e0 == 0) load_codes(0, cw);
#pragma unroll
      for (int e = 0; e < PB; ++e) {
        const int pi = pi0 + (e0 + e) * PSTEP;
        const int g = (pi % vqd::kWave) * L + pi / vqd::kWave;
        const int c0 = 4 * (s * SG + g);
        float xv[4];
        const uint32_t raw[4] = {xw[e].x & 0xFFFFu, xw[e].x >> 16, xw[e].y & 0xFFFFu, xw[e].y >> 16};
#pragma unroll
        for (int t = 0; t < 4; ++t) xv[t] = (pm_live && c0 + t < IN) ? vqd::x_to_f32<XT>(raw[t]) : 0.0f;
        float h[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          h[u] = 0.0f;
#pragma unroll
          for (int t = 0; t < 4; ++t) h[u] = __builtin_fmaf(A[t][u], xv[t], h[u]);
          h[u] = h[u] * quarter_pow[u];
        }
        xh[(pm * XS) / 4 + pi] = make_float4(h[0], h[1], h[2], h[3]);
        float cb = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) cb = __builtin_fmaf(B[t], xv[t], cb);
        cpart += cb;
      }
    }
    if (s + 1 < nsl) load_codes(s + 1, cn);  // next slice's codes in flight during this one
    __syncthreads();

    float xr[MT][4 * L];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const float4 v = xh[(m * XS) / 4 + i * vqd::kWave + lane];
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
#pragma unroll
    for (int r = 0; r < R; ++r) cw[r] = cn[r];
    __syncthreads();  // xh is rewritten by the next slice
  }

  // constant term B . sum_j x_mj, over the workgroup in a fixed order: lanes that serve
  // the same batch row (lane % MT) are added across the wavefront, then the wavefronts
  cpart = wave_sum_stride<MT>(cpart);
  if (lane < MT) cbuf[wave * MT + lane] = cpart;
  __syncthreads();
  if (tid < MT) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < kSvqWaves; ++w) c += cbuf[w * MT + tid];
    cfin[tid] = c;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    const int rc = min(row, N - 1);
    const float sc = p.scale ? vqd::f16_to_f32(p.scale[rc]) : 1.0f;
    const float bi = p.bias ? vqd::f16_to_f32(p.bias[rc]) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        float v = wave_sum(acc[r][m]) + cfin[m];
        if (lane == 0 && row < N) {
          if (p.scale) v = v * sc;
          if (p.bias) v = v + bi;
          vqd::store_out(p.y, (size_t)m * N + row, v, p.y_dtype);
        }
      }
    }
  }
}

// M = 1 with the whole row's pre-applied activations resident in LDS (IN4 floats): a
// persistent workgroup of 16 wavefronts computes them once, then each wavefront streams
// work items (a block of R of its rows, one 4096-column slice) with the code loads of the
// next two items in flight, and no barrier until the end.
constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / vqd::kWave;
constexpr int kStreamSW = 4096;              // columns per slice: 16 code bytes per lane
constexpr int kStreamSG = kStreamSW / 4;
constexpr int kStreamMaxSlices = 7;          // 28672 columns
constexpr size_t kStreamLdsMax = (size_t)kStreamMaxSlices * kStreamSW * sizeof(float);

template <int XT, int R>
__global__ __launch_bounds__(kStreamThreads) void svq_gemv_stream_kernel(SvqArgs p, int nsl, int nblocks) {
  extern __shared__ float4 xs[];  // [nsl][16][64]: slice s, vector i of lane l
  __shared__ float cbuf[kStreamWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (vqd::kWave - 1);
  const int wave = tid / vqd::kWave;
  const int IN = p.in_features, N = p.n;
  float A[4][4], B[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    B[t] = vqd::f16_to_f32(p.b[t]);
#pragma unroll
    for (int u = 0; u < 4; ++u) A[t][u] = vqd::f16_to_f32(p.a[t * 4 + u]);
  }
  const float quarter_pow[4] = {1.0f, 0.25f, 0.0625f, 0.015625f};

  // Work items of this wavefront, in order: (k, sl) for its row blocks k (block index
  // blockIdx.x + k * gridDim.x, rows block * 16R + wave * R + r) and slices sl.
  const int my_blocks = (nblocks - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int items = my_blocks * nsl;
  auto load_item = [&](int k, int sl, uint4 (&cw)[R]) __attribute__((always_inline)) {
    const int row0 = ((int)blockIdx.x + k * (int)gridDim.x) * (kStreamWaves * R) + wave * R;
    const uint32_t boff = (uint32_t)sl * kStreamSG + (uint32_t)lane * 16u;
    const uint32_t off = boff < (uint32_t)p.stride ? boff : 0u;  // past the row: its start
#pragma unroll
    for (int r = 0; r < R; ++r)
      cw[r] = *(const uint4*)(p.packed + (size_t)min(row0 + r, N - 1) * (size_t)p.stride + off);
  };
  // next item; past the last one the cursor stays there (its loads repeat, unused)
  auto advance = [&](int& k, int& sl) __attribute__((always_inline)) {
    if (sl + 1 < nsl) {
      ++sl;
    } else if (k + 1 < my_blocks) {
      ++k;
      sl = 0;
    }
  };

  // pre-applied activations of the whole row (zero past IN), and the constant term.
  // Thread tid serves the 4-vectors idx = tid + e * 1024, e < nsl (at most 7): their
  // activations are loaded first, all at once, ahead of the code prefetch, so that the
  // pre-pass waits on L2 only.
  const int total = nsl * kStreamSG;
  uint2 xw[kStreamMaxSlices];
#pragma unroll
  for (int e = 0; e < kStreamMaxSlices; ++e) {
    const int idx = min(tid + e * kStreamThreads, total - 1);
    const int sl = idx / kStreamSG;
    const int pi = idx - sl * kStreamSG;
    const int g = (pi % vqd::kWave) * 16 + pi / vqd::kWave;
    const int c0c = 4 * (sl * kStreamSG + g);
    if (p.x_vec4) {
      xw[e] = *(const uint2*)(p.x + min(c0c, IN - 4));
    } else {
      uint32_t raw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) raw[t] = p.x[min(c0c + t, IN - 1)];
      xw[e] = make_uint2(raw[0] | (raw[1] << 16), raw[2] | (raw[3] << 16));
    }
  }
  uint4 c0[R], c1[R], c2[R];
  int pk = 0, ps = 0;  // prefetch cursor: two items ahead of the one in use
  load_item(pk, ps, c0);
  advance(pk, ps);
  load_item(pk, ps, c1);
  advance(pk, ps);

  float cpart = 0.0f;
#pragma unroll
  for (int e = 0; e < kStreamMaxSlices; ++e) {
    const int idx = tid + e * kStreamThreads;
    if (idx >= total) break;  // uniform across the workgroup: total is a multiple of 1024
    const int sl = idx / kStreamSG;
    const int pi = idx - sl * kStreamSG;
    const int g = (pi % vqd::kWave) * 16 + pi / vqd::kWave;
    const int c0c = 4 * (sl * kStreamSG + g);
    const uint32_t raw[4] = {xw[e].x & 0xFFFFu, xw[e].x >> 16, xw[e].y & 0xFFFFu, xw[e].y >> 16};
    float xv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) xv[t] = c0c + t < IN ? vqd::x_to_f32<XT>(raw[t]) : 0.0f;
    float h[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      h[u] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) h[u] = __builtin_fmaf(A[t][u], xv[t], h[u]);
      h[u] = h[u] * quarter_pow[u];
    }
    xs[idx] = make_float4(h[0], h[1], h[2], h[3]);
    float cb = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) cb = __builtin_fmaf(B[t], xv[t], cb);
    cpart += cb;
  }
  cpart = wave_sum(cpart);
  if (lane == 0) cbuf[wave] = cpart;
  __syncthreads();  // the activations and the wavefront partials of the constant term
  float c = 0.0f;
#pragma unroll
  for (int w = 0; w < kStreamWaves; ++w) c += cbuf[w];

  float xr[64];
  auto load_xr = [&](int sl) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 v = xs[sl * kStreamSG + i * vqd::kWave + lane];
      xr[4 * i] = v.x;
      xr[4 * i + 1] = v.y;
      xr[4 * i + 2] = v.z;
      xr[4 * i + 3] = v.w;
    }
  };
  if (nsl == 1) load_xr(0);
  // four partial sums per row (code position k of each byte), so the FMAs of a row form
  // four independent chains
  float acc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc[r][kk] = 0.0f;
  }
  int ck = 0, cs = 0;  // item in use
  for (int it = 0; it < items; ++it) {
    load_item(pk, ps, c2);
    advance(pk, ps);
    if (nsl > 1) load_xr(cs);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t wd[4] = {c0[r].x, c0[r].y, c0[r].z, c0[r].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          float q[4];
          bytes_to_f32<4>(wd[d] & (0x03030303u << (2 * kk)), q);
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[r][kk] = __builtin_fmaf(q[b], xr[16 * d + 4 * b + kk], acc[r][kk]);
        }
      }
    }
    if (cs == nsl - 1) {  // row block done
      const int row0 = ((int)blockIdx.x + ck * (int)gridDim.x) * (kStreamWaves * R) + wave * R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
        float v = wave_sum((acc[r][0] + acc[r][1]) + (acc[r][2] + acc[r][3])) + c;
        if (lane == 0 && row < N) {
          if (p.scale) v = v * vqd::f16_to_f32(p.scale[row]);
          if (p.bias) v = v + vqd::f16_to_f32(p.bias[row]);
          vqd::store_out(p.y, row, v, p.y_dtype);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc[r][kk] = 0.0f;
      }
    }
    advance(ck, cs);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      c0[r] = c1[r];
      c1[r] = c2[r];
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
  // four rows per wavefront once there are enough rows to fill the chip in steps of 32
  // rows, one below that; from M = 8 the per-slice activation copy is worth sharing
  // over four rows (two at M = 16, where four would not fit in registers)
  if constexpr (MT >= 16) {
    return launch_rows<MT, XT, L, 2>(p, s);
  } else if constexpr (MT >= 8) {
    return launch_rows<MT, XT, L, 4>(p, s);
  } else {
    if (p.n >= 16384) return launch_rows<MT, XT, L, 4>(p, s);
    return launch_rows<MT, XT, L, 1>(p, s);
  }
}

template <int XT, int R>
vq_status launch_stream(const SvqArgs& p, int nsl, hipStream_t s) {
  auto kern = svq_gemv_stream_kernel<XT, R>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLdsMax);
  if (attr != hipSuccess) return VQ_ERR_HIP;
  const int nblocks = (p.n + kStreamWaves * R - 1) / (kStreamWaves * R);
  const int grid = nblocks < 256 ? nblocks : 256;  // one persistent workgroup per CU
  const size_t lds = (size_t)nsl * kStreamSW * sizeof(float);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kStreamThreads), lds, s, p, nsl, nblocks);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int XT>
vq_status launch_x(const SvqArgs& p, hipStream_t s) {
  if (p.m <= 1) {
    // the streaming kernel when one row's pre-applied activations fit in LDS
    const int nsl = (p.nv + kStreamSG - 1) / kStreamSG;
    // when one row's pre-applied activations fit in LDS and there are enough rows for
    // every persistent workgroup to stream several items
    if (nsl > 0 && nsl <= kStreamMaxSlices && p.n >= 2 * 256 * kStreamWaves) return launch_stream<XT, 2>(p, nsl, s);
    return launch_m<1, XT>(p, s);
  }
  if (p.m <= 2) return launch_m<2, XT>(p, s);
  if (p.m <= 4) return launch_m<4, XT>(p, s);
  if (p.m <= 8) return launch_m<8, XT>(p, s);
  return launch_m<16, XT>(p, s);
}

}  // namespace

namespace vqi {

vq_status launch_svq_gemv(const SvqArgs& p, void* stream) {
  // From M = 4 the matrix-core kernel of vq_svq_gemm is as fast or faster: its cost hardly
  // grows with M, the VALU kernels' grows linearly (us, VALU / matrix cores: 4096^2 at M = 8
  // 20.8 / 11.1; 8192 x 28672 at M = 4 85.0 / 51.6; 14336 x 4096 at M = 4 13.5 / 13.5; at
  // M = 2 the VALU kernel is ahead on three of these four layers).
  if (p.in_features > 0 && p.m >= 4) return launch_svq_gemm(p, stream);
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
