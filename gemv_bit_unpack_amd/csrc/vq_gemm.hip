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
constexpr int kNumCUs = 256;
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

// ---------------------------------------------------------------------------------
// Fast path for v = 8 (IN % 8 == 0, even index widths, 16-byte aligned codebooks and x):
// 32*RB output rows per workgroup, K-tiles of 64 columns (8 vectors per row),
// software-pipelined.  While the wavefronts run the MFMAs of tile t from LDS, the
// centroid gathers and x chunks of tile t+1 are already in flight into registers; at the
// top of the next iteration they are rebuilt/converted and written to LDS.  The index
// streams are staged in LDS a super-tile (64 vectors = 8 K-tiles) at a time, prefetched
// one super-tile ahead, so each index line is read from L2 once instead of per tile.
// Main book: global (16-bit indices, K1 = 65536) or LDS (K1 <= 4096); residual in LDS.
constexpr int kBK8 = 64;               // columns per K-tile
constexpr int kLd8 = kBK8 + 8;         // LDS row stride (halves): +16 bytes against bank conflicts
constexpr int kSuper = 8;              // K-tiles per index super-tile

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Field jj (bits [jj*bits, (jj+1)*bits)) of a super-tile row staged in LDS (one spare
// word after each row keeps the second read in bounds).
template <int IB>
__device__ __forceinline__ uint32_t lds_index(const uint32_t* row, uint32_t jj, uint32_t bits) {
  if constexpr (IB == 16) {
    return ((const uint16_t*)row)[jj];
  } else {
    const uint32_t bitpos = jj * bits;
    const uint32_t w = bitpos >> 5;
    return __builtin_amdgcn_alignbit(row[w + 1], row[w], bitpos & 31u) & ((1u << bits) - 1u);
  }
}

__device__ __forceinline__ float h_at(const uint4& q, int t) {
  const uint32_t w = t < 2 ? q.x : t < 4 ? q.y : t < 6 ? q.z : q.w;
  return vqd::f16_to_f32((t & 1) ? (w >> 16) : w);
}

// KS streams of four wavefronts each take every KS-th K-tile of the same row block
// (same barriers, own LDS tiles and accumulators); their partial sums are added through
// LDS at the end.  KS = 2 doubles the loads in flight per CU when a layer has too few
// row blocks to give each CU two workgroups.
template <int RB, int MB, int XT, int IB1, bool RES, int KS>
__global__ __launch_bounds__(kThreads * KS) void gemm8_kernel(ProductArgs a) {
  constexpr int BN = 32 * RB;
  constexpr int MC = 32 * MB;
  constexpr int kTiles = XT == 1 ? 2 : 1;
  constexpr int kSlots = BN * 8 / kThreads;            // vector slots per thread per K-tile (1 or 2)
  constexpr int kXChunks = MC * (kBK8 / 8) / kThreads;  // 16-byte x chunks per thread per K-tile
  constexpr int kGroups = 4 / RB;                       // wavefronts of a stream sharing a row block
  constexpr int kAcc = (MB + kGroups - 1) / kGroups;    // 32x32 batch blocks per wavefront
  constexpr bool kLds1 = IB1 != 16;
  constexpr int kStreamHalves = (kTiles * BN + MC) * kLd8;  // LDS tiles of one stream
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int tid_all = threadIdx.x;
  const int stream = tid_all / kThreads;
  const int tid = tid_all % kThreads;
  uint16_t* wt = smem + stream * kStreamHalves;         // [kTiles][BN][kLd8]
  uint16_t* xt = wt + kTiles * BN * kLd8;               // [MC][kLd8]
  uint32_t* idx_lds = (uint32_t*)(smem + KS * kStreamHalves);  // [2][BN][row_words]
  const int w1 = 2 * a.bits1, w2 = RES ? 2 * a.bits2 : 0;
  const int row_words = w1 + 1 + (RES ? w2 + 1 : 0);
  uint4* books = (uint4*)(idx_lds + 2 * BN * row_words + 2 * BN);  // [K1 if LDS][K2], 16-byte aligned start
  const int k1 = kLds1 ? (1 << a.bits1) : 0;
  const int k2 = RES ? (1 << a.bits2) : 0;
  for (int e = tid_all; e < k1 + k2; e += kThreads * KS)
    books[e] = e < k1 ? *(const uint4*)(a.cb1 + (size_t)e * 8) : *(const uint4*)(a.cb2 + (size_t)(e - k1) * 8);
  const uint4* book1 = books;
  const uint4* book2 = books + k1;

  const int lane = tid & 63;
  const int wave = tid >> 6;  // wavefront within the stream
  const int row0 = blockIdx.x * BN;
  const int ntiles = (a.in_features + kBK8 - 1) / kBK8;
  const int nsuper = (ntiles + kSuper - 1) / kSuper;

  // Super-tile staging (all streams together): 16-byte chunks of the index rows (bits
  // are even, so a super-tile starts on a 16-byte boundary); chunks past the stored row
  // read as zero.
  const int c1_per_row = a.bits1 / 2, c2_per_row = RES ? a.bits2 / 2 : 0;
  const int chunks_per_row = c1_per_row + c2_per_row;
  const int total_chunks = BN * chunks_per_row;  // at most 64 * 14 = 896
  constexpr int kIdxChunks = 4 / KS;
  uint4 iq[kIdxChunks];
  auto load_super = [&](int sidx) {
#pragma unroll
    for (int c = 0; c < kIdxChunks; ++c) {
      const int ch = tid_all + c * kThreads * KS;
      const int r = ch / max(chunks_per_row, 1);
      const int q = ch - r * chunks_per_row;
      const int row = min(row0 + r, a.n - 1);
      const bool second = q >= c1_per_row;
      const uint32_t* base = second ? a.packed2 + (size_t)row * a.s2_words : a.packed1 + (size_t)row * a.s1_words;
      const int words = second ? a.s2_words : a.s1_words;
      const int wd = (second ? sidx * w2 + (q - c1_per_row) * 4 : sidx * w1 + q * 4);
      const int wd_c = min(wd, words - 4);
      iq[c] = *(const uint4*)(base + wd_c);
      if (ch >= total_chunks || wd >= words || row0 + r >= a.n) iq[c] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_super = [&](int buf) {
#pragma unroll
    for (int c = 0; c < kIdxChunks; ++c) {
      const int ch = tid_all + c * kThreads * KS;
      if (ch < total_chunks) {
        const int r = ch / chunks_per_row;
        const int q = ch - r * chunks_per_row;
        uint32_t* dst = idx_lds + (buf * BN + r) * row_words + (q >= c1_per_row ? w1 + 1 + (q - c1_per_row) * 4 : q * 4);
        dst[0] = iq[c].x; dst[1] = iq[c].y; dst[2] = iq[c].z; dst[3] = iq[c].w;
      }
    }
  };

  // per-thread slot coordinates
  int srow[kSlots], sjl[kSlots];
  bool srow_ok[kSlots];
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    const int sl = tid + i * kThreads;
    srow[i] = sl >> 3;
    sjl[i] = sl & 7;
    srow_ok[i] = row0 + srow[i] < a.n;
  }

  // Two register sets per stream: its next two tiles are in flight while one is written
  // and multiplied.
  struct Stage {
    uint4 c1[kSlots], c2[kSlots], xq[kXChunks];
  };
  Stage st0, st1;
  auto issue = [&](int t, Stage& sg) {
    const int buf = (t / kSuper) & 1;
    const int tin = t % kSuper;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      const uint32_t* irow = idx_lds + (buf * BN + srow[i]) * row_words;
      const uint32_t jj = (uint32_t)(tin * 8 + sjl[i]);
      const uint32_t i1 = lds_index<IB1>(irow, jj, a.bits1);
      if constexpr (kLds1) {
        sg.c1[i] = book1[i1];
      } else {
        sg.c1[i] = *(const uint4*)(a.cb1 + (size_t)i1 * 8);
      }
      if constexpr (RES) sg.c2[i] = book2[lds_index<0>(irow + w1 + 1, jj, a.bits2)];
    }
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
      const int ch = tid + c * kThreads;
      const int m = ch >> 3;
      const int k = t * kBK8 + (ch & 7) * 8;
      const int mm = min(m, a.m - 1);
      const int kk = min(k, a.in_features - 8);
      sg.xq[c] = *(const uint4*)(a.x + (size_t)mm * a.in_features + kk);
      if (m >= a.m || k >= a.in_features) sg.xq[c] = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  float16_t acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  if (ntiles > 0) {
    load_super(0);
    store_super(0);
  }
  __syncthreads();  // books and the first index super-tile staged
  // stream s takes tiles s, s + KS, s + 2*KS, ...; step k covers tiles k*KS .. k*KS + KS - 1
  const int nsteps = (ntiles + KS - 1) / KS;
  constexpr int kStepsPerSuper = kSuper / KS;
  if (stream < ntiles) issue(stream, st0);
  if (KS + stream < ntiles) issue(KS + stream, st1);
  if (nsuper > 1) load_super(1);
  const int rb = wave % RB;
  const int mg = wave / RB;
  const int ar = lane & 31;
  const int kh = (lane >> 5) * 8;
  // one pipeline step: write this stream's tile of step k from `sg`, then refill `sg`
  // with its tile of step k+2 and run the MFMAs of the written tile
  auto step = [&](int k, Stage& sg) {
    const int t = k * KS + stream;
    const bool mine = t < ntiles;
    __syncthreads();  // the previous step's MFMAs are done with the LDS tiles
    if (mine) {
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const bool live = srow_ok[i] && (t * 8 + sjl[i]) < a.nv;
        uint32_t hi_w[4], lo_w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float w0 = h_at(sg.c1[i], 2 * p), w1v = h_at(sg.c1[i], 2 * p + 1);
          if constexpr (RES) {
            w0 = w0 + h_at(sg.c2[i], 2 * p);
            w1v = w1v + h_at(sg.c2[i], 2 * p + 1);
          }
          w0 = live ? w0 : 0.0f;
          w1v = live ? w1v : 0.0f;
          if constexpr (XT == 0) {
            hi_w[p] = (uint32_t)vqd::f32_to_f16_rne(w0) | ((uint32_t)vqd::f32_to_f16_rne(w1v) << 16);
            lo_w[p] = 0u;
          } else {
            // hi = nearest bf16 pair (one v_cvt_pk_bf16_f32), lo = bf16 of the exact fp32 remainders
            const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){w0, w1v}, bf16x2_t));
            const float r0 = w0 - __builtin_bit_cast(float, hb << 16);
            const float r1 = w1v - __builtin_bit_cast(float, hb & 0xFFFF0000u);
            hi_w[p] = hb;
            lo_w[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){r0, r1}, bf16x2_t));
          }
        }
        *(uint4*)(wt + srow[i] * kLd8 + sjl[i] * 8) = make_uint4(hi_w[0], hi_w[1], hi_w[2], hi_w[3]);
        if constexpr (XT == 1)
          *(uint4*)(wt + BN * kLd8 + srow[i] * kLd8 + sjl[i] * 8) = make_uint4(lo_w[0], lo_w[1], lo_w[2], lo_w[3]);
      }
#pragma unroll
      for (int c = 0; c < kXChunks; ++c) {
        const int ch = tid + c * kThreads;
        *(uint4*)(xt + (ch >> 3) * kLd8 + (ch & 7) * 8) = sg.xq[c];
      }
    }
    // the index super-tile after the current one: stored mid-way, its loads long landed
    const int sidx = k / kStepsPerSuper;
    if (k % kStepsPerSuper == kStepsPerSuper / 2 && sidx + 1 < nsuper) store_super((sidx + 1) & 1);
    __syncthreads();  // tiles complete
    if (t + 2 * KS < ntiles) issue(t + 2 * KS, sg);  // two steps in flight during the MFMAs
    if ((k + 1) % kStepsPerSuper == 0 && (k + 1) / kStepsPerSuper + 1 < nsuper)
      load_super((k + 1) / kStepsPerSuper + 1);
    if (mine) {
#pragma unroll
      for (int ks = 0; ks < kBK8; ks += 16) {
        const uint4 aw = *(const uint4*)(wt + (rb * 32 + ar) * kLd8 + ks + kh);
        uint4 aw_lo = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (XT == 1) aw_lo = *(const uint4*)(wt + BN * kLd8 + (rb * 32 + ar) * kLd8 + ks + kh);
#pragma unroll
        for (int i = 0; i < kAcc; ++i) {
          const int mb = mg + kGroups * i;
          if (mb < MB) {
            const uint4 bw = *(const uint4*)(xt + (mb * 32 + ar) * kLd8 + ks + kh);
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
    }
  };
  for (int k = 0; k < nsteps; k += 2) {
    step(k, st0);
    if (k + 1 < nsteps) step(k + 1, st1);
  }
  if constexpr (KS > 1) {
    // add the other streams' partial sums into stream 0 through LDS (the tile area of
    // streams 1..KS-1 is free now)
    __syncthreads();
    float* red = (float*)(smem + kStreamHalves);
    if (stream > 0) {
#pragma unroll
      for (int i = 0; i < kAcc; ++i) {
        if (mg + kGroups * i < MB) {
          float* dst = red + (((stream - 1) * 4 + wave) * kAcc + i) * 16 * 64;
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[r * 64 + lane] = acc[i][r];
        }
      }
    }
    __syncthreads();
    if (stream > 0) return;
#pragma unroll
    for (int sidx = 1; sidx < KS; ++sidx) {
#pragma unroll
      for (int i = 0; i < kAcc; ++i) {
        if (mg + kGroups * i < MB) {
          const float* src = red + (((sidx - 1) * 4 + wave) * kAcc + i) * 16 * 64;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] += src[r * 64 + lane];
        }
      }
    }
  }
  // Epilogue: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4 of the block and
  // batch row l%32.
#pragma unroll
  for (int i = 0; i < kAcc; ++i) {
    const int mb = mg + kGroups * i;
    if (mb >= MB) continue;
    const int m = mb * 32 + (lane & 31);
    if (m >= a.m) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = row0 + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (n < a.n) {
        float out = acc[i][r];
        if (a.scale) out = out * vqd::f16_to_f32(a.scale[n]);
        if (a.bias) out = out + vqd::f16_to_f32(a.bias[n]);
        vqd::store_out(a.y, (size_t)m * a.n + n, out, a.y_dtype);
      }
    }
  }
}

template <int RB, int MB, int XT, int IB1, bool RES, int KS>
vq_status launch_gemm8(const ProductArgs& a, hipStream_t s) {
  auto kern = gemm8_kernel<RB, MB, XT, IB1, RES, KS>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return VQ_ERR_HIP;
  constexpr int kTilesW = XT == 1 ? 2 : 1;
  const size_t k1 = IB1 != 16 ? ((size_t)1 << a.bits1) : 0;
  const size_t k2 = RES ? ((size_t)1 << a.bits2) : 0;
  const int row_words = 2 * a.bits1 + 1 + (RES ? 2 * a.bits2 + 1 : 0);
  size_t lds = (size_t)KS * (kTilesW * 32 * RB + 32 * MB) * kLd8 * 2 +
               4 * (size_t)(2 * 32 * RB * row_words + 2 * 32 * RB);
  lds = (lds + 15) & ~(size_t)15;
  lds += 16 * (k1 + k2);
  const unsigned grid = (unsigned)((a.n + 32 * RB - 1) / (32 * RB));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads * KS), lds, s, a);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

// Partial sums of the extra streams fit in the tile area they leave behind.
template <int RB, int MB, int XT>
constexpr bool ks2_fits() {
  constexpr int kGroups = 4 / RB;
  constexpr int kAcc = (MB + kGroups - 1) / kGroups;
  constexpr int waves_with_blocks = MB < kGroups ? MB * RB : 4;
  constexpr int red_bytes = waves_with_blocks * kAcc * 16 * 64 * 4;
  constexpr int stream_bytes = ((XT == 1 ? 2 : 1) * 32 * RB + 32 * MB) * kLd8 * 2;
  return red_bytes <= stream_bytes;
}

template <int RB, int MB, int XT, int IB1, bool RES>
vq_status gemm8_ks(const ProductArgs& a, hipStream_t s) {
  // at most one row block per CU: two K-streams per workgroup keep more loads in flight
  const long blocks = (a.n + 32 * RB - 1) / (32 * RB);
  if constexpr (ks2_fits<RB, MB, XT>()) {
    if (blocks <= kNumCUs) return launch_gemm8<RB, MB, XT, IB1, RES, 2>(a, s);
  }
  return launch_gemm8<RB, MB, XT, IB1, RES, 1>(a, s);
}

template <int RB, int XT, int IB1, bool RES>
vq_status gemm8_mb(const ProductArgs& a, hipStream_t s) {
  const int mb = (a.m + 31) / 32;
  if (mb <= 1) return gemm8_ks<RB, 1, XT, IB1, RES>(a, s);
  if (mb <= 2) return gemm8_ks<RB, 2, XT, IB1, RES>(a, s);
  if (mb <= 4) return gemm8_ks<RB, 4, XT, IB1, RES>(a, s);
  return gemm8_ks<RB, 8, XT, IB1, RES>(a, s);
}

template <int XT, int IB1, bool RES>
vq_status gemm8_rb(const ProductArgs& a, hipStream_t s) {
  // 64-row blocks when there are enough rows to give every CU work, else 32-row blocks
  return a.n >= 64 * 320 ? gemm8_mb<2, XT, IB1, RES>(a, s) : gemm8_mb<1, XT, IB1, RES>(a, s);
}

template <int XT>
vq_status gemm8_books(const ProductArgs& a, hipStream_t s) {
  const bool main16 = a.bits1 == 16;
  if (a.bits2) return main16 ? gemm8_rb<XT, 16, true>(a, s) : gemm8_rb<XT, 0, true>(a, s);
  return main16 ? gemm8_rb<XT, 16, false>(a, s) : gemm8_rb<XT, 0, false>(a, s);
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
    const bool fast8 = v == 8 && (a.bits1 == 16 || a.bits1 <= 12) && a.bits2 <= 12 && a.bits1 % 2 == 0 &&
                       a.bits2 % 2 == 0 && a.in_features >= 8 && aligned(a.packed1, 16) &&
                       a.in_features % 8 == 0 && g.x_vec && fast_v == 8 &&
                       (a.bits1 == 16 ? 0 : (16u << a.bits1)) + (a.bits2 ? (16u << a.bits2) : 0) <= 64 * 1024;
    if (fast8) {
      st = a.x_dtype == VQ_BF16 ? gemm8_books<1>(a, s) : gemm8_books<0>(a, s);
    } else if (fast_v == 8) {
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
