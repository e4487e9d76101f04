// vq_gemv for a 65536-entry main codebook (v = 8, 16-bit indices), 1 <= M <= 16: the
// codebook-sliced kernel, used by vq_gemv_ws.
//
// Random 16-byte lookups into a 1 MiB book are served by L2 at well under one per clock
// per CU (the production-VQ post, "Lookup Table (LUT) Overhead vs. Bit-Shifting", warns
// that lookups spilling out of fast memory eat the bandwidth savings), while LDS returns
// a 64-lane 16-byte read every ~5 clocks.  So the book is cut into S = 8 slices of 8192
// centroids (128 KiB) and each workgroup keeps one slice in LDS:
//   - 256 persistent workgroups, one per CU: workgroup (slice s, group p).  The 8 slice
//     workgroups of a group are launched onto one XCD and walk the same tiles in the
//     same order, so a tile's index lines come from HBM once and from that XCD's L2
//     seven more times;
//   - a tile is 128 rows x a range of 256-vector chunks; each group takes every 32nd
//     tile; inside a tile the chunks are walked in order;
//   - wavefront w owns column block w (32 of a chunk's 256 vectors) and all 128 rows;
//     a lane is one (row, 8-vector group) of a v_mfma_f32_16x16x32_f16: for each of its
//     8 vectors the lane reads its centroid from the LDS slice if the index falls in
//     slice s and a zero centroid otherwise (a select, no branch), and the matrix core
//     forms the 16 rows' dot products with x, batch row m in output column m.  The 8
//     row groups of the tile keep their accumulators in registers across the chunks;
//   - the residual centroids of the tile's row group s are added by slice workgroup s;
//   - a chunk's activations are loaded one chunk ahead, and each row group's index words
//     for the next chunk are loaded right after the row group is used;
//   - at the end of a tile the 8 column blocks are added in LDS and the workgroup stores
//     one fp32 partial sum per (row, batch row) into the caller's workspace;
//   - a second kernel adds the 8 x (column splits) partials of each output in a fixed
//     order and applies the channel scale and bias, so results do not depend on
//     scheduling.
// bf16 activations are first rewritten as fp16 times a power of two per batch row (a
// small pass over x): exact for every bf16 value from 2^-16 to 65504 times that power.
#include "vq_device.h"

namespace {

using vqi::ProductArgs;

constexpr int kThreads = 512;            // 8 wavefronts, one per column block
constexpr int kSliceBits = 13;
constexpr int kSlice = 1 << kSliceBits;  // centroids per slice
constexpr int kSlices = 8;
constexpr int kChunk = 256;              // vectors per chunk: 8 column blocks of 32
constexpr int kGroups = 32;              // workgroup groups: 8 x 32 = 256 workgroups
constexpr int kRes = 256;                // residual centroids (8-bit indices)
constexpr int kRT = 128;                 // rows per tile
constexpr int kRG = kRT / 16;            // 16-row groups per tile
constexpr int kRedFloats = 8 * 16 * 16;  // column-block sums of one row group, M <= 16

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct SlicedCfg {
  int32_t n_rb;         // row blocks of kRT rows
  int32_t n_chunks;     // 256-vector chunks per row
  int32_t n_cs;         // column splits
  int32_t cpc;          // chunks per column split
  int32_t groups;       // workgroup groups in use
  float* part;          // [8 * n_cs][M][N] partial sums
  const uint16_t* x16;  // fp16 activations [M][IN]
  const int32_t* xexp;  // [M] power of two taken out of each bf16 row, or nullptr
};

__device__ __forceinline__ float4_t mfma16(const uint4& a, const uint4& b, const float4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}

// LDS byte offsets of the centroids of 8 consecutive 16-bit indices: index XOR
// (s << 13) is below 8192 exactly when the centroid lives in slice s; anything else
// clamps to entry 8192, the zero centroid.  Per two indices: one XOR, one packed min and
// two shifts that read one 16-bit half each (SDWA word select), four VALU in all.
__device__ __forceinline__ void slice_addrs(const uint4& w, uint32_t tag, uint32_t (&ad)[8]) {
  const uint32_t wd[4] = {w.x ^ tag, w.y ^ tag, w.z ^ tag, w.w ^ tag};
  const u16x2 lim = {(unsigned short)kSlice, (unsigned short)kSlice};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t v = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, wd[h]), lim));
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
        : "=v"(ad[2 * h]) : "v"(v));
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(ad[2 * h + 1]) : "v"(v));
  }
}

template <bool RES>
__global__ __launch_bounds__(kThreads) void gemv_sliced_kernel(ProductArgs a, SlicedCfg g) {
  // static LDS: the slice's base address is fixed when compiling, so a centroid read needs
  // no base add on top of index * 16
  __shared__ uint4 slice[kSlice + 1];
  __shared__ uint4 resb[RES ? kRes + 1 : 1];
  __shared__ float red[kRedFloats];

  const int tid = threadIdx.x;
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int s = rest & 7;
  const int grp = (rest >> 3) * 8 + xcd;
  if (grp >= g.groups) return;  // the whole workgroup leaves before any barrier

  const int lane = tid & 63;
  const int cb = tid >> 6;  // column block = wavefront
  const int g4 = lane >> 4;
  const int r16 = lane & 15;
  const int M = a.m, N = a.n, nv = a.nv;
  const int U = g.n_rb * g.n_cs;
  const uint32_t tag = ((uint32_t)s << kSliceBits) * 0x10001u;
  const uint32_t s1b = (uint32_t)a.s1_words * 4u;
  const uint32_t s2b = (uint32_t)a.s2_words * 4u;
  const char* p1 = (const char*)a.packed1;
  const char* p2 = (const char*)a.packed2;
  const char* xbase = (const char*)g.x16;
  const uint32_t lane_col = (uint32_t)(cb * 32 + g4 * 8);  // the lane's first vector within a chunk

  // current tile u (row block rbk, column split cs) and chunk c
  int u = grp, rbk = u / g.n_cs, cs = u - rbk * g.n_cs;
  int c = cs * g.cpc, cend = min(c + g.cpc, g.n_chunks);
  // prefetch cursor: the chunk after the current one (possibly in the next tile); past
  // the last tile it stays on a valid chunk, so the extra loads read real memory
  int pu = u, prb = rbk, pc = c, pcend = cend;
  auto adv_pre = [&]() __attribute__((always_inline)) {
    if (++pc >= pcend) {
      pu += g.groups;
      if (pu < U) {
        prb = pu / g.n_cs;
        const int pcs = pu - prb * g.n_cs;
        pc = pcs * g.cpc;
        pcend = min(pc + g.cpc, g.n_chunks);
      } else {
        pc = pcend - 1;
      }
    }
  };
  // byte offsets of the lane's index words for row group q of row block rb, chunk cc
  // (rows past N read row N - 1; vectors past the row end read chunk 0 or vector nv - 1)
  auto idx_off = [&](int rb, int cc, int q) __attribute__((always_inline)) -> uint32_t {
    const int row = min(rb * kRT + q * 16 + r16, N - 1);
    const uint32_t j0 = (uint32_t)cc * kChunk + lane_col;
    const uint32_t c16 = j0 < (uint32_t)nv ? (j0 >> 3) : 0u;
    return (uint32_t)row * s1b + c16 * 16u;
  };
  // byte offset of the lane's 8 residual indices (row group s of row block rb, chunk cc)
  auto res_off = [&](int rb, int cc) __attribute__((always_inline)) -> uint32_t {
    const int row = min(rb * kRT + s * 16 + r16, N - 1);
    const uint32_t j0 = (uint32_t)cc * kChunk + lane_col;
    return (uint32_t)row * s2b + (j0 < (uint32_t)nv ? j0 : 0u);
  };
  // activations of the lane's 8 vectors; lanes of batch rows >= M load row M - 1 (they
  // feed output columns that are dropped)
  auto load_x = [&](int cc, uint4 (&xr)[8]) __attribute__((always_inline)) {
    const uint32_t j0 = (uint32_t)cc * kChunk + lane_col;
    const char* row = xbase + (size_t)min(r16, M - 1) * a.in_features * 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) xr[k] = *(const uint4*)(row + (size_t)min(j0 + k, (uint32_t)nv - 1u) * 16u);
  };

  uint4 iw[kRG];  // index words of the current chunk, one per row group
  uint2 ir = make_uint2(0u, 0u);  // residual indices of row group s, one byte per vector
  uint4 xa[8], xb[8];

  // stage the slice (and the residual book): the 16 loads per thread first, then the
  // first chunk's indices and activations, then the LDS writes
  {
    const u32x4* src = (const u32x4*)a.cb1 + (size_t)s * kSlice + tid;
    u32x4* dst = (u32x4*)slice + tid;
    static_assert(kSlice / kThreads == 16, "sixteen staging loads per thread");
    u32x4 q0 = src[0 * kThreads], q1 = src[1 * kThreads], q2 = src[2 * kThreads], q3 = src[3 * kThreads],
          q4 = src[4 * kThreads], q5 = src[5 * kThreads], q6 = src[6 * kThreads], q7 = src[7 * kThreads],
          q8 = src[8 * kThreads], q9 = src[9 * kThreads], q10 = src[10 * kThreads], q11 = src[11 * kThreads],
          q12 = src[12 * kThreads], q13 = src[13 * kThreads], q14 = src[14 * kThreads], q15 = src[15 * kThreads];
    u32x4 qr = {0u, 0u, 0u, 0u};
    if (RES && tid < kRes) qr = ((const u32x4*)a.cb2)[tid];
#pragma unroll
    for (int q = 0; q < kRG; ++q) iw[q] = *(const uint4*)(p1 + idx_off(rbk, c, q));
    if constexpr (RES) ir = *(const uint2*)(p2 + res_off(rbk, c));
    load_x(c, xa);
    dst[0 * kThreads] = q0;
    dst[1 * kThreads] = q1;
    dst[2 * kThreads] = q2;
    dst[3 * kThreads] = q3;
    dst[4 * kThreads] = q4;
    dst[5 * kThreads] = q5;
    dst[6 * kThreads] = q6;
    dst[7 * kThreads] = q7;
    dst[8 * kThreads] = q8;
    dst[9 * kThreads] = q9;
    dst[10 * kThreads] = q10;
    dst[11 * kThreads] = q11;
    dst[12 * kThreads] = q12;
    dst[13 * kThreads] = q13;
    dst[14 * kThreads] = q14;
    dst[15 * kThreads] = q15;
    if (tid == 0) slice[kSlice] = make_uint4(0u, 0u, 0u, 0u);
    if (RES && tid <= kRes) ((u32x4*)resb)[tid] = qr;  // entry kRes stays zero
  }
  adv_pre();
  __syncthreads();

  float4_t d[kRG];
#pragma unroll
  for (int q = 0; q < kRG; ++q) d[q] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // One chunk: the next chunk's activations first, then per row group the centroid
  // reads (those of row group q + 1 are issued before the products of row group q), the
  // refill of the row group's index slot with the next chunk, and the 8 products; row
  // group s also takes the 8 residual centroids.  In the ragged last chunk of a row the
  // vectors past its end get zero x and an index outside every slice (bit 13 set after
  // the slice XOR), so they read the zero centroid; this fix-up is a uniform branch.
  auto chunk = [&](uint4 (&xr)[8], uint4 (&xn)[8]) __attribute__((always_inline)) {
    load_x(pc, xn);
    const int nvalid = nv - (c * kChunk + (int)lane_col);
    uint32_t rmask = 0u;  // residual slots past the row end
    if ((c + 1) * kChunk > nv) {
      // a 16-bit index (s ^ 7) << 13 gives 0xE000 after the slice XOR: the zero centroid
      const uint32_t fill = ((uint32_t)(s ^ 7) << 13) * 0x10001u;
      uint32_t keep[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) keep[h] = (2 * h < nvalid ? 0xFFFFu : 0u) | (2 * h + 1 < nvalid ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int q = 0; q < kRG; ++q) {
        iw[q].x = (iw[q].x & keep[0]) | (fill & ~keep[0]);
        iw[q].y = (iw[q].y & keep[1]) | (fill & ~keep[1]);
        iw[q].z = (iw[q].z & keep[2]) | (fill & ~keep[2]);
        iw[q].w = (iw[q].w & keep[3]) | (fill & ~keep[3]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) xr[k] = k < nvalid ? xr[k] : make_uint4(0u, 0u, 0u, 0u);
      rmask = nvalid >= 8 ? 0u : (nvalid > 0 ? 0xFFu & ~((1u << nvalid) - 1u) : 0xFFu);
    }
    uint4 cv[2][8];
    auto reads = [&](int q, uint4 (&c8)[8]) __attribute__((always_inline)) {
      uint32_t ad[8];
      slice_addrs(iw[q], tag, ad);
#pragma unroll
      for (int k = 0; k < 8; ++k) c8[k] = *(const uint4*)((const char*)slice + ad[k]);
    };
    reads(0, cv[0]);
#pragma unroll
    for (int q = 0; q < kRG; ++q) {
      if (q + 1 < kRG) reads(q + 1, cv[(q + 1) & 1]);
      iw[q] = *(const uint4*)(p1 + idx_off(prb, pc, q));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 8; ++k) d[q] = mfma16(cv[q & 1][k], xr[k], d[q]);
      if constexpr (RES) {
        if (q == s) {  // uniform: this slice's residual row group
          const uint32_t rw[2] = {ir.x, ir.y};
          uint4 cr[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const uint32_t e = (rw[k >> 2] >> (8 * (k & 3))) & 0xFFu;
            cr[k] = resb[(rmask >> k) & 1u ? (uint32_t)kRes : e];
          }
          ir = *(const uint2*)(p2 + res_off(prb, pc));
#pragma unroll
          for (int k = 0; k < 8; ++k) d[q] = mfma16(cr[k], xr[k], d[q]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    adv_pre();
  };

  // End of a tile: per row group, the 8 column blocks are added in LDS (fixed order) and
  // one partial per (row, batch row) goes to the workspace.  Lane l of a wavefront holds
  // rows 4 * (l / 16) + r of output column l % 16 in register r.
  auto tile_end = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kRG; ++q) {
      if (r16 < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(cb * 16 + 4 * g4 + r) * M + r16] = d[q][r];
      }
      __syncthreads();
      if (tid < 16 * M) {
        const int m = tid / 16;
        const int rl = tid - m * 16;
        float v = 0.0f;
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) v += red[(c2 * 16 + rl) * M + m];
        const int row = rbk * kRT + q * 16 + rl;
        if (row < N) g.part[((size_t)(cs * kSlices + s) * M + m) * N + row] = v;
      }
      __syncthreads();
      d[q] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };

  auto next = [&]() __attribute__((always_inline)) -> bool {
    if (++c >= cend) {
      tile_end();
      u += g.groups;
      if (u >= U) return false;
      rbk = u / g.n_cs;
      cs = u - rbk * g.n_cs;
      c = cs * g.cpc;
      cend = min(c + g.cpc, g.n_chunks);
    }
    return true;
  };

  for (;;) {  // activations alternate between two register sets
    chunk(xa, xb);
    if (!next()) break;
    chunk(xb, xa);
    if (!next()) break;
  }
}

// y[m][row] = scale[row] * 2^e[m] * (sum of the partials in a fixed order) + bias[row].
// The exponent, scale and bias are loaded beside the partials (a missing one reads a
// partial in its place, unused), so a thread waits for memory once.
__global__ __launch_bounds__(256) void gemv_sliced_finalize(ProductArgs a, const float* __restrict__ part,
                                                            const int32_t* __restrict__ xexp, int nparts) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= a.n * a.m) return;
  const int m = t / a.n;
  const int row = t - m * a.n;
  const float* p = part + (size_t)m * a.n + row;
  const size_t stride = (size_t)a.m * a.n;
  const int32_t e = *(xexp ? xexp + m : (const int32_t*)p);
  const uint16_t sc = *(a.scale ? a.scale + row : (const uint16_t*)p);
  const uint16_t bi = *(a.bias ? a.bias + row : (const uint16_t*)p);
  float acc = 0.0f;
  int q = 0;
  for (; q + 8 <= nparts; q += 8) {  // eight loads in flight, added in order
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[(size_t)(q + k) * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += v[k];
  }
  for (; q < nparts; ++q) acc += p[(size_t)q * stride];
  if (xexp) acc = ldexpf(acc, e);
  if (a.scale) acc = acc * vqd::f16_to_f32(sc);
  if (a.bias) acc = acc + vqd::f16_to_f32(bi);
  vqd::store_out(a.y, (size_t)m * a.n + row, acc, a.y_dtype);
}

// bf16 activations -> fp16 * 2^e, one workgroup per batch row: e is the smallest
// exponent >= 0 that brings max |x| below 2^15, so every finite value stays finite.
// Rows of up to 4 * 1024 * 8 values are read once into registers (all loads in flight
// together) and converted from there; longer rows are walked in passes of that size.
constexpr int kXprepHold = 4;  // 16-byte words per thread held in registers

__device__ __forceinline__ uint32_t xprep_absmax(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t mx = 0;
#pragma unroll
  for (int h = 0; h < 4; ++h) mx = max(mx, max(w[h] & 0x7FFFu, (w[h] >> 16) & 0x7FFFu));
  return mx;
}

__device__ __forceinline__ uint4 xprep_convert(const uint4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t lo = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w[h] & 0xFFFFu), -e));
    const uint32_t hi = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w[h] >> 16), -e));
    o[h] = lo | (hi << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ __launch_bounds__(1024) void xprep_kernel(const uint16_t* __restrict__ x, int in_features,
                                                     uint16_t* __restrict__ x16, int32_t* __restrict__ xexp) {
  __shared__ uint32_t wmax[16];
  const int m = blockIdx.x;
  const uint4* xr = (const uint4*)(x + (size_t)m * in_features);
  uint4* xo = (uint4*)(x16 + (size_t)m * in_features);
  const int n8 = in_features / 8;
  const int tid = threadIdx.x;
  // max of |x| as bits: orders like the values, NaN above infinity
  uint32_t mx = 0;
  uint4 held[kXprepHold];
#pragma unroll
  for (int k = 0; k < kXprepHold; ++k) held[k] = xr[min(tid + k * 1024, n8 - 1)];  // clamped: no branch
#pragma unroll
  for (int k = 0; k < kXprepHold; ++k) mx = max(mx, tid + k * 1024 < n8 ? xprep_absmax(held[k]) : 0u);
  for (int i = tid + kXprepHold * 1024; i < n8; i += 1024) mx = max(mx, xprep_absmax(xr[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  mx = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, wmax[i]);
  const int e = max(0, (int)((mx >> 7) & 0xFFu) - 127 - 14);
#pragma unroll
  for (int k = 0; k < kXprepHold; ++k) {
    const int i = tid + k * 1024;
    if (i < n8) xo[i] = xprep_convert(held[k], e);
  }
  for (int i = tid + kXprepHold * 1024; i < n8; i += 1024) xo[i] = xprep_convert(xr[i], e);
  if (tid == 0) xexp[m] = e;
}

struct Plan {
  SlicedCfg cfg;
  size_t part_off, x16_off, exp_off, bytes;
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Row blocks of 128 rows; the columns are split until every group has a tile (or the
// chunks run out).
Plan make_plan(int32_t n, int32_t in_features, int32_t m, bool bf16) {
  Plan p{};
  SlicedCfg& g = p.cfg;
  const int nv = in_features / 8;
  g.n_chunks = (nv + kChunk - 1) / kChunk;
  g.n_rb = (n + kRT - 1) / kRT;
  int n_cs = 1;
  while (g.n_rb * n_cs < kGroups && n_cs < g.n_chunks) n_cs *= 2;
  if (n_cs > g.n_chunks) n_cs = g.n_chunks;
  g.cpc = (g.n_chunks + n_cs - 1) / n_cs;
  g.n_cs = (g.n_chunks + g.cpc - 1) / g.cpc;
  const int units = g.n_rb * g.n_cs;
  g.groups = units < kGroups ? units : kGroups;
  p.part_off = 0;
  p.x16_off = round256((size_t)kSlices * g.n_cs * m * n * sizeof(float));
  p.exp_off = p.x16_off + (bf16 ? round256((size_t)m * in_features * 2) : 0);
  p.bytes = p.exp_off + (bf16 ? round256((size_t)m * sizeof(int32_t)) : 0);
  return p;
}


template <bool RES>
vq_status launch_res(const ProductArgs& a, const SlicedCfg& g, hipStream_t s) {
  auto kern = gemv_sliced_kernel<RES>;
  const unsigned grid = 64u * (unsigned)((g.groups + 7) / 8);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, a, g);
  if (hipGetLastError() != hipSuccess) return VQ_ERR_HIP;
  const int total = a.n * a.m;
  hipLaunchKernelGGL(gemv_sliced_finalize, dim3((total + 255) / 256), dim3(256), 0, s, a, (const float*)g.part, g.xexp,
                     kSlices * g.n_cs);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace

namespace vqi {

bool sliced_gemv_shape_ok(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (d.v != 8 || d.bits1 != 16 || !(d.bits2 == 0 || d.bits2 == 8)) return false;
  if (m < 1 || m > 16 || !(x_dtype == VQ_F16 || x_dtype == VQ_BF16)) return false;
  if (d.in_features % 8 != 0 || d.out_features < 1) return false;
  // Filling 256 LDS slices costs a few microseconds per call: below about four million
  // vectors the L2-gather kernel is as fast up to M = 4.  From M = 8 the slices win from
  // half a million vectors, since one matrix instruction serves every batch row.
  const int64_t vectors = (int64_t)d.out_features * (d.in_features / 8);
  return vectors >= ((int64_t)1 << (m >= 8 ? 19 : 22));
}

size_t sliced_gemv_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (!sliced_gemv_shape_ok(d, m, x_dtype)) return 0;
  return make_plan(d.out_features, d.in_features, m, x_dtype == VQ_BF16).bytes;
}

bool sliced_gemv_pointers_ok(const ProductArgs& a) {
  return aligned(a.packed1, 16) && aligned(a.cb1, 16) && (a.bits2 == 0 || aligned(a.cb2, 16)) && aligned(a.x, 16);
}

vq_status launch_gemv_sliced(const ProductArgs& a, void* workspace, void* stream) {
  // the kernels store partial sums into the workspace: never launch without one
  if (!workspace) return VQ_ERR_NULL;
  const bool bf16 = a.x_dtype == VQ_BF16;
  Plan p = make_plan(a.n, a.in_features, a.m, bf16);
  char* ws = (char*)workspace;
  p.cfg.part = (float*)(ws + p.part_off);
  hipStream_t s = (hipStream_t)stream;
  if (bf16) {
    uint16_t* x16 = (uint16_t*)(ws + p.x16_off);
    int32_t* xexp = (int32_t*)(ws + p.exp_off);
    hipLaunchKernelGGL(xprep_kernel, dim3(a.m), dim3(1024), 0, s, a.x, a.in_features, x16, xexp);
    if (hipGetLastError() != hipSuccess) return VQ_ERR_HIP;
    p.cfg.x16 = x16;
    p.cfg.xexp = xexp;
  } else {
    p.cfg.x16 = a.x;
    p.cfg.xexp = nullptr;
  }
  return a.bits2 == 8 ? launch_res<true>(a, p.cfg, s) : launch_res<false>(a, p.cfg, s);
}

}  // namespace vqi
