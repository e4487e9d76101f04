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
// small pass over x), chosen from the row's largest magnitude: exact for every value down
// to 2^-31 of that magnitude, whether the row is large, small or in between.
#include <atomic>

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
constexpr int kRedFloats = 8 * 16 * 16;  // column-block sums of one row group (M <= 16), or of
                                         // all 8 row groups for M <= 2

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
  int32_t* xexp_out;    // M <= 2, bf16: where the product kernel writes those powers
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

// The same for 4 indices in two words.
__device__ __forceinline__ void slice_addrs4(uint32_t w0, uint32_t w1, uint32_t tag, uint32_t (&ad)[4]) {
  const uint32_t wd[2] = {w0 ^ tag, w1 ^ tag};
  const u16x2 lim = {(unsigned short)kSlice, (unsigned short)kSlice};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t v = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, wd[h]), lim));
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
        : "=v"(ad[2 * h]) : "v"(v));
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(ad[2 * h + 1]) : "v"(v));
  }
}

// Raw buffer resource over n bytes at p (stride 0).  A buffer load returns zero for every
// dword that does not lie wholly inside the n bytes (the vector, scalar and instruction
// offsets all counted) and reads no memory for it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

// LDS layout (one array, fixed at compile time): the residual book (256 entries and a zero
// entry) first, so a residual read needs no base; then the slice (8192 entries and the
// zero centroid), whose base fits the 16-bit offset field of ds_read_b128; then the
// reduction area.
template <bool RES, bool SM>
struct SlicedLds {
  static constexpr int kResEntries = RES ? kRes + 1 : 0;
  static constexpr int kSliceAt = kResEntries;              // in 16-byte entries
  static constexpr int kRedAt = kSliceAt + kSlice + 1;
  static constexpr int kXAt = kRedAt + kRedFloats / 4;
  // M <= 2: each wavefront's activations, [wave][2 buffers][2 batch rows][32 vectors]
  static constexpr int kEntries = kXAt + (SM ? 8 * 2 * 2 * 32 : 0);
};

// SM: M <= 2, where every row group's column-block sums fit the reduction area at once and
// the activations go through LDS: each wavefront loads its 32 vectors of x (8 bytes per
// lane per batch row), converts bf16 to fp16 times 2^-e itself (e from the row's largest
// magnitude, found by every workgroup at the start), and reads its MFMA operands back
// from LDS; no separate pass over x.  Larger M reads fp16 x (converted by xprep_kernel for
// bf16) straight into registers, one chunk ahead.
template <bool RES, bool SM>
__global__ __launch_bounds__(kThreads) void gemv_sliced_kernel(ProductArgs a, SlicedCfg g) {
  using L = SlicedLds<RES, SM>;
  __shared__ uint4 lds[L::kEntries];
  uint4* const slice = lds + L::kSliceAt;
  float* const red = (float*)(lds + L::kRedAt);
  uint4* const xs = lds + L::kXAt;

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
  const uint32_t lane_col = (uint32_t)(cb * 32 + g4 * 8);  // the lane's first vector within a chunk
  // One buffer per stream: rows past N and vectors past the end of the last row read as
  // zero.  The lane's part of every offset is fixed; the rest (row block, row group, chunk)
  // is uniform and goes in the scalar offset.
  const __amdgpu_buffer_rsrc_t b1 = span(a.packed1, (uint32_t)N * s1b);
  const __amdgpu_buffer_rsrc_t b2 = span(RES ? (const void*)a.packed2 : (const void*)a.packed1,
                                         RES ? (uint32_t)N * s2b : 0u);
  const __amdgpu_buffer_rsrc_t bx = span(SM ? (const void*)a.x : (const void*)g.x16,
                                         (uint32_t)M * (uint32_t)a.in_features * 2u);
  const uint32_t v_idx = (uint32_t)r16 * s1b + lane_col * 2u;
  const uint32_t v_res = (uint32_t)r16 * s2b + lane_col;
  const uint32_t v_x = (uint32_t)min(r16, M - 1) * (uint32_t)a.in_features * 2u + lane_col * 16u;
  // M <= 2: lane l stages half l & 1 (4 values) of vector l >> 1 of the wavefront's 32
  const uint32_t v_xs = (uint32_t)(cb * 32 + (lane >> 1)) * 16u + (uint32_t)(lane & 1) * 8u;
  const bool xbf16 = a.x_dtype == VQ_BF16;

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
  // index words of row group q of row block rb, chunk cc; the lane's 8 residual indices
  // (row group s); the activations of the lane's 8 vectors (lanes of batch rows >= M read
  // row M - 1: they feed output columns that are dropped)
  auto load_idx = [&](int rb, int cc, int q) __attribute__((always_inline)) -> uint4 {
    return ld16(b1, v_idx, (uint32_t)(rb * kRT + q * 16) * s1b + (uint32_t)cc * (kChunk * 2));
  };
  auto load_res = [&](int rb, int cc) __attribute__((always_inline)) -> uint2 {
    return ld8(b2, v_res, (uint32_t)(rb * kRT + s * 16) * s2b + (uint32_t)cc * kChunk);
  };
  auto load_x = [&](int cc, uint4 (&xr)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 8; ++k) xr[k] = ld16(bx, v_x + k * 16u, (uint32_t)cc * (kChunk * 16));
  };
  // M <= 2: raw activations of chunk cc (8 bytes per lane and batch row), and their
  // conversion into the wavefront's LDS buffer followed by the operand reads
  int xe[2] = {0, 0};  // power of two taken out of each bf16 batch row
  auto load_xraw = [&](int cc, uint2 (&xw)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      xw[m] = m < M ? ld8(bx, v_xs, (uint32_t)cc * (kChunk * 16) + (uint32_t)m * (uint32_t)a.in_features * 2u)
                    : make_uint2(0u, 0u);
    }
  };
  auto stage_x = [&](int buf, const uint2 (&xw)[2], uint4 (&xr)[8]) __attribute__((always_inline)) {
    char* wbase = (char*)(xs + (cb * 2 + buf) * 64);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint2 h = xw[m];
      if (xbf16) {
        const uint32_t w2[2] = {h.x, h.y};
        uint32_t o[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t lo = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w2[i] & 0xFFFFu), -xe[m]));
          const uint32_t hi = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w2[i] >> 16), -xe[m]));
          o[i] = lo | (hi << 16);
        }
        h = make_uint2(o[0], o[1]);
      }
      *(uint2*)(wbase + m * 512 + v_xs - (uint32_t)cb * 512u) = h;
    }
    const uint4* rbase = (const uint4*)(wbase + min(r16, M - 1) * 512) + g4 * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) xr[k] = rbase[k];
  };

  uint4 iw[kRG];  // index words of the current chunk, one per row group
  uint2 ir = make_uint2(0u, 0u);  // residual indices of row group s, one byte per vector
  uint4 xa[8], xb[8];
  uint2 xw[2];    // M <= 2: raw activations of the next chunk

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
    for (int q = 0; q < kRG; ++q) iw[q] = load_idx(rbk, c, q);
    if constexpr (RES) ir = load_res(rbk, c);
    if constexpr (SM) {
      load_xraw(c, xw);
    } else {
      load_x(c, xa);
    }
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
    if (RES && tid <= kRes) ((u32x4*)lds)[tid] = qr;  // entry kRes stays zero
  }
  if constexpr (SM) {
    // largest |x| of each bf16 batch row (as bits: they order like the values), reduced
    // over the workgroup; e puts it in [2^14, 2^15) after scaling by 2^-e
    if (xbf16) {
      const __amdgpu_buffer_rsrc_t bxr = span(a.x, (uint32_t)M * (uint32_t)a.in_features * 2u);
      const int n16 = a.in_features / 8;
      uint32_t mx[2] = {0u, 0u};
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m < M) {
          for (int i = tid; i < n16; i += kThreads) {
            const uint4 v = ld16(bxr, (uint32_t)i * 16u, (uint32_t)m * (uint32_t)a.in_features * 2u);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) mx[m] = max(mx[m], max(w4[h] & 0x7FFFu, (w4[h] >> 16) & 0x7FFFu));
          }
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) mx[m] = max(mx[m], (uint32_t)__shfl_xor((int)mx[m], off, 64));
        }
      }
      if (lane == 0) {
        ((uint32_t*)red)[cb] = mx[0];
        ((uint32_t*)red)[8 + cb] = mx[1];
      }
    }
  }
  adv_pre();
  __syncthreads();
  if constexpr (SM) {
    if (xbf16) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t mx = 0u;
#pragma unroll
        for (int w = 0; w < 8; ++w) mx = max(mx, ((const uint32_t*)red)[8 * m + w]);
        xe[m] = (int)((mx >> 7) & 0xFFu) - 127 - 14;
      }
      if (blockIdx.x == 0 && tid < M) g.xexp_out[tid] = xe[tid];
    }
    __syncthreads();  // the reduction area is reused at the first tile end
    stage_x(0, xw, xa);
  }

  float4_t d[kRG];
#pragma unroll
  for (int q = 0; q < kRG; ++q) d[q] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // One chunk: the next chunk's activations first, then per row group the centroid
  // reads (those of row group q + 1 are issued before the products of row group q), the
  // refill of the row group's index slot with the next chunk, and the 8 products; row
  // group s also takes the 8 residual centroids.  In the ragged last chunk of a row the
  // vectors past its end get zero x and an index outside every slice (bit 13 set after
  // the slice XOR), so they read the zero centroid; their residual centroids meet zero x.
  // This fix-up is a uniform branch.
  int xbuf = 0;  // M <= 2: the LDS buffer holding the current chunk's activations
  auto chunk = [&](uint4 (&xr)[8], uint4 (&xn)[8]) __attribute__((always_inline)) {
    if constexpr (SM) {
      load_xraw(pc, xw);
    } else {
      load_x(pc, xn);
    }
    const int nvalid = nv - (c * kChunk + (int)lane_col);
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
    }
    // 16 half steps: half h is row group h / 2, vectors 4 (h & 1) .. 4 (h & 1) + 3 of the
    // lane's 8.  The centroid reads of half h + 2 are issued before the products of half h;
    // three buffers of 4 centroids rotate.
    uint4 cv[3][4];
    auto reads = [&](int h, uint4 (&c4)[4]) __attribute__((always_inline)) {
      const uint4& w = iw[h >> 1];
      uint32_t ad[4];
      slice_addrs4((h & 1) ? w.z : w.x, (h & 1) ? w.w : w.y, tag, ad);
#pragma unroll
      for (int k = 0; k < 4; ++k) c4[k] = *(const uint4*)((const char*)slice + ad[k]);
    };
    reads(0, cv[0]);
    reads(1, cv[1]);
#pragma unroll
    for (int h = 0; h < 2 * kRG; ++h) {
      const int q = h >> 1;
      if (h + 2 < 2 * kRG) reads(h + 2, cv[(h + 2) % 3]);
      if (h & 1) iw[q] = load_idx(prb, pc, q);  // both halves of row group q have been read
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) d[q] = mfma16(cv[h % 3][k], xr[4 * (h & 1) + k], d[q]);
      if constexpr (RES) {
        if ((h & 1) && q == s) {  // uniform: this slice's residual row group
          // byte k of the residual words, times 16: the entry's LDS address (the book is
          // at address 0), one SDWA shift each
          uint32_t ra[8];
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
              : "=v"(ra[0]) : "v"(ir.x));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
              : "=v"(ra[1]) : "v"(ir.x));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
              : "=v"(ra[2]) : "v"(ir.x));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
              : "=v"(ra[3]) : "v"(ir.x));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
              : "=v"(ra[4]) : "v"(ir.y));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
              : "=v"(ra[5]) : "v"(ir.y));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
              : "=v"(ra[6]) : "v"(ir.y));
          asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
              : "=v"(ra[7]) : "v"(ir.y));
          // two groups of 4 into the buffer the products just issued read from: the first
          // group's LDS latency hides behind those products
          uint4 (&cr)[4] = cv[h % 3];
#pragma unroll
          for (int k = 0; k < 4; ++k) cr[k] = *(const uint4*)((const char*)lds + ra[k]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int k = 0; k < 4; ++k) d[q] = mfma16(cr[k], xr[k], d[q]);
#pragma unroll
          for (int k = 0; k < 4; ++k) cr[k] = *(const uint4*)((const char*)lds + ra[4 + k]);
          ir = load_res(prb, pc);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int k = 0; k < 4; ++k) d[q] = mfma16(cr[k], xr[4 + k], d[q]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SM) {  // the next chunk's activations: converted, staged, read back
      xbuf ^= 1;
      stage_x(xbuf, xw, xr);
    }
    adv_pre();
  };

  // End of a tile: per row group, the 8 column blocks are added in LDS (fixed order) and
  // one partial per (row, batch row) goes to the workspace.  Lane l of a wavefront holds
  // rows 4 * (l / 16) + r of output column l % 16 in register r.  For M <= 2 every row
  // group fits the reduction area at once (two barriers per tile); larger M takes the
  // row groups one at a time.
  auto store_part = [&](int q, int rl, int m, float v) __attribute__((always_inline)) {
    const int row = rbk * kRT + q * 16 + rl;
    if (row < N) g.part[((size_t)(cs * kSlices + s) * M + m) * N + row] = v;
  };
  auto tile_end = [&]() __attribute__((always_inline)) {
    if constexpr (SM) {
      if (r16 < M) {
#pragma unroll
        for (int q = 0; q < kRG; ++q) {
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((q * 8 + cb) * 16 + 4 * g4 + r) * 2 + r16] = d[q][r];
        }
      }
      __syncthreads();
      if (tid < kRT * M) {  // thread = (row group, row, batch row)
        const int m = tid & (M - 1);
        const int qr = tid / M;
        const int q = qr >> 4, rl = qr & 15;
        float v = 0.0f;
#pragma unroll
        for (int c2 = 0; c2 < 8; ++c2) v += red[((q * 8 + c2) * 16 + rl) * 2 + m];
        store_part(q, rl, m, v);
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kRG; ++q) d[q] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      return;
    }
    // one row group at a time (few row groups' addresses held live: no unrolling)
#pragma unroll 1
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
        store_part(q, rl, m, v);
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

  if constexpr (SM) {
    for (;;) {  // one register set: refilled from LDS at the end of each chunk
      chunk(xa, xa);
      if (!next()) break;
    }
  } else {
    for (;;) {  // activations alternate between two register sets
      chunk(xa, xb);
      if (!next()) break;
      chunk(xb, xa);
      if (!next()) break;
    }
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

// bf16 activations -> fp16 * 2^e, one workgroup per batch row: e puts max |x| * 2^-e in
// [2^14, 2^15), so every finite value stays finite and a row of small values is scaled up
// into the normal fp16 range as a row of large ones is scaled down.  Every value at least
// max |x| * 2^-31 converts exactly; smaller ones round with absolute error below
// 2^-25 * 2^e.  An all-zero row takes e = -141 (its zeros stay zeros).
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
  const int e = (int)((mx >> 7) & 0xFFu) - 127 - 14;
#pragma unroll
  for (int k = 0; k < kXprepHold; ++k) {
    const int i = tid + k * 1024;
    if (i < n8) xo[i] = xprep_convert(held[k], e);
  }
  for (int i = tid + kXprepHold * 1024; i < n8; i += 1024) xo[i] = xprep_convert(xr[i], e);
  if (tid == 0) xexp[m] = e;
}

// The x pass with the randomized Hadamard transform ahead of the rescale: per batch row,
// x~ = H_b (s . x) / sqrt(b) for every block of b = rht_block(IN) columns (H_b in
// Sylvester order, s_j = -1 where bit j of `signs` is set), in fp32, then the fp16 rewrite
// times 2^-e.  One workgroup per (batch row, block), b / 8 threads with one 16-byte word
// of x each.  The power of two comes from a bound every workgroup of the row computes the
// same way, |x~_i| <= sqrt(b) max |x|: e puts that bound in [2^14, 2^15), so nothing
// overflows, and since fp16 keeps 11 significant bits anywhere in its normal range the
// values lose nothing to the bound's slack until they are 2^-20 or so of the largest.
// The block sits in LDS; the butterflies run in phases of up to 4 index bits: a thread
// takes the 2^ST values of a group (consecutive in the phase's bits, the other bits
// fixed), transforms them in registers and writes them back; one barrier per phase.
constexpr int kRhtMaxBlock = 16384;

template <int ST>
__device__ __forceinline__ void rht_phase(float* blk, int b, int lo_bits) {
  constexpr int kLen = 1 << ST;
  const int span = 1 << lo_bits;
  const int groups = b >> ST;
  for (int it = threadIdx.x; it < groups; it += blockDim.x) {
    const int base = ((it >> lo_bits) << (lo_bits + ST)) | (it & (span - 1));
    float v[kLen];
#pragma unroll
    for (int j = 0; j < kLen; ++j) v[j] = blk[base + j * span];
#pragma unroll
    for (int h = 1; h < kLen; h <<= 1) {
#pragma unroll
      for (int j = 0; j < kLen; ++j) {
        if ((j & h) == 0) {
          const float u = v[j], w = v[j + h];
          v[j] = u + w;
          v[j + h] = u - w;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kLen; ++j) blk[base + j * span] = v[j];
  }
}

// 16-point transform of v in registers (index bits 0..3).
__device__ __forceinline__ void wht16(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float u = v[j], w = v[j + h];
        v[j] = u + w;
        v[j + h] = u - w;
      }
    }
  }
}

// block / 16 threads; thread t owns the block's values 16 t .. 16 t + 15.
__global__ __launch_bounds__(1024) void xprep_rht_kernel(const uint16_t* __restrict__ x, int xbf16, int in_features,
                                                         int block, float inv, float root_b,
                                                         const uint8_t* __restrict__ signs,
                                                         uint16_t* __restrict__ x16, int32_t* __restrict__ xexp) {
  __shared__ float blk[kRhtMaxBlock];
  __shared__ uint32_t smax;
  const int nblk = in_features / block;
  const int m = blockIdx.x / nblk;
  const int bk = blockIdx.x - m * nblk;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int n8 = in_features / 8;
  const uint4* xr = (const uint4*)(x + (size_t)m * in_features);
  if (tid == 0) smax = 0;
  // this thread's 16 values (two words, two sign bytes), then the whole row for the bound
  const int w0 = bk * (block / 8) + 2 * tid;
  const uint4 q0 = xr[w0], q1 = xr[w0 + 1];
  const uint32_t sb = signs[w0] | ((uint32_t)signs[w0 + 1] << 8);
  uint32_t mx = 0;  // largest |x| of the row, as bits of the 16-bit format (they order like the values)
  for (int i0 = tid; i0 < n8; i0 += 8 * nt) {  // 8 loads in flight per thread (clamped, no branch)
    uint4 q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = xr[min(i0 + k * nt, n8 - 1)];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) mx = max(mx, max(w[h] & 0x7FFFu, (w[h] >> 16) & 0x7FFFu));
    }
  }
  float v[16];
  {
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      const uint32_t b = (h & 1) ? (w[h >> 1] >> 16) : (w[h >> 1] & 0xFFFFu);
      const float f = xbf16 ? vqd::bf16_to_f32(b) : vqd::f16_to_f32(b);
      v[h] = ((sb >> h) & 1u) ? -f : f;
    }
  }
  wht16(v);  // index bits 0..3 in registers
  const int lb = 31 - __builtin_clz(block);  // block = 2^lb >= 16
  if (lb > 4) {
    float4* bp = (float4*)(blk + 16 * tid);
#pragma unroll
    for (int k = 0; k < 4; ++k) bp[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
  __syncthreads();  // smax cleared, the block in LDS
  atomicMax(&smax, mx);
  for (int lo = 4; lo < lb; lo += 4) {
    switch (min(4, lb - lo)) {
      case 1: rht_phase<1>(blk, block, lo); break;
      case 2: rht_phase<2>(blk, block, lo); break;
      case 3: rht_phase<3>(blk, block, lo); break;
      default: rht_phase<4>(blk, block, lo); break;
    }
    __syncthreads();
  }
  if (lb <= 4) __syncthreads();  // smax complete
  mx = smax;
  // bound = sqrt(b) max |x| (rounded up), e = its fp32 exponent less 141 - 127
  const float xmax = xbf16 ? vqd::bf16_to_f32(mx) : vqd::f16_to_f32(mx);
  const float bound = xmax * root_b * (1.0f + 0x1p-20f);
  const int e = (int)((__builtin_bit_cast(uint32_t, bound) >> 23) & 0xFFu) - 141;
  if (lb > 4) {
    const float4* bp = (const float4*)(blk + 16 * tid);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = bp[k];
      v[4 * k] = f.x;
      v[4 * k + 1] = f.y;
      v[4 * k + 2] = f.z;
      v[4 * k + 3] = f.w;
    }
  }
  uint32_t o[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const uint32_t l = vqd::f32_to_f16_rne(ldexpf(v[2 * h] * inv, -e));
    const uint32_t u = vqd::f32_to_f16_rne(ldexpf(v[2 * h + 1] * inv, -e));
    o[h] = l | (u << 16);
  }
  uint4* xo = (uint4*)(x16 + (size_t)m * in_features);
  xo[w0] = make_uint4(o[0], o[1], o[2], o[3]);
  xo[w0 + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  if (bk == 0 && tid == 0) xexp[m] = e;
}

struct Plan {
  SlicedCfg cfg;
  size_t part_off, x16_off, exp_off, bytes;
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Row blocks of 128 rows; the columns are split until every group has a tile (or the
// chunks run out).
Plan make_plan(int32_t n, int32_t in_features, int32_t m, bool bf16, bool rht = false) {
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
  // the fp16 copy of x only where an x pass runs (bf16 at M > 2, or the transform)
  p.exp_off = p.x16_off + ((bf16 && m > 2) || rht ? round256((size_t)m * in_features * 2) : 0);
  p.bytes = p.exp_off + (bf16 || rht ? round256((size_t)m * sizeof(int32_t)) : 0);
  return p;
}


template <bool RES>
vq_status launch_res(const ProductArgs& a, const SlicedCfg& g, hipStream_t s) {
  auto kern = a.m <= 2 ? gemv_sliced_kernel<RES, true> : gemv_sliced_kernel<RES, false>;
  const unsigned grid = 64u * (unsigned)((g.groups + 7) / 8);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, s, a, g);
  if (hipGetLastError() != hipSuccess) return VQ_ERR_HIP;
  const int total = a.n * a.m;
  hipLaunchKernelGGL(gemv_sliced_finalize, dim3((total + 255) / 256), dim3(256), 0, s, a, (const float*)g.part, g.xexp,
                     kSlices * g.n_cs);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

// Workspace for callers that cannot allocate (vq_gemv_noalloc): a fixed array in device
// memory, one copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address of this GPU's copy is
// looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

}  // namespace

namespace vqi {

size_t static_scratch_bytes() { return kScratchBytes; }

vq_status static_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VQ_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {  // first call on this device (concurrent first calls find the same address)
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VQ_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return VQ_OK;
}

vq_status launch_x_to_f16(const ProductArgs& a, uint16_t* x16, int32_t* xexp, void* stream) {
  hipLaunchKernelGGL(xprep_kernel, dim3(a.m), dim3(1024), 0, (hipStream_t)stream, a.x, a.in_features, x16, xexp);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

vq_status launch_partials_finalize(const ProductArgs& a, const float* part, const int32_t* xexp, int nparts,
                                   void* stream) {
  const int total = a.n * a.m;
  hipLaunchKernelGGL(gemv_sliced_finalize, dim3((total + 255) / 256), dim3(256), 0, (hipStream_t)stream, a, part, xexp,
                     nparts);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

bool sliced_gemv_shape_ok(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (d.v != 8 || d.bits1 != 16 || !(d.bits2 == 0 || d.bits2 == 8)) return false;
  if (m < 1 || m > 16 || !(x_dtype == VQ_F16 || x_dtype == VQ_BF16)) return false;
  if (d.in_features % 8 != 0 || d.out_features < 1) return false;
  // 32-bit buffer offsets, the rows of the last row block included
  const uint64_t rows = (uint64_t)d.out_features + 256;
  if (rows * (uint64_t)row_stride(d.in_features, 8, 16) >= ((uint64_t)1 << 32)) return false;
  if (rows * (uint64_t)row_stride(d.in_features, 8, d.bits2) >= ((uint64_t)1 << 32)) return false;
  if ((uint64_t)m * (uint64_t)d.in_features * 2u >= ((uint64_t)1 << 32)) return false;
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

vq_status launch_x_rht_to_f16(const ProductArgs& a, const uint8_t* signs, uint16_t* x16, int32_t* xexp,
                              void* stream) {
  if (a.in_features > vqi::kFusedRhtMaxIn || a.in_features % 16 != 0) return VQ_ERR_UNSUPPORTED;
  const int b = rht_block(a.in_features);  // 16 <= b <= 16384
  const float inv = (float)(1.0 / __builtin_sqrt((double)b));
  const float root_b = (float)__builtin_sqrt((double)b);
  const unsigned grid = (unsigned)a.m * (unsigned)(a.in_features / b);
  // block / 16 threads, 16 values each (1 .. 1024 threads)
  hipLaunchKernelGGL(xprep_rht_kernel, dim3(grid), dim3(b / 16), 0, (hipStream_t)stream, a.x,
                     a.x_dtype == VQ_BF16 ? 1 : 0, a.in_features, b, inv, root_b, signs, x16, xexp);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

size_t sliced_gemv_rht_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (!sliced_gemv_shape_ok(d, m, x_dtype) || d.in_features > vqi::kFusedRhtMaxIn || d.in_features % 16 != 0) return 0;
  return make_plan(d.out_features, d.in_features, m, x_dtype == VQ_BF16, true).bytes;
}

vq_status launch_gemv_sliced(const ProductArgs& a, void* workspace, void* stream, const uint8_t* rht_signs) {
  // the kernels store partial sums into the workspace: never launch without one
  if (!workspace) return VQ_ERR_NULL;
  const bool bf16 = a.x_dtype == VQ_BF16;
  Plan p = make_plan(a.n, a.in_features, a.m, bf16, rht_signs != nullptr);
  char* ws = (char*)workspace;
  p.cfg.part = (float*)(ws + p.part_off);
  hipStream_t s = (hipStream_t)stream;
  p.cfg.xexp_out = nullptr;
  if (rht_signs) {
    // the transform and the fp16 rewrite in one pass; the product then reads fp16 x
    uint16_t* x16 = (uint16_t*)(ws + p.x16_off);
    int32_t* xexp = (int32_t*)(ws + p.exp_off);
    const vq_status st = launch_x_rht_to_f16(a, rht_signs, x16, xexp, stream);
    if (st != VQ_OK) return st;
    ProductArgs a16 = a;
    a16.x = x16;
    a16.x_dtype = VQ_F16;
    p.cfg.x16 = x16;
    p.cfg.xexp = xexp;
    return a.bits2 == 8 ? launch_res<true>(a16, p.cfg, s) : launch_res<false>(a16, p.cfg, s);
  }
  if (bf16 && a.m > 2) {
    uint16_t* x16 = (uint16_t*)(ws + p.x16_off);
    int32_t* xexp = (int32_t*)(ws + p.exp_off);
    hipLaunchKernelGGL(xprep_kernel, dim3(a.m), dim3(1024), 0, s, a.x, a.in_features, x16, xexp);
    if (hipGetLastError() != hipSuccess) return VQ_ERR_HIP;
    p.cfg.x16 = x16;
    p.cfg.xexp = xexp;
  } else if (bf16) {  // M <= 2: the product kernel converts x itself and writes the powers
    p.cfg.x16 = a.x;
    p.cfg.xexp_out = (int32_t*)(ws + p.exp_off);
    p.cfg.xexp = p.cfg.xexp_out;
  } else {
    p.cfg.x16 = a.x;
    p.cfg.xexp = nullptr;
  }
  return a.bits2 == 8 ? launch_res<true>(a, p.cfg, s) : launch_res<false>(a, p.cfg, s);
}

}  // namespace vqi
