// vq_gemv_ws over the slice-bucketed layout (VQ_LAYOUT_BUCKETED): the 65536-entry main
// book (v = 8) at one batch row, with every weight vector read and used exactly once.
//
// The book does not fit one CU's LDS, so it is cut into 8 slices of 8192 centroids and
// each workgroup holds one slice (the production-VQ post, "Lookup Table (LUT) Overhead vs.
// Bit-Shifting": lookups must stay in fast memory).  In the row-stream layout every slice
// workgroup has to look at every index to find its own; here the packer has already
// sorted each row's vectors by slice: bucket (chunk c, slice s, row o) lists the vectors
// j of row o with c*1024 <= j < (c+1)*1024 and idx1 >> 13 == s, one 32-bit word each:
//   bits [0, 10)  j - c*1024      bits [10, 23) idx1 & 8191      bits [23, 31) idx2
// behind a prefix table start[(c*8 + s)*N + o] of bucket offsets.
//   - 256 persistent workgroups of 1024 threads (16 wavefronts), one per CU; workgroup
//     (slice s, group p); the 32 workgroups of slice s share one XCD (and its L2 copy of
//     the slice's centroids);
//   - a unit is (chunk c, tile of 128 rows); group p takes units p, p + 32, ... in
//     chunk-major order; the chunk's 1024 activation vectors sit in LDS (reloaded when
//     the chunk changes, bf16 rewritten as fp16 times 2^-e);
//   - wavefront w takes rows 8w .. 8w + 7 of the tile; lane l handles words l, l + 64 and
//     l + 128 of a row's bucket (lanes past its end read zero entries); the rare bucket
//     longer than 192 words is finished by a loop after the tile's rows;
//   - per word: three 16-byte LDS reads (x at the position, the main centroid, the
//     residual centroid) and eight packed fp16 dot products into fp32;
//   - the next unit's bucket words are loaded while the current unit runs (each row's
//     words as soon as its LDS reads are issued), the prefix entries of the unit after
//     that one unit earlier still; all of row i + 1's LDS reads are issued before row i's
//     products;
//   - the 8 rows' lane sums are reduced together (a butterfly that halves the rows held
//     per lane at each of the first three exchanges) and stored as one fp32 partial per
//     (chunk, slice, row); the shared finalize kernel adds the 8 * chunks partials of
//     each output in a fixed order and applies 2^e, scale and bias.
#include "vq_device.h"

namespace {

using vqi::ProductArgs;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 8;
constexpr int kTileRows = kWaves * kRowsPerWave;  // 128
constexpr int kSlices = 8;
constexpr int kSlice = 8192;
constexpr int kGroups = 32;
constexpr int kChunk = vqi::kBucketChunk;  // 1024 vectors
constexpr int kRes = 256;
constexpr int kSteps = 3;  // bucket words per lane held in registers per row

// LDS, in 16-byte entries: the residual book and a zero entry; the chunk's activations
// and a zero entry; the slice (from an entry index that is a multiple of 16) and a zero
// entry; the per-wavefront maxima of the bf16 pass.  Every base fits the 16-bit offset
// field of ds_read_b128.
//
// A 16-byte read is served as fast as a read of consecutive entries when lanes 4q .. 4q + 3
// of every 16-lane group read entries in columns 4q .. 4q + 3 (column = entry mod 16; rows
// free, any order inside the four), as measured; random columns cost about 2.5 times as
// much.  The slice starting on a column-0 entry makes a main centroid's column its index
// mod 16, and the packer places each bucket word where bits [2, 4) of its index match bits
// [2, 4) of the lane (where the bucket's mix of indices allows).
constexpr int kResAt = 0;
constexpr int kXAt = kRes + 1;
constexpr int kSliceAt = (kXAt + kChunk + 1 + 15) / 16 * 16;
constexpr int kMaxAt = kSliceAt + kSlice + 1;
constexpr int kLdsEntries = kMaxAt + 4;  // 16 four-byte maxima
static_assert(kSliceAt % 16 == 0, "slice on a column-0 entry");
static_assert(kSliceAt * 16 < 65536, "slice base in the ds_read offset field");
static_assert(kLdsEntries * 16 <= 160 * 1024, "fits one CU's LDS");

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct BucketCfg {
  int32_t n_tiles;     // tiles of 64 rows
  int32_t n_chunks;    // chunks of 1024 vectors
  int32_t units;       // n_tiles * n_chunks
  uint32_t n_starts;   // prefix entries: 8 * n_chunks * N + 1
  uint32_t n_words;    // bucket words: N * nv
  float* part;         // [8 * n_chunks][N] partial sums
  int32_t* xexp_out;   // bf16: the power of two taken out of x (written by workgroup 0)
};

// Raw buffer resource over n bytes at p: a load whose offset (all in the vector operand
// here) lies past the n bytes returns zero and reads no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ float dot8(const uint4& c, const uint4& x, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.x), __builtin_bit_cast(half2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.y), __builtin_bit_cast(half2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.z), __builtin_bit_cast(half2_t, x.z), acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.w), __builtin_bit_cast(half2_t, x.w), acc, false);
}

// LDS byte addresses of one bucket word's operands; a lane past the bucket's end reads
// the three zero entries.
struct Addr {
  uint32_t x, c, r;
};
// Offsets within each region: the region bases are constants that the reads carry in
// their instruction offset field.
__device__ __forceinline__ Addr word_addr(uint32_t wd, bool valid) {
  Addr ad;
  ad.x = valid ? ((wd << 4) & 0x3FF0u) : (uint32_t)(kChunk * 16);
  ad.c = valid ? ((wd >> 6) & 0x1FFF0u) : (uint32_t)(kSlice * 16);
  ad.r = valid ? ((wd >> 19) & 0xFF0u) : (uint32_t)(kRes * 16);
  return ad;
}

struct Ops {
  uint4 x, c, r;
};

template <bool RES>
__device__ __forceinline__ void read_ops(const char* lds, const Addr& ad, Ops& o) {
  o.x = *(const uint4*)(lds + kXAt * 16 + ad.x);
  o.c = *(const uint4*)(lds + kSliceAt * 16 + ad.c);
  if constexpr (RES) o.r = *(const uint4*)(lds + kResAt * 16 + ad.r);
}

template <bool RES>
__device__ __forceinline__ void use_ops(const Ops& o, float& a0, float& a1) {
  a0 = dot8(o.c, o.x, a0);
  if constexpr (RES) a1 = dot8(o.r, o.x, a1);
}

// Sum of eight per-lane values r[0..7] over the wavefront: after the exchanges across 32,
// 16 and 8 lanes each lane holds one row's partial, finished within its group of 8
// lanes.  Lanes with (lane & 7) == 0 return row ((lane >> 5) & 1) * 4 + ((lane >> 4) &
// 1) * 2 + ((lane >> 3) & 1).  A fixed order: deterministic.
__device__ __forceinline__ float reduce8(const float (&r)[8], int lane) {
  float t[4], u[2];
  const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = h32 ? r[4 + k] : r[k];
    const float send = h32 ? r[k] : r[4 + k];
    t[k] = keep + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = h16 ? t[2 + k] : t[k];
    const float send = h16 ? t[k] : t[2 + k];
    u[k] = keep + __shfl_xor(send, 16, 64);
  }
  const float keep = h8 ? u[1] : u[0];
  const float send = h8 ? u[0] : u[1];
  float v = keep + __shfl_xor(send, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

template <bool RES>
__global__ __launch_bounds__(kThreads) void gemv_bucket_kernel(ProductArgs a, BucketCfg g) {
  __shared__ uint4 lds4[kLdsEntries];  // the only LDS array: it starts at address 0
  uint32_t* const wmax = (uint32_t*)(lds4 + kMaxAt);
  static_assert(kWaves <= 16, "one maximum per wavefront");
  const char* lds = (const char*)lds4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: row offsets stay scalar
  const int s = blockIdx.x & 7;
  const int grp = blockIdx.x >> 3;
  const int N = a.n, nv = a.nv;
  const bool xbf16 = a.x_dtype == VQ_BF16;

  const __amdgpu_buffer_rsrc_t bst = span(a.packed1, g.n_starts * 4u);
  const __amdgpu_buffer_rsrc_t bw = span(a.packed2, g.n_words * 4u);
  const __amdgpu_buffer_rsrc_t bx = span(a.x, (uint32_t)a.in_features * 2u);

  // the unit cursor and the prefix entries of this wavefront's rows
  int u = grp;
  auto unit_rows = [&](int uu, int& c, int& row0) __attribute__((always_inline)) {
    c = uu / g.n_tiles;
    row0 = (uu - c * g.n_tiles) * kTileRows + w * kRowsPerWave;
  };
  auto load_starts = [&](int uu) __attribute__((always_inline)) -> uint32_t {
    int c, row0;
    unit_rows(min(uu, g.units - 1), c, row0);
    const uint32_t b0 = (uint32_t)(c * kSlices + s) * (uint32_t)N + (uint32_t)row0;
    return ld4(bst, (b0 + (uint32_t)min(lane, kRowsPerWave)) * 4u, 0u);
  };

  // stage the slice and the residual book (loads first), and the first unit's words
  uint32_t ew[kRowsPerWave][kSteps];  // bucket words of the rows in flight
  int nrow[kRowsPerWave];             // their lengths (0 past N)
  uint32_t brow[kRowsPerWave];        // their first words
  uint32_t st_next;                   // prefix entries of the next unit
  {
    const uint4* src = (const uint4*)a.cb1 + (size_t)s * kSlice + tid;
    uint4* dst = lds4 + kSliceAt + tid;
    uint4 q[kSlice / kThreads];
#pragma unroll
    for (int k = 0; k < kSlice / kThreads; ++k) q[k] = src[k * kThreads];
    uint4 qr = make_uint4(0u, 0u, 0u, 0u);
    if (RES && tid < kRes) qr = ((const uint4*)a.cb2)[tid];
    const uint32_t st0 = load_starts(u);
    st_next = load_starts(u + kGroups);
    int c0, row0;
    unit_rows(u, c0, row0);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const uint32_t beg = (uint32_t)__builtin_amdgcn_readlane((int)st0, i);
      const uint32_t end = (uint32_t)__builtin_amdgcn_readlane((int)st0, i + 1);
      nrow[i] = row0 + i < N ? (int)(end - beg) : 0;
      brow[i] = beg;
#pragma unroll
      for (int k = 0; k < kSteps; ++k) ew[i][k] = ld4(bw, (beg + (uint32_t)(k * 64 + lane)) * 4u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kSlice / kThreads; ++k) dst[k * kThreads] = q[k];
    if (RES && tid <= kRes) lds4[kResAt + tid] = qr;  // entry kRes stays zero
    if (tid == 0) {
      lds4[kSliceAt + kSlice] = make_uint4(0u, 0u, 0u, 0u);
      lds4[kXAt + kChunk] = make_uint4(0u, 0u, 0u, 0u);
      if (!RES) lds4[kResAt + kRes] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // bf16: the largest |x| (as bits: they order like the values) over the row; e puts it
  // in [2^14, 2^15) after scaling by 2^-e
  int xe = 0;
  if (xbf16) {
    uint32_t mx = 0u;
    const int n16 = a.in_features / 8;
    for (int i = tid; i < n16; i += kThreads) {
      const uint4 v = ld16(bx, (uint32_t)i * 16u, 0u);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) mx = max(mx, max(w4[h] & 0x7FFFu, (w4[h] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
    if (lane == 0) wmax[w] = mx;
    __syncthreads();
    mx = 0u;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) mx = max(mx, wmax[k]);
    xe = (int)((mx >> 7) & 0xFFu) - 127 - 14;
    if (blockIdx.x == 0 && tid == 0) g.xexp_out[0] = xe;
  }

  // the activations of chunk c into LDS (two 16-byte vectors per thread)
  constexpr int kXPer = kChunk / kThreads;  // activation vectors per thread
  auto load_chunk = [&](int c) __attribute__((always_inline)) {
    uint4 v[kXPer];
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      const int j = c * kChunk + tid + k * kThreads;
      v[k] = j < nv ? ld16(bx, (uint32_t)j * 16u, 0u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kXPer; ++k) {
      if (xbf16) {
        const uint32_t w4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t lo = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w4[h] & 0xFFFFu), -xe));
          const uint32_t hi = vqd::f32_to_f16_rne(ldexpf(vqd::bf16_to_f32(w4[h] >> 16), -xe));
          o[h] = lo | (hi << 16);
        }
        v[k] = make_uint4(o[0], o[1], o[2], o[3]);
      }
      lds4[kXAt + tid + k * kThreads] = v[k];
    }
  };

  int chunk_in_lds = -1;
  while (u < g.units) {
    int c, row0;
    unit_rows(u, c, row0);
    if (c != chunk_in_lds) {  // uniform over the workgroup: every wavefront walks the same units
      __syncthreads();        // every wavefront is done with the previous chunk
      load_chunk(c);
      __syncthreads();
      chunk_in_lds = c;
    }
    const int un = u + kGroups;
    int cn, row0n;
    unit_rows(min(un, g.units - 1), cn, row0n);
    const uint32_t st_cur = st_next;
    st_next = load_starts(un + kGroups);

    // Row by row: the reads of row i + 1's three steps are issued before row i's products
    // (always issued, so the compiler counts them exactly; lanes past a bucket's end read
    // the zero entries); the products of a row's second and third steps run only when its
    // bucket reaches them (a uniform branch around VALU work only); a row's words are
    // replaced by the next unit's as soon as its reads are issued.
    float r[kRowsPerWave];
    int ncur[kRowsPerWave];
    uint32_t bcur[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      ncur[i] = nrow[i];
      bcur[i] = brow[i];
    }
    Ops op[2][kSteps];  // [row parity][step]
    auto row_reads = [&](int i, Ops (&o)[kSteps]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < kSteps; ++q) read_ops<RES>(lds, word_addr(ew[i][q], q * 64 + lane < ncur[i]), o[q]);
      // row i's words are consumed: fetch the next unit's row i (past the last unit these
      // reads repeat it, unused: no branch)
      const uint32_t beg = (uint32_t)__builtin_amdgcn_readlane((int)st_cur, i);
      const uint32_t end = (uint32_t)__builtin_amdgcn_readlane((int)st_cur, i + 1);
      nrow[i] = row0n + i < N ? (int)(end - beg) : 0;
      brow[i] = beg;
#pragma unroll
      for (int q = 0; q < kSteps; ++q) ew[i][q] = ld4(bw, (beg + (uint32_t)(q * 64 + lane)) * 4u, 0u);
    };
    row_reads(0, op[0]);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (i + 1 < kRowsPerWave) row_reads(i + 1, op[(i + 1) & 1]);
      const Ops (&o)[kSteps] = op[i & 1];
      float a0 = 0.0f, a1 = 0.0f;
      if (ncur[i] > 0) use_ops<RES>(o[0], a0, a1);
      if (ncur[i] > 64) use_ops<RES>(o[1], a0, a1);
      if (ncur[i] > 128) use_ops<RES>(o[2], a0, a1);
      r[i] = a0 + a1;
      asm volatile("" : "+v"(r[i]));  // the products happen here
    }

    // buckets longer than the 192 words held in registers (uniform per row; rare for
    // uniform indices, every word for a row whose indices all fall in one slice)
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (ncur[i] > kSteps * 64) {
        float t0 = 0.0f, t1 = 0.0f;
        for (int base = kSteps * 64; base < ncur[i]; base += 64) {
          const uint32_t wd = ld4(bw, (bcur[i] + (uint32_t)(base + lane)) * 4u, 0u);
          Ops o;
          read_ops<RES>(lds, word_addr(wd, base + lane < ncur[i]), o);
          use_ops<RES>(o, t0, t1);
        }
        r[i] += t0 + t1;
      }
    }

    const float sum = reduce8(r, lane);
    if ((lane & 7) == 0) {
      const int rr = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
      const int row = row0 + rr;
      if (row < N) g.part[(size_t)(c * kSlices + s) * (size_t)N + (size_t)row] = sum;
    }
    u = un;
  }
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

BucketCfg make_cfg(const ProductArgs& a) {
  BucketCfg g{};
  g.n_tiles = (a.n + kTileRows - 1) / kTileRows;
  g.n_chunks = (a.nv + kChunk - 1) / kChunk;
  g.units = g.n_tiles * g.n_chunks;
  g.n_starts = (uint32_t)(kSlices * g.n_chunks) * (uint32_t)a.n + 1u;
  g.n_words = (uint32_t)a.n * (uint32_t)a.nv;
  return g;
}

}  // namespace

namespace vqi {

bool bucketed_gemv_shape_ok(const vq_desc& d) {
  if (d.v != 8 || d.bits1 != 16 || !(d.bits2 == 0 || d.bits2 == 8)) return false;
  if (d.in_features % 8 != 0) return false;
  // bucket words and prefix entries addressed with 32-bit byte offsets
  const uint64_t nv = (uint64_t)d.in_features / 8;
  const uint64_t chunks = (nv + kChunk - 1) / kChunk;
  if ((uint64_t)d.out_features * nv * 4u >= ((uint64_t)1 << 31)) return false;
  if (((uint64_t)kSlices * chunks * (uint64_t)d.out_features + 1u) * 4u >= ((uint64_t)1 << 31)) return false;
  return true;
}

size_t bucketed_gemv_workspace(const vq_desc& d) {
  const int64_t nv = d.in_features / 8;
  const int64_t chunks = (nv + kChunk - 1) / kChunk;
  return round256((size_t)kSlices * (size_t)chunks * (size_t)d.out_features * sizeof(float)) + 256;
}

vq_status launch_gemv_bucketed(const ProductArgs& a, void* workspace, void* stream) {
  if (!workspace) return VQ_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  BucketCfg g = make_cfg(a);
  char* ws = (char*)workspace;
  g.part = (float*)ws;
  const size_t exp_off = round256((size_t)kSlices * (size_t)g.n_chunks * (size_t)a.n * sizeof(float));
  g.xexp_out = (int32_t*)(ws + exp_off);
  const int nparts = kSlices * g.n_chunks;
  if (g.units > 0) {
    const int groups = g.units < kGroups ? g.units : kGroups;
    const unsigned grid = (unsigned)(kSlices * groups);
    if (a.bits2 == 8) {
      hipLaunchKernelGGL(gemv_bucket_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a, g);
    } else {
      hipLaunchKernelGGL(gemv_bucket_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a, g);
    }
    if (hipGetLastError() != hipSuccess) return VQ_ERR_HIP;
  }
  return launch_partials_finalize(a, g.part, a.x_dtype == VQ_BF16 && g.units > 0 ? g.xexp_out : nullptr,
                                  g.units > 0 ? nparts : 0, stream);
}

}  // namespace vqi
