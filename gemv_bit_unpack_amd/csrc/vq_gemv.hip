// vq_gemv: decode-batch product y[M][N] = x[M][IN] * W^T (+ bias), 1 <= M <= 16.
//
// The weight vectors are rebuilt on the fly, never stored (VPTQ guide, "Step 3: Fused
// Low-Bit VPTQ Linear Layer": one fused kernel per linear layer, indices read from
// device memory, looked up in an on-chip codebook, dot product in registers; the
// production-VQ post's "Dequantization Kernels and Inference Dynamics": small books in
// on-chip memory, K >= 65536 books served from L2).
//
// gfx950 mapping.  A wavefront walks its rows in groups of 64*U vectors; lane l takes
// vectors g*64*U + u*64 + l (u < U), so the index words, the x slices and the gathers
// of one instruction are spread over a contiguous run of the row: index and x loads are
// coalesced, only the centroid gathers are random.  Per vector a lane unpacks its
// indices, gathers the main centroid (LDS when K1 <= 4096, else global memory: a 1 MiB
// book stays resident in each XCD's L2), gathers the residual centroid from LDS, adds
// them in fp32 and multiply-accumulates with x in fp32.  The loop is software-pipelined:
// the index loads of the next group are in flight while the current group's gathers
// return, so every lane keeps U gathers outstanding.  At the end of a row the 64 partial
// sums are reduced across the wavefront and lane 0 applies the channel scale and bias.
// Small codebooks are staged once per workgroup (16 bytes per centroid, v <= 8) and
// workgroups are persistent (grid-stride over rows) so the staging is amortised.  A
// global main book is first streamed through L2 with coalesced loads (each workgroup its
// share), so the random gathers that follow do not each pay an HBM miss.
#include <mutex>

#include "vq_device.h"

namespace {

using vqi::ProductArgs;

// Index j of a row: IB = 16 reads a 16-bit field directly, IB = 0 funnels two words
// (any width up to 16 bits).  Branch-free: the second word's index is clamped into the
// row, so the last field of the last row never reads past the buffer.
template <int IB>
__device__ __forceinline__ uint32_t load_index(const uint32_t* __restrict__ row, int32_t row_words, uint32_t j,
                                               uint32_t bits) {
  if constexpr (IB == 16) {
    return ((const uint16_t*)row)[j];
  } else {
    const uint32_t bitpos = j * bits;
    const uint32_t w = bitpos >> 5;
    const uint32_t lo = row[w];
    const uint32_t hi = row[min(w + 1u, (uint32_t)row_words - 1u)];
    return __builtin_amdgcn_alignbit(hi, lo, bitpos & 31u) & ((1u << bits) - 1u);
  }
}

// A raw centroid: fp16 bits in 16-byte words, zero padded (v = 6 and 8: one word; v = 16:
// two, read with two 16-byte loads of the same cache line, which the memory pipeline
// serves as one request).
template <int V>
struct Cent {
  static constexpr int kWords = V > 8 ? 2 : 1;
  uint4 q[kWords];
};

template <int V>
__device__ __forceinline__ Cent<V> gather_global(const uint16_t* __restrict__ cb, uint32_t k) {
  Cent<V> c;
  if constexpr (V == 16) {
    c.q[0] = *(const uint4*)(cb + (size_t)k * 16);
    c.q[1] = *(const uint4*)(cb + (size_t)k * 16 + 8);
  } else if constexpr (V == 8) {
    c.q[0] = *(const uint4*)(cb + (size_t)k * 8);
  } else {
    static_assert(V == 6, "fast path covers v = 6, 8 and 16");
    const uint32_t* p = (const uint32_t*)(cb + (size_t)k * 6);
    c.q[0] = make_uint4(p[0], p[1], p[2], 0u);
  }
  return c;
}

template <int V>
__device__ __forceinline__ float half_at(const Cent<V>& c, int t) {
  const uint4& q = c.q[t / 8];
  const int tt = t % 8;
  const uint32_t w = tt < 2 ? q.x : tt < 4 ? q.y : tt < 6 ? q.z : q.w;
  return vqd::f16_to_f32((tt & 1) ? (w >> 16) : w);
}

// x[m][col0 .. col0 + V) as fp32, branch-free.  The fast path guarantees IN % 8 == 0 for
// v = 8 and 16 (so each group of 8 columns is either whole or past the row: such groups
// read a clamped group and the caller zeroes their weights) and IN even for v = 6 (each x
// pair is either inside the row or dropped, so the last, partial vector keeps exactly its
// valid lanes).
template <int V, int XT>
__device__ __forceinline__ void load_x(const uint16_t* __restrict__ xrow, int32_t col0, int32_t in_features,
                                       float (&xv)[V]) {
  uint32_t w[V / 2];
  if constexpr (V == 8 || V == 16) {
#pragma unroll
    for (int h = 0; h < V / 8; ++h) {
      const uint4 q = *(const uint4*)(xrow + min(col0 + 8 * h, in_features - 8));
      w[4 * h] = q.x; w[4 * h + 1] = q.y; w[4 * h + 2] = q.z; w[4 * h + 3] = q.w;
    }
  } else {
    const uint32_t* p = (const uint32_t*)xrow;
    const int32_t last_pair = in_features / 2 - 1;
#pragma unroll
    for (int d = 0; d < V / 2; ++d) {
      const int32_t pair = col0 / 2 + d;
      const uint32_t raw = p[min(pair, last_pair)];
      w[d] = pair <= last_pair ? raw : 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    xv[2 * i] = vqd::x_to_f32<XT>(w[i] & 0xFFFFu);
    xv[2 * i + 1] = vqd::x_to_f32<XT>(w[i] >> 16);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, vqd::kWave);
  return v;
}

// Stage books into LDS as entries of Cent<V>::kWords 16-byte words.  Each thread first
// loads all of its entries (up to kStageBatch per pass), then writes them, so the loads
// overlap.
constexpr int kStageBatch = 8;
template <int V>
__device__ __forceinline__ void stage_books(Cent<V>* lds, const uint16_t* cb1, int k1, const uint16_t* cb2, int k2,
                                            int block) {
  const int total = k1 + k2;
  for (int base = 0; base < total; base += kStageBatch * block) {
    Cent<V> q[kStageBatch];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = min(base + b * block + (int)threadIdx.x, total - 1);
      q[b] = e < k1 ? gather_global<V>(cb1, (uint32_t)e) : gather_global<V>(cb2, (uint32_t)(e - k1));
    }
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int e = base + b * block + (int)threadIdx.x;
      if (e < total) lds[e] = q[b];
    }
  }
}

// Stream this workgroup's share of a global book through L2 (one 4-byte load per
// 128-byte line, at most two per thread).  Workgroups are dealt to the XCDs round-robin,
// so the groups on one XCD together cover the book.  The loaded words are only consumed
// at the end of the kernel, so nothing waits for them.
__device__ __forceinline__ void warm_book(const uint16_t* __restrict__ cb, uint32_t book_bytes, uint32_t block,
                                          uint32_t grid, uint32_t (&w)[2]) {
  const uint32_t lines = (book_bytes + 127u) / 128u;
  const uint32_t per_xcd = (grid + 7u) / 8u;
  const uint32_t share = (lines + per_xcd - 1u) / per_xcd;
  const uint32_t first = (blockIdx.x / 8u) * share;
  const uint32_t end = min(first + share, lines);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t l = first + threadIdx.x + k * block;
    w[k] = 0u;
    if (l < end) w[k] = *(const uint32_t*)((const uint8_t*)cb + (size_t)l * 128u);
  }
}

// IB1 = 16: 16-bit main indices into a global book (K1 = 65536); IB1 = 0: main book in
// LDS (K1 <= 4096), any index width.  RK: the second book -- 0 none, 1 in LDS
// (K2 <= 4096), 2 a global book with 16-bit indices (K2 = 65536: two large additive
// books, as in the production-VQ post's AQLM 2 x 2^16 configuration).
template <int V, int MT, int XT, int IB1, int RK, int U>
__global__ __launch_bounds__(1024) void gemv_kernel(ProductArgs a, int block, int grid) {
  constexpr bool kLds1 = IB1 != 16;
  extern __shared__ uint4 lds_words[];
  Cent<V>* lds_books = (Cent<V>*)lds_words;
  const int k1 = kLds1 ? (1 << a.bits1) : 0;
  const int k2 = RK == 1 ? (1 << a.bits2) : 0;
  const Cent<V>* book1 = lds_books;
  const Cent<V>* book2 = lds_books + k1;
  uint32_t warm[2] = {0u, 0u}, warm2[2] = {0u, 0u};
  if constexpr (!kLds1) warm_book(a.cb1, (uint32_t)(V * 2) << a.bits1, (uint32_t)block, (uint32_t)grid, warm);
  if constexpr (RK == 2) warm_book(a.cb2, (uint32_t)(V * 2) << a.bits2, (uint32_t)block, (uint32_t)grid, warm2);
  if (k1 + k2 > 0) {
    stage_books<V>(lds_books, a.cb1, k1, a.cb2, k2, block);
    __syncthreads();
  }
  const int lane = threadIdx.x & (vqd::kWave - 1);
  const int waves_per_block = block / vqd::kWave;
  const int total_waves = grid * waves_per_block;
  const int m_count = a.m;
  constexpr int kGroup = vqd::kWave * U;
  const int groups = (a.nv + kGroup - 1) / kGroup;
  const uint32_t last_j = (uint32_t)a.nv - 1u;

  int row = blockIdx.x * waves_per_block + (threadIdx.x / vqd::kWave);
  int g = 0;
  if (row < a.n) {
    uint32_t i1[U], i2[U];
    auto fetch_idx = [&](int r, int gg, uint32_t(&o1)[U], uint32_t(&o2)[U]) {
      const uint32_t* r1 = a.packed1 + (size_t)r * a.s1_words;
      const uint32_t* r2 = RK ? a.packed2 + (size_t)r * a.s2_words : nullptr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t j = min((uint32_t)(gg * kGroup + u * vqd::kWave + lane), last_j);
        o1[u] = load_index<IB1>(r1, a.s1_words, j, a.bits1);
        if constexpr (RK == 1) o2[u] = load_index<0>(r2, a.s2_words, j, a.bits2);
        if constexpr (RK == 2) o2[u] = load_index<16>(r2, a.s2_words, j, a.bits2);
      }
    };
    fetch_idx(row, g, i1, i2);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    while (true) {
      // gathers of the current group
      Cent<V> c1[U], c2[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (kLds1) {
          c1[u] = book1[i1[u]];
        } else {
          c1[u] = gather_global<V>(a.cb1, i1[u]);
        }
        if constexpr (RK == 1) c2[u] = book2[i2[u]];
        if constexpr (RK == 2) c2[u] = gather_global<V>(a.cb2, i2[u]);
      }
      // index loads of the next group (or a harmless repeat of this row's last group),
      // in flight while the gathers return
      int nrow = row, ng = g + 1;
      if (ng == groups) {
        ng = 0;
        nrow = row + total_waves;
      }
      const bool has_next = nrow < a.n;
      uint32_t n1[U], n2[U];
      fetch_idx(has_next ? nrow : row, has_next ? ng : g, n1, n2);
      // multiply-accumulate; lanes past the row contribute exactly zero
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = g * kGroup + u * vqd::kWave + lane;
        const int32_t col0 = j * V;
        float w[V];
#pragma unroll
        for (int t = 0; t < V; ++t) {
          w[t] = half_at<V>(c1[u], t);
          if constexpr (RK != 0) w[t] = w[t] + half_at<V>(c2[u], t);
          // v = 8, 16: columns past the row (whole groups of 8, IN % 8 == 0) weigh zero;
          // v = 6 zeroes them through x instead
          if constexpr (V != 6) w[t] = col0 + t < a.in_features ? w[t] : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < m_count) {
            float xv[V];
            load_x<V, XT>(a.x + (size_t)m * a.in_features, col0, a.in_features, xv);
#pragma unroll
            for (int t = 0; t < V; ++t) acc[m] = __builtin_fmaf(xv[t], w[t], acc[m]);
          }
        }
      }
      if constexpr (V == 6) {
#pragma unroll
        for (int u = 0; u < U; ++u) {  // whole 16-byte LDS entries read: ds_read_b128, not b96
          if constexpr (kLds1) asm volatile("" ::"v"(c1[u].q[0].w));
          if constexpr (RK == 1) asm volatile("" ::"v"(c2[u].q[0].w));
        }
      }
      if (ng == 0 || !has_next) {  // row finished
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
          acc[m] = 0.0f;
        }
      }
      if (!has_next) break;
      row = nrow;
      g = ng;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        i1[u] = n1[u];
        if constexpr (RK != 0) i2[u] = n2[u];
      }
    }
  }
  if (a.n < 0 && (warm[0] ^ warm[1] ^ warm2[0] ^ warm2[1]) == 0x9E3779B9u)  // never true: keeps the loads
    ((uint32_t*)a.y)[0] = warm[0];
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
#ifndef VQ_GEMV_SMALL_BLOCK
#define VQ_GEMV_SMALL_BLOCK 256  // threads per workgroup when the books need little LDS
#endif
#ifndef VQ_GEMV_SMALL_PER_CU
#define VQ_GEMV_SMALL_PER_CU 8  // resident workgroups per CU assumed for the persistent grid
#endif
#ifndef VQ_GEMV_U1
#define VQ_GEMV_U1 8  // vectors in flight per lane for M <= 2 (rows of up to 512 vectors: 4)
#endif


// ---------------------------------------------------------------------------------------
// v = 6 decode kernel for fp16 activations with both books in LDS (the 8B-class MLP
// layers: K1 = K2 = 4096, 12-bit indices).  The general kernel above spends ~97 VALU and
// ~10 memory instructions per 64 vectors here (each lane extracts its own index fields
// from global words and converts x and both centroids to fp32).  This one keeps the books'
// fp16 values and x in fp16 and multiplies them on the packed dot unit
// (v_dot2_f32_f16: exact products, fp32 sums; the main book is added first, so a one-hot
// x still yields fp32(c1 + c2)), and moves the index streams through LDS: per chunk of
// U groups of 64 vectors of a row (U = 4 for one batch row, 2 for two), the wavefront
// loads the chunk's index dwords with coalesced loads (2 * U * bits dwords per stream,
// 32-bit aligned), stores them in its own LDS
// area, and each lane reads its two fields from there.  Two register sets take chunks in
// turn: while one chunk is multiplied, the loads of the next one and of the one after it
// are in flight (about two chunks of work cover each load; one chunk ahead left the
// latency exposed).  Each lane loads its vector's three x pairs as one 12-byte load.
// All loads are buffer loads bounded by the row (IN is even): what lies past it reads as
// zero, so the vectors past a row's end and the missing pairs of a partial last vector
// add nothing.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Dwords of one wavefront's LDS area per index stream: a chunk of U groups holds 2 * U * bits
// dwords per stream; the area rounds the wider stream up to a multiple of 64 dwords.
__host__ __device__ constexpr int area6(int u, int bits1, int bits2) {
  return 64 * ((u * (bits1 > bits2 ? bits1 : bits2) + 31) / 32);
}

// LDS bytes of the v = 6 kernel: both books, 16 wavefronts' two index areas, one dword of
// slack for the last field's read of the dword after it.
inline size_t gemv6_lds(int u, int bits1, int bits2) {
  return 16u * (((size_t)1 << bits1) + (bits2 ? ((size_t)1 << bits2) : 0u)) +
         16u * 2u * 4u * (size_t)area6(u, bits1, bits2) + 16u;
}

__device__ __forceinline__ float dot6(const uint4& c, const uint32_t (&x)[3], float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.x), __builtin_bit_cast(half2_t, x[0]), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.y), __builtin_bit_cast(half2_t, x[1]), acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, c.z), __builtin_bit_cast(half2_t, x[2]), acc, false);
}

// A register copy the compiler cannot fold away: the early-clobber output takes a register
// of its own.  The chunk loop multiplies copies of a chunk's activations while the same
// registers already receive the chunk after next; folded, the copies would move the new
// loads between registers where the loop turns, which waits for them.
__device__ __forceinline__ uint32_t own_copy(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=&v"(r) : "v"(v));
  return r;
}

// One chunk's loads: U groups of 64 vectors.  q1/q2 hold this lane's share of the index
// dwords, x the three dwords its vector's activation pairs sit in (per group and batch row).
template <int MT, int U>
struct Chunk6 {
  uint32_t q1[U / 2], q2[U / 2], x[U][MT][3];
};

// Raw buffer resource over n bytes at p (stride 0, dword data).  A buffer load returns
// zero for every dword that does not lie wholly inside the n bytes, offsets included, and
// reads no memory for it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc6(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

template <int U>
__device__ __forceinline__ void load_q6(__amdgpu_buffer_rsrc_t b, int voff, int soff, uint32_t (&q)[U / 2]) {
  static_assert(U == 2 || U == 4, "one or two index dwords per lane");
  if constexpr (U == 4) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b, voff, soff, 0);
    q[0] = v.x;
    q[1] = v.y;
  } else {
    q[0] = __builtin_amdgcn_raw_buffer_load_b32(b, voff, soff, 0);
  }
}

// Loads of chunk cc of row r.  Buffer loads bounded by the row: index dwords and
// activation pairs past the row's end read as zero, so a row's last chunk needs no masking
// (its vectors past the end have zero indices and zero x) and the addresses stay scalar.
template <int MT, int RK, int U>
__device__ __forceinline__ void fetch6(const ProductArgs& a, int r, int cc, int lane, int dw1, int dw2,
                                       Chunk6<MT, U>& k) {
  // index dwords: lane l takes dwords (U / 2) l .. (U / 2) l + U / 2 - 1 of the chunk in one load
  const __amdgpu_buffer_rsrc_t b1 = rsrc6(a.packed1 + (size_t)r * a.s1_words, 4u * (uint32_t)a.s1_words);
  load_q6<U>(b1, 4 * (U / 2) * lane, 4 * cc * dw1, k.q1);
  if constexpr (RK != 0) {
    const __amdgpu_buffer_rsrc_t b2 = rsrc6(a.packed2 + (size_t)r * a.s2_words, 4u * (uint32_t)a.s2_words);
    load_q6<U>(b2, 4 * (U / 2) * lane, 4 * cc * dw2, k.q2);
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const __amdgpu_buffer_rsrc_t bx =
        rsrc6(a.x + (size_t)min(m, a.m - 1) * a.in_features, 2u * (uint32_t)a.in_features);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x3_t v = __builtin_amdgcn_raw_buffer_load_b96(bx, 12 * (u * 64 + lane), 12 * 64 * U * cc, 0);
      k.x[u][m][0] = v.x;
      k.x[u][m][1] = v.y;
      k.x[u][m][2] = v.z;
    }
  }
}

// Per-wavefront walk state: the chunk being multiplied and the two behind it.
struct Walk6 {
  int row, c, row1, c1, row2, c2, rk;  // rk: how many rows this wavefront finished before w.row
};

// Multiplies the chunk held in k (row w.row, chunk w.c), then refills k with the chunk two
// ahead.  Past the wavefront's last chunk (w.row >= n) it runs on in-bounds repeat data
// and stores nothing.
template <int MT, int RK, int U>
__device__ __forceinline__ void step6(const ProductArgs& a, Walk6& w, int chunks, int total_waves, int lane,
                                      int dw1, int dw2, uint32_t mask1, uint32_t mask2, const uint4* book1,
                                      const uint4* book2, uint32_t* my1, uint32_t* my2, int area, Chunk6<MT, U>& k,
                                      uint32_t scv, uint32_t biv, float (&acc)[MT]) {
  // this chunk's index dwords into the wavefront's LDS area (lane l's U / 2 dwords at
  // (U / 2) l; the area ends on a whole store, or half of one), this lane's three x pairs
  // per group into xc
  if ((U / 2) * lane < area) {
#pragma unroll
    for (int i = 0; i < U / 2; ++i) {
      my1[(U / 2) * lane + i] = k.q1[i];
      if constexpr (RK != 0) my2[(U / 2) * lane + i] = k.q2[i];
    }
  }
  uint32_t xc[U][MT][3];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int d = 0; d < 3; ++d) xc[u][m][d] = own_copy(k.x[u][m][d]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // the chunk two ahead (past the end, an in-bounds row) in flight meanwhile
  fetch6<MT, RK, U>(a, min(w.row2, a.n - 1), w.c2, lane, dw1, dw2, k);
  // all fields first, then all centroid reads, then the products: every LDS read of the
  // chunk is in flight before the first product waits on one
  uint32_t i1[U], i2[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t jl = (uint32_t)(u * 64 + lane);
    const uint32_t b1 = jl * (uint32_t)a.bits1;
    i1[u] = __builtin_amdgcn_alignbit(my1[(b1 >> 5) + 1], my1[b1 >> 5], b1 & 31u) & mask1;
    if constexpr (RK != 0) {
      const uint32_t b2 = jl * (uint32_t)a.bits2;
      i2[u] = __builtin_amdgcn_alignbit(my2[(b2 >> 5) + 1], my2[b2 >> 5], b2 & 31u) & mask2;
    }
  }
  uint4 c1[U], c2[U];
  u32x4_t e1[U], e2[U];  // whole 16-byte entries (ds_read_b128; the fourth word is padding)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    e1[u] = *(const u32x4_t*)(book1 + i1[u]);
    c1[u] = make_uint4(e1[u].x, e1[u].y, e1[u].z, 0u);
    if constexpr (RK != 0) {
      e2[u] = *(const u32x4_t*)(book2 + i2[u]);
      c2[u] = make_uint4(e2[u].x, e2[u].y, e2[u].z, 0u);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float r = dot6(c1[u], xc[u][m], acc[m]);
      if constexpr (RK != 0) r = dot6(c2[u], xc[u][m], r);
      acc[m] = r;
    }
#pragma unroll
  for (int u = 0; u < U; ++u) {  // whole 16-byte LDS entries read: ds_read_b128, not b96
    asm volatile("" ::"v"(e1[u]));
    if constexpr (RK != 0) asm volatile("" ::"v"(e2[u]));
  }
  __builtin_amdgcn_wave_barrier();  // this chunk's index reads stay before the next chunk's writes
  if (w.row < a.n && (w.row1 != w.row || w.row1 >= a.n)) {  // row finished
    // the row's scale and bias, loaded at the start into lane w.rk
    const float sc = a.scale ? vqd::f16_to_f32((uint16_t)__builtin_amdgcn_readlane((int)scv, w.rk)) : 1.0f;
    const float bi = a.bias ? vqd::f16_to_f32((uint16_t)__builtin_amdgcn_readlane((int)biv, w.rk)) : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < a.m) {
        float r = wave_sum(acc[m]);
        if (lane == 0) {
          if (a.scale) r = r * sc;
          if (a.bias) r = r + bi;
          vqd::store_out(a.y, (size_t)m * a.n + w.row, r, a.y_dtype);
        }
      }
      acc[m] = 0.0f;
    }
  }
  w.rk += w.row1 != w.row ? 1 : 0;
  w.row = w.row1;
  w.c = w.c1;
  w.row1 = w.row2;
  w.c1 = w.c2;
  const bool wrap = w.c2 + 1 == chunks;
  w.c2 = wrap ? 0 : w.c2 + 1;
  w.row2 += wrap ? total_waves : 0;
}

template <int MT, int RK, int U>
__global__ __launch_bounds__(1024) void gemv6_kernel(ProductArgs a, int grid) {
  extern __shared__ uint4 lds_words[];
  const int k1 = 1 << a.bits1;
  const int k2 = RK != 0 ? 1 << a.bits2 : 0;
  const uint4* book1 = lds_words;
  const uint4* book2 = lds_words + k1;
  stage_books<6>((Cent<6>*)lds_words, a.cb1, k1, a.cb2, k2, 1024);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // uniform to the compiler: the walk state and loop control stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int area = area6(U, a.bits1, RK != 0 ? a.bits2 : 0);
  uint32_t* my1 = (uint32_t*)(lds_words + k1 + k2) + wave * 2 * area;  // this wavefront's index areas
  uint32_t* my2 = my1 + area;
  const int dw1 = 2 * U * a.bits1;
  const int dw2 = RK != 0 ? 2 * U * a.bits2 : 0;
  const uint32_t mask1 = (1u << a.bits1) - 1u, mask2 = (1u << a.bits2) - 1u;
  const int chunks = (a.nv + 64 * U - 1) / (64 * U);
  const int total_waves = grid * 16;
  Walk6 w;
  w.row = blockIdx.x * 16 + wave;
  if (w.row >= a.n) return;
  w.rk = 0;
  // scale and bias of this wavefront's rows (at most 64: the launch checks), lane k
  // holding those of its k-th row; a missing one reads the first index halfword (unused)
  uint32_t scv, biv;
  {
    const int r = min(w.row + lane * total_waves, a.n - 1);
    scv = *(a.scale ? a.scale + r : (const uint16_t*)a.packed1);
    biv = *(a.bias ? a.bias + r : (const uint16_t*)a.packed1);
  }
  w.c = 0;
  w.row1 = w.row;
  w.c1 = 1;
  if (w.c1 == chunks) {
    w.c1 = 0;
    w.row1 += total_waves;
  }
  w.row2 = w.row1;
  w.c2 = w.c1 + 1;
  if (w.c2 == chunks) {
    w.c2 = 0;
    w.row2 += total_waves;
  }
  // two register sets in turn, so no register moves wait on loads in flight
  Chunk6<MT, U> ka, kb;
  fetch6<MT, RK, U>(a, w.row, w.c, lane, dw1, dw2, ka);
  fetch6<MT, RK, U>(a, min(w.row1, a.n - 1), w.c1, lane, dw1, dw2, kb);
  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
  // both first chunks in before the loop, so that where the loop turns only the second
  // set's loads are outstanding and the first step waits for none of them
  __builtin_amdgcn_s_waitcnt(0);
  // two steps per trip and one exit test: an exit between them leaves values undefined on
  // that path, and the compiler then reads them out of registers whose loads are in flight
  while (w.row < a.n) {
    step6<MT, RK, U>(a, w, chunks, total_waves, lane, dw1, dw2, mask1, mask2, book1, book2, my1, my2, area, ka, scv, biv, acc);
    step6<MT, RK, U>(a, w, chunks, total_waves, lane, dw1, dw2, mask1, mask2, book1, book2, my1, my2, area, kb, scv, biv, acc);
  }
}

template <int MT, int RK, int U>
vq_status launch_gemv6(const ProductArgs& a, hipStream_t s) {
  auto kern = gemv6_kernel<MT, RK, U>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return VQ_ERR_HIP;
  const size_t lds = gemv6_lds(U, a.bits1, RK != 0 ? a.bits2 : 0);
  const long want = (a.n + 15) / 16;
  const unsigned grid = (unsigned)(want < kNumCU ? want : kNumCU);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(1024), lds, s, a, (int)grid);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int RK>
vq_status dispatch_gemv6(const ProductArgs& a, hipStream_t s) {
  // four groups per chunk; two batch rows take two to stay within 128 registers
  return a.m >= 2 ? launch_gemv6<2, RK, 2>(a, s) : launch_gemv6<1, RK, 4>(a, s);
}

// v = 6 with 12-bit fields, one fp16 batch row: both books and x in LDS, the index fields
// taken straight from registers.
//
// Lane l takes the four consecutive vectors 4l .. 4l + 3 of a 256-vector chunk: its 48 bits
// of each index stream are one 8-byte load (dword 3l / 2, shifted right by 16 (l & 1) bits),
// its x slice three 16-byte LDS reads at a 48-byte lane stride (no bank conflicts), and the
// only random LDS reads left are the two centroids per vector (16-byte entries, the residual
// book 64 KiB above the main one).  Each workgroup owns a block of consecutive rows; its (row, chunk) items
// are dealt evenly to the 16 wavefronts (a row may be shared by two or three), each
// wavefront writes its partial sum of a row to an LDS slot, and after a barrier one thread
// per row adds the slots in wavefront order, then applies the scale and bias.  Index loads
// are buffer loads bounded by the row, so vectors past its end read index 0 (and meet zero
// x): no masking.  kX6Depth chunks of index loads are in flight per wavefront.
constexpr int kX6Chunk = 256;                 // vectors per chunk (4 per lane)
constexpr int kX6ChunkBytes = kX6Chunk * 12;  // fp16 x bytes per chunk
constexpr int kX6Depth = 4;                   // chunks of index loads in flight per wavefront
constexpr int kX6Waves = 16;
constexpr int kX6Threads = 64 * kX6Waves;

inline size_t gemv6x_lds(bool residual, int in_features, int rows_wg) {
  const int chunks = (int)((vqi::num_vectors(in_features, 6) + kX6Chunk - 1) / kX6Chunk);
  return (size_t)16 * (residual ? 8192 : 4096) + (size_t)chunks * kX6ChunkBytes + (size_t)rows_wg * kX6Waves * 4;
}

// Sum over the wavefront without LDS traffic: within each row of 16 lanes by DPP (swap
// neighbours, swap pairs, rotate by 4, rotate by 8), then the four row sums.  Uniform result.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x124>(v);  // row_ror 4
  v += dpp_f32<0x128>(v);  // row_ror 8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Byte offsets in LDS of the four 12-bit fields of a lane's 48 bits (16-byte entries from
// byte `at`): lo, hi are the dwords holding them, sh (0 or 16) where they start.
__device__ __forceinline__ void fields12(uint32_t lo, uint32_t hi, uint32_t sh, uint32_t at, uint32_t (&ad)[4]) {
  const uint32_t w0 = __builtin_amdgcn_alignbit(hi, lo, sh);  // bits sh .. sh + 31
  const uint32_t w1 = hi >> sh;                               // bits sh + 32 ..
  ad[0] = (__builtin_amdgcn_ubfe(w0, 0, 12) << 4) | at;
  ad[1] = (__builtin_amdgcn_ubfe(w0, 12, 12) << 4) | at;
  ad[2] = ((__builtin_amdgcn_alignbit(w1, w0, 24) & 0xFFFu) << 4) | at;
  ad[3] = (__builtin_amdgcn_ubfe(w1, 4, 12) << 4) | at;
}

template <int RK>
__global__ __launch_bounds__(kX6Threads) void gemv6x_kernel(ProductArgs a, int rows_wg, int chunks) {
  // one workgroup per CU: all of the LDS, statically (addresses known when compiling)
  __shared__ uint4 lds_x6[160 * 1024 / 16];
  constexpr int kEntries = RK != 0 ? 8192 : 4096;
  uint8_t* base = (uint8_t*)lds_x6;
  const uint8_t* xl = base + (kEntries << 4);
  float* part = (float*)(base + (kEntries << 4) + chunks * kX6ChunkBytes);
  const int tid = threadIdx.x;
  {  // books (all loads of a thread in flight, then the stores) and x, zero past IN
    uint4 q[kEntries / kX6Threads];
#pragma unroll
    for (int b = 0; b < kEntries / kX6Threads; ++b) {
      const int e = b * kX6Threads + tid;
      q[b] = e < 4096 ? gather_global<6>(a.cb1, (uint32_t)e).q[0] : gather_global<6>(a.cb2, (uint32_t)(e - 4096)).q[0];
    }
#pragma unroll
    for (int b = 0; b < kEntries / kX6Threads; ++b) {
      const int e = b * kX6Threads + tid;
      *(uint4*)(base + 16 * e) = q[b];
    }
    const int units = chunks * (kX6ChunkBytes / 16), xunits = a.in_features / 8;
    for (int u = tid; u < units; u += kX6Threads) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (u < xunits) v = ((const uint4*)a.x)[u];
      ((uint4*)(base + (kEntries << 4)))[u] = v;
    }
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row0 = blockIdx.x * rows_wg;
  const int nrows = min(rows_wg, a.n - row0);
  const int items = nrows * chunks;
  const int i0 = wave * items / kX6Waves, i1 = (wave + 1) * items / kX6Waves;
  if (i1 > i0) {
    const uint32_t sh = (uint32_t)(lane & 1) << 4;
    const int voff = 4 * ((3 * lane) >> 1);
    // consumed item (it, cr, cc) and prefetched item (pr, pc), uniform
    int it = i0, cr = i0 / chunks, cc = i0 - cr * chunks;
    int pr = cr, pc = cc;
    // the prefetched item's row (past the wavefront's rows: its last one, in-bounds repeat data)
    const uint32_t* p1 = a.packed1 + (size_t)(row0 + pr) * a.s1_words;
    const uint32_t* p2 = RK != 0 ? a.packed2 + (size_t)(row0 + pr) * a.s2_words : nullptr;
    const uint32_t n1 = 4u * (uint32_t)a.s1_words, n2 = 4u * (uint32_t)a.s2_words;
    int soff = pc * 384;  // the chunk's byte offset in each index stream's row
    auto fetch = [&](uint32_t (&q)[4]) __attribute__((always_inline)) {
      const u32x2_t v1 = __builtin_amdgcn_raw_buffer_load_b64(rsrc6(p1, n1), voff, soff, 0);
      q[0] = v1.x;
      q[1] = v1.y;
      if constexpr (RK != 0) {
        const u32x2_t v2 = __builtin_amdgcn_raw_buffer_load_b64(rsrc6(p2, n2), voff, soff, 0);
        q[2] = v2.x;
        q[3] = v2.y;
      }
      soff += 384;
      if (++pc == chunks) {
        pc = 0;
        soff = 0;
        if (++pr < nrows) {
          p1 += a.s1_words;
          if constexpr (RK != 0) p2 += a.s2_words;
        }
      }
    };
    // one accumulator per vector slot (each vector's main then residual terms stay in order)
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // An item's LDS reads (x slice, centroids) are issued one step before its products, so a
    // wavefront always has the next item's reads in flight while it multiplies.
    int nc = cc;  // chunk of the item whose reads are issued next
    auto issue = [&](uint32_t (&q)[4], u32x4_t (&bx)[3], u32x4_t (&be1)[4], u32x4_t (&be2)[4])
                     __attribute__((always_inline)) {
      uint32_t ad1[4], ad2[4];
      fields12(q[0], q[1], sh, 0u, ad1);
      if constexpr (RK != 0) fields12(q[2], q[3], sh, 65536u, ad2);
      // the fields are out of q before its refill is issued, so the refill lands in the same
      // registers (no copies where the loop turns, which would wait for the loads)
      asm volatile("" ::"v"(ad1[0]), "v"(ad1[1]), "v"(ad1[2]), "v"(ad1[3]) : "memory");
      if constexpr (RK != 0) asm volatile("" ::"v"(ad2[0]), "v"(ad2[1]), "v"(ad2[2]), "v"(ad2[3]) : "memory");
      fetch(q);  // the item kX6Depth ahead into the same registers
      const u32x4_t* xp = (const u32x4_t*)(xl + nc * kX6ChunkBytes + 48 * lane);
      bx[0] = xp[0];
      bx[1] = xp[1];
      bx[2] = xp[2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        be1[u] = *(const u32x4_t*)(base + ad1[u]);
        if constexpr (RK != 0) be2[u] = *(const u32x4_t*)(base + ad2[u]);
      }
      if (++nc == chunks) nc = 0;
    };
    auto consume = [&](u32x4_t (&bx)[3], u32x4_t (&be1)[4], u32x4_t (&be2)[4]) __attribute__((always_inline)) {
      const uint32_t xw[12] = {bx[0].x, bx[0].y, bx[0].z, bx[0].w, bx[1].x, bx[1].y,
                               bx[1].z, bx[1].w, bx[2].x, bx[2].y, bx[2].z, bx[2].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t xv[3] = {xw[3 * u], xw[3 * u + 1], xw[3 * u + 2]};
        acc[u] = dot6(make_uint4(be1[u].x, be1[u].y, be1[u].z, 0u), xv, acc[u]);
        if constexpr (RK != 0) acc[u] = dot6(make_uint4(be2[u].x, be2[u].y, be2[u].z, 0u), xv, acc[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {  // whole 16-byte entries read: ds_read_b128, not b96 + b32
        asm volatile("" ::"v"(be1[u]));
        if constexpr (RK != 0) asm volatile("" ::"v"(be2[u]));
      }
      if (it < i1 && (cc == chunks - 1 || it == i1 - 1)) {  // this wavefront's share of row cr ends
        const float r = wave_sum_dpp((acc[0] + acc[1]) + (acc[2] + acc[3]));
        if (lane == 0) part[cr * kX6Waves + wave] = r;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = 0.0f;
      }
      ++it;
      if (++cc == chunks) {
        cc = 0;
        ++cr;
      }
    };
    uint32_t s0[4], s1[4], s2[4], s3[4];
    static_assert(kX6Depth == 4, "four register sets in turn");
    fetch(s0);
    fetch(s1);
    fetch(s2);
    fetch(s3);
    u32x4_t xa[3], a1[4], a2[4], xb[3], b1[4], b2[4];
    issue(s0, xa, a1, a2);
    // four steps per trip (the register sets in turn), then the last n % 4 items; the reads
    // issued for the item after the wavefront's last run on in-bounds data and are dropped
    const int n_w = i1 - i0;
    for (int t = n_w / kX6Depth; t > 0; --t) {
      issue(s1, xb, b1, b2);
      __builtin_amdgcn_sched_barrier(0);
      consume(xa, a1, a2);
      issue(s2, xa, a1, a2);
      __builtin_amdgcn_sched_barrier(0);
      consume(xb, b1, b2);
      issue(s3, xb, b1, b2);
      __builtin_amdgcn_sched_barrier(0);
      consume(xa, a1, a2);
      issue(s0, xa, a1, a2);
      __builtin_amdgcn_sched_barrier(0);
      consume(xb, b1, b2);
    }
    const int rem = n_w % kX6Depth;
    if (rem > 0) {
      issue(s1, xb, b1, b2);
      __builtin_amdgcn_sched_barrier(0);
      consume(xa, a1, a2);
      if (rem > 1) {
        issue(s2, xa, a1, a2);
        __builtin_amdgcn_sched_barrier(0);
        consume(xb, b1, b2);
        if (rem > 2) {
          issue(s3, xb, b1, b2);
          __builtin_amdgcn_sched_barrier(0);
          consume(xa, a1, a2);
        }
      }
    }
  }
  __syncthreads();
  if (tid < nrows) {  // row tid: the slots of the wavefronts whose items cover it, in order
    float r = 0.0f;
    for (int w = 0; w < kX6Waves; ++w) {
      const int w0 = w * items / kX6Waves, w1 = (w + 1) * items / kX6Waves;
      if (w1 > w0 && w1 > tid * chunks && w0 < (tid + 1) * chunks) r += part[tid * kX6Waves + w];
    }
    const int row = row0 + tid;
    if (a.scale) r = r * vqd::f16_to_f32(a.scale[row]);
    if (a.bias) r = r + vqd::f16_to_f32(a.bias[row]);
    vqd::store_out(a.y, (size_t)row, r, a.y_dtype);
  }
}

// Rows per workgroup for the x-in-LDS kernel (0: the shape does not fit it).
inline int gemv6x_rows(const ProductArgs& a) {
  const int grid = a.n < kNumCU ? a.n : kNumCU;
  const int rows = (a.n + grid - 1) / grid;
  if (rows > kX6Threads) return 0;  // one thread per row adds the slots
  return gemv6x_lds(a.bits2 != 0, a.in_features, rows) <= 160u * 1024u ? rows : 0;
}

template <int RK>
vq_status launch_gemv6x(const ProductArgs& a, int rows_wg, hipStream_t s) {
  auto kern = gemv6x_kernel<RK>;
  const int chunks = (a.nv + kX6Chunk - 1) / kX6Chunk;
  const unsigned grid = (unsigned)((a.n + rows_wg - 1) / rows_wg);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kX6Threads), 0, s, a, rows_wg, chunks);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

// v = 6 with 12-bit fields, 2 <= M <= 16 fp16 batch rows: the same LDS books, the products
// on the matrix cores.
//
// A 16-byte LDS entry is 6 centroid values and two zero halves, which is exactly one lane's
// A operand of v_mfma_f32_16x16x32_f16 (8 consecutive k of one row): each vector takes 8
// k slots, the last two multiplying zeros.  Lane l of a wavefront is row l % 16 of a
// 16-row tile and takes vectors 4 (l / 16) .. + 3 of a 16-vector step, one per matrix
// instruction, so its 48 bits of each index stream are one 8-byte load, as in the
// one-row kernel.  Its B operand is x[l % 16][those 6 values] and two zeros: three 16-byte
// loads per step cover its four vectors (rows past M read zeros, the x buffer ends there).
// Main and residual entries go through two matrix instructions into the same fp32
// accumulators: the products are exact and each vector's two terms are summed in fp32, so a
// one-hot x still returns fp32(c1 + c2).  Lane l ends a tile with rows 4 (l / 16) .. + 3 of
// output column (batch row) l % 16.
// A workgroup owns whole tiles; its (tile, step) items are dealt evenly to the 16
// wavefronts, each writes its partial tile to an LDS slot, and after a barrier the slots are
// added in wavefront order.  The last step of a row may reach past IN: there the x values
// past IN (the next batch row's, or zeros) are masked.
constexpr int kM6Step = 16;  // vectors per step (4 per lane group)

// LDS slots of partial tiles in a workgroup of nt tiles: a tile's slot k belongs to
// wavefront first + k, first being the first wavefront whose items meet the tile; the most
// any of the nt tiles needs.
inline int gemv6m_slots(int nt, int steps) {
  int most = 0;
  const int items = nt * steps;
  for (int t = 0; t < nt; ++t) {
    int wf = 0;
    while ((wf + 1) * items / kX6Waves <= t * steps) ++wf;
    int wl = wf;
    for (int w = wf; w < kX6Waves; ++w) {
      const int w0 = w * items / kX6Waves, w1 = (w + 1) * items / kX6Waves;
      if (w0 >= (t + 1) * steps) break;
      if (w1 > w0) wl = w;
    }
    most = wl - wf + 1 > most ? wl - wf + 1 : most;
  }
  return most;
}

template <int RK>
__global__ __launch_bounds__(kX6Threads) void gemv6m_kernel(ProductArgs a, int tiles_wg, int steps, int slots_full,
                                                           int slots_last) {
  __shared__ uint4 lds_m6[160 * 1024 / 16];
  constexpr int kEntries = RK != 0 ? 8192 : 4096;
  uint8_t* base = (uint8_t*)lds_m6;
  float* part = (float*)(base + (kEntries << 4));  // [tile][slot][16 rows][16 columns]
  const int tid = threadIdx.x;
  {
    uint4 q[kEntries / kX6Threads];
#pragma unroll
    for (int b = 0; b < kEntries / kX6Threads; ++b) {
      const int e = b * kX6Threads + tid;
      q[b] = e < 4096 ? gather_global<6>(a.cb1, (uint32_t)e).q[0] : gather_global<6>(a.cb2, (uint32_t)(e - 4096)).q[0];
    }
#pragma unroll
    for (int b = 0; b < kEntries / kX6Threads; ++b) {
      const int e = b * kX6Threads + tid;
      *(uint4*)(base + 16 * e) = q[b];
    }
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int tile0 = blockIdx.x * tiles_wg;
  const int ntiles = min(tiles_wg, (a.n + 15) / 16 - tile0);
  const int slots = ntiles == tiles_wg ? slots_full : slots_last;  // the last workgroup may hold fewer tiles
  const int items = ntiles * steps;
  const int i0 = wave * items / kX6Waves, i1 = (wave + 1) * items / kX6Waves;
  const uint32_t s1b = 4u * (uint32_t)a.s1_words, s2b = 4u * (uint32_t)a.s2_words;
  if (i1 > i0) {
    // one buffer per index stream over all N rows (rows past N read zeros); the lane's row
    // and window go in the vector offset, the tile and step in the scalar one
    const __amdgpu_buffer_rsrc_t b1 = rsrc6(a.packed1, (uint32_t)a.n * s1b);
    const __amdgpu_buffer_rsrc_t b2 = rsrc6(RK != 0 ? a.packed2 : a.packed1, RK != 0 ? (uint32_t)a.n * s2b : 0u);
    const __amdgpu_buffer_rsrc_t bx = rsrc6(a.x, (uint32_t)a.m * (uint32_t)a.in_features * 2u);
    const uint32_t row_l = (uint32_t)(tile0 * 16 + r16);
    const int v1 = (int)(row_l * s1b) + 4 * ((3 * g4) >> 1);
    const int v2 = (int)(row_l * s2b) + 4 * ((3 * g4) >> 1);
    const int vx = r16 * a.in_features * 2 + 48 * g4;
    const uint32_t sh = (uint32_t)(g4 & 1) << 4;
    const int have_last = a.in_features - 6 * (kM6Step * (steps - 1) + 4 * g4);  // valid halves, last step
    int it = i0, ct = i0 / steps, cs = i0 - ct * steps;  // consumed item (tile, step)
    int pt = ct, ps = cs;                                 // prefetched item
    // the prefetched item's scalar offsets (past the wavefront's tiles: its last one again)
    int so1 = (int)((uint32_t)(16 * pt) * s1b) + 24 * ps, so2 = (int)((uint32_t)(16 * pt) * s2b) + 24 * ps;
    int sox = 192 * ps;
    auto fetch = [&](uint32_t (&q)[4], u32x4_t (&xq)[3]) __attribute__((always_inline)) {
      const u32x2_t w1 = __builtin_amdgcn_raw_buffer_load_b64(b1, v1, so1, 0);
      q[0] = w1.x;
      q[1] = w1.y;
      if constexpr (RK != 0) {
        const u32x2_t w2 = __builtin_amdgcn_raw_buffer_load_b64(b2, v2, so2, 0);
        q[2] = w2.x;
        q[3] = w2.y;
      }
#pragma unroll
      for (int h = 0; h < 3; ++h)
        xq[h] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(bx, vx, sox + 16 * h, 0));
      so1 += 24;
      so2 += 24;
      sox += 192;
      if (++ps == steps) {
        ps = 0;
        sox = 0;
        if (++pt < ntiles) {
          so1 += (int)(16u * s1b) - 24 * steps;
          so2 += (int)(16u * s2b) - 24 * steps;
        } else {
          so1 -= 24 * steps;
          so2 -= 24 * steps;
        }
      }
    };
    float4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
    auto step = [&](uint32_t (&q)[4], u32x4_t (&xq)[3]) __attribute__((always_inline)) {
      uint32_t ad1[4], ad2[4];
      fields12(q[0], q[1], sh, 0u, ad1);
      if constexpr (RK != 0) fields12(q[2], q[3], sh, 65536u, ad2);
      // the row's last step: x past IN (the next batch row's values) reads as zero; selects
      // on loop-invariant lane masks, no branch (a branch here makes the other path copy x,
      // waiting for every load in flight)
      const bool last = cs == steps - 1;
      u32x4_t xs[3];
#pragma unroll
      for (int h = 0; h < 3; ++h) {
        xs[h].x = last && 8 * h + 2 > have_last ? 0u : xq[h].x;
        xs[h].y = last && 8 * h + 4 > have_last ? 0u : xq[h].y;
        xs[h].z = last && 8 * h + 6 > have_last ? 0u : xq[h].z;
        xs[h].w = last && 8 * h + 8 > have_last ? 0u : xq[h].w;
      }
      // fields and x out of the set before its refill is issued (same registers)
      asm volatile("" ::"v"(ad1[0]), "v"(ad1[1]), "v"(ad1[2]), "v"(ad1[3]) : "memory");
      if constexpr (RK != 0) asm volatile("" ::"v"(ad2[0]), "v"(ad2[1]), "v"(ad2[2]), "v"(ad2[3]) : "memory");
      asm volatile("" ::"v"(xs[0]), "v"(xs[1]), "v"(xs[2]) : "memory");
      fetch(q, xq);
      u32x4_t e1[4], e2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        e1[u] = *(const u32x4_t*)(base + ad1[u]);
        if constexpr (RK != 0) e2[u] = *(const u32x4_t*)(base + ad2[u]);
      }
      const uint32_t xw[12] = {xs[0].x, xs[0].y, xs[0].z, xs[0].w, xs[1].x, xs[1].y,
                               xs[1].z, xs[1].w, xs[2].x, xs[2].y, xs[2].z, xs[2].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 bfrag = make_uint4(xw[3 * u], xw[3 * u + 1], xw[3 * u + 2], 0u);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, e1[u]),
                                                   __builtin_bit_cast(half8_t, bfrag), d, 0, 0, 0);
        if constexpr (RK != 0)
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, e2[u]),
                                                     __builtin_bit_cast(half8_t, bfrag), d, 0, 0, 0);
      }
      if (it < i1 && (cs == steps - 1 || it == i1 - 1)) {  // this wavefront's share of tile ct ends
        // slot: this wavefront less the first one whose items meet the tile
        int w = (ct * steps) * kX6Waves / items;  // a lower bound on that first one
        while ((w + 1) * items / kX6Waves <= ct * steps) ++w;
        float* dst = part + ((size_t)(ct * slots + (wave - w)) * 256);
        if (r16 < a.m) {
#pragma unroll
          for (int q = 0; q < 4; ++q) dst[(4 * g4 + q) * 16 + r16] = d[q];
        }
        d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
      ++it;
      if (++cs == steps) {
        cs = 0;
        ++ct;
      }
    };
    uint32_t q0[4], q1[4], q2[4], q3[4];
    u32x4_t x0[3], x1[3], x2[3], x3[3];
    fetch(q0, x0);
    fetch(q1, x1);
    fetch(q2, x2);
    fetch(q3, x3);
    const int n_w = i1 - i0;
    for (int t = n_w / 4; t > 0; --t) {
      step(q0, x0);
      step(q1, x1);
      step(q2, x2);
      step(q3, x3);
    }
    const int rem = n_w % 4;
    if (rem > 0) {
      step(q0, x0);
      if (rem > 1) {
        step(q1, x1);
        if (rem > 2) step(q2, x2);
      }
    }
  }
  __syncthreads();
  // (tile, row, batch row) outputs: the slots of the wavefronts whose items meet the tile,
  // in wavefront order, then scale and bias
  for (int o = tid; o < ntiles * 16 * a.m; o += kX6Threads) {
    const int m = o % a.m, tr = o / a.m;
    const int t = tr >> 4, rr = tr & 15;
    const int row = (tile0 + t) * 16 + rr;
    if (row >= a.n) continue;
    float r = 0.0f;
    int wf = (t * steps) * kX6Waves / items;  // the first wavefront whose items meet the tile
    while ((wf + 1) * items / kX6Waves <= t * steps) ++wf;
    for (int w = wf; w < kX6Waves; ++w) {
      const int w0 = w * items / kX6Waves, w1 = (w + 1) * items / kX6Waves;
      if (w0 >= (t + 1) * steps) break;
      if (w1 > w0) r += part[(size_t)(t * slots + (w - wf)) * 256 + rr * 16 + m];
    }
    if (a.scale) r = r * vqd::f16_to_f32(a.scale[row]);
    if (a.bias) r = r + vqd::f16_to_f32(a.bias[row]);
    vqd::store_out(a.y, (size_t)m * a.n + row, r, a.y_dtype);
  }
}

// Tiles per workgroup and partial-tile slots (full workgroups, the last one) for the
// matrix-core v = 6 kernel (false: the shape does not fit it).
inline bool gemv6m_plan(const ProductArgs& a, int* tiles_wg, int* steps, int* slots_full, int* slots_last) {
  const int tiles = (a.n + 15) / 16;
  const int grid = tiles < kNumCU ? tiles : kNumCU;
  *tiles_wg = (tiles + grid - 1) / grid;
  *steps = (a.nv + kM6Step - 1) / kM6Step;
  const int last = tiles - (tiles - 1) / *tiles_wg * *tiles_wg;  // tiles of the last workgroup
  *slots_full = gemv6m_slots(*tiles_wg, *steps);
  *slots_last = gemv6m_slots(last, *steps);
  const size_t books = (size_t)16 * (a.bits2 ? 8192 : 4096);
  const size_t most = (size_t)*tiles_wg * *slots_full > (size_t)last * *slots_last ? (size_t)*tiles_wg * *slots_full
                                                                                   : (size_t)last * *slots_last;
  if (books + most * 1024 > 160u * 1024u) return false;
  // 32-bit buffer offsets over the index streams and x
  const uint64_t s1b = 4ull * (uint64_t)a.s1_words, s2b = 4ull * (uint64_t)a.s2_words;
  const uint64_t rows = (uint64_t)(tiles + 1) * 16;
  if (rows * s1b >= (1ull << 31) || rows * s2b >= (1ull << 31)) return false;
  return (uint64_t)16 * (uint64_t)a.in_features * 2u + 192ull * (uint64_t)*steps < (1ull << 31);
}

template <int RK>
vq_status launch_gemv6m(const ProductArgs& a, int tiles_wg, int steps, int slots_full, int slots_last,
                        hipStream_t s) {
  const int tiles = (a.n + 15) / 16;
  const unsigned grid = (unsigned)((tiles + tiles_wg - 1) / tiles_wg);
  hipLaunchKernelGGL(gemv6m_kernel<RK>, dim3(grid), dim3(kX6Threads), 0, s, a, tiles_wg, steps, slots_full,
                     slots_last);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int V, int MT, int XT, int IB1, int RK, int UQ>  // UQ: vectors per lane for MT <= 2
vq_status launch_fast(const ProductArgs& a, hipStream_t s) {
  // vectors in flight per lane: fewer for wide centroids and large batches (registers)
  constexpr int U0 = MT <= 2 ? UQ : (MT <= 8 ? 4 : 2);
  constexpr int U = V > 8 ? (U0 > 4 ? 4 : (U0 > 1 ? U0 / 2 : 1)) : U0;
  constexpr bool kLds1 = IB1 != 16;
  const size_t lds_bytes =
      16u * Cent<V>::kWords * ((kLds1 ? (1u << a.bits1) : 0u) + (RK == 1 ? (1u << a.bits2) : 0u));
  auto kern = gemv_kernel<V, MT, XT, IB1, RK, U>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return VQ_ERR_HIP;
  // Big LDS footprint: one 1024-thread workgroup per CU; otherwise smaller groups.  (The
  // 128-register budget of the 1024-thread bound costs a few bytes of spill in the
  // residual-book instances for M <= 2; measured, the occupancy it keeps is worth more.)
  const bool big = lds_bytes > 32 * 1024;
  const int block = big ? 1024 : VQ_GEMV_SMALL_BLOCK;
  const int per_cu = big ? 1 : VQ_GEMV_SMALL_PER_CU;
  const int waves_per_block = block / vqd::kWave;
  const long want = (a.n + waves_per_block - 1) / waves_per_block;
  const long cap = (long)kNumCU * per_cu;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(block), lds_bytes, s, a, block, (int)grid);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

template <int V, int XT, int IB1, int RK>
vq_status dispatch_m(const ProductArgs& a, hipStream_t s) {
  // M <= 2: a row of at most 512 vectors takes four per lane, so that it runs in two
  // steps with the second step's index loads in flight during the first one's gathers
  // (4096-column layers: 14.6 -> 14.1 us with one global book, 18.3 -> 17.0 with a residual
  // in LDS); longer rows, and two global books, keep eight (more gathers in flight)
  if (a.m <= 2) {
    if constexpr (V <= 8 && RK != 2)
      if (a.nv <= 512)
        return a.m <= 1 ? launch_fast<V, 1, XT, IB1, RK, 4>(a, s) : launch_fast<V, 2, XT, IB1, RK, 4>(a, s);
    return a.m <= 1 ? launch_fast<V, 1, XT, IB1, RK, VQ_GEMV_U1>(a, s)
                    : launch_fast<V, 2, XT, IB1, RK, VQ_GEMV_U1>(a, s);
  }
  if (a.m <= 4) return launch_fast<V, 4, XT, IB1, RK, 0>(a, s);
  if (a.m <= 8) return launch_fast<V, 8, XT, IB1, RK, 0>(a, s);
  return launch_fast<V, 16, XT, IB1, RK, 0>(a, s);
}

// Book placements with a fast kernel (checked by launch_gemv): main book global (16-bit)
// or in LDS; second book none, in LDS, or global with 16-bit indices when the main book is
// global too.  v = 16 only with the global 65536-entry main book.
template <int V, int XT>
vq_status dispatch_books(const ProductArgs& a, hipStream_t s) {
  const bool main16 = a.bits1 == 16;
  if constexpr (V == 6) {
    // fp16 activations, decode batches, both books in LDS (with room for the index areas)
    // one batch row, 12-bit fields, IN a multiple of 8 and a 16-byte aligned x: x in LDS too
    if (XT == 0 && a.m == 1 && a.bits1 == 12 && (a.bits2 == 0 || a.bits2 == 12) && a.in_features % 8 == 0 &&
        vqi::aligned(a.x, 16)) {
      const int rows = gemv6x_rows(a);
      if (rows > 0) return a.bits2 ? launch_gemv6x<1>(a, rows, s) : launch_gemv6x<0>(a, rows, s);
    }
    // 2..16 batch rows, 12-bit fields, IN a multiple of 8 and a 16-byte aligned x: matrix cores
    if (XT == 0 && a.m >= 2 && a.m <= 16 && a.bits1 == 12 && (a.bits2 == 0 || a.bits2 == 12) &&
        a.in_features % 8 == 0 && vqi::aligned(a.x, 16)) {
      int tw = 0, st = 0, sf = 0, sl = 0;
      if (gemv6m_plan(a, &tw, &st, &sf, &sl))
        return a.bits2 ? launch_gemv6m<1>(a, tw, st, sf, sl, s) : launch_gemv6m<0>(a, tw, st, sf, sl, s);
    }
    if (XT == 0 && a.m <= 2 && !main16 && a.in_features >= 6 && a.n <= 64 * 16 * kNumCU &&
        gemv6_lds(4, a.bits1, a.bits2) <= 160u * 1024u) {
      return a.bits2 ? dispatch_gemv6<1>(a, s) : dispatch_gemv6<0>(a, s);
    }
    if (a.bits2) return main16 ? dispatch_m<V, XT, 16, 1>(a, s) : dispatch_m<V, XT, 0, 1>(a, s);
    return main16 ? dispatch_m<V, XT, 16, 0>(a, s) : dispatch_m<V, XT, 0, 0>(a, s);
  } else if constexpr (V == 16) {
    if (a.bits2 == 16) return dispatch_m<V, XT, 16, 2>(a, s);
    return a.bits2 ? dispatch_m<V, XT, 16, 1>(a, s) : dispatch_m<V, XT, 16, 0>(a, s);
  } else {
    if (a.bits2 == 16) return dispatch_m<V, XT, 16, 2>(a, s);
    if (a.bits2) return main16 ? dispatch_m<V, XT, 16, 1>(a, s) : dispatch_m<V, XT, 0, 1>(a, s);
    return main16 ? dispatch_m<V, XT, 16, 0>(a, s) : dispatch_m<V, XT, 0, 0>(a, s);
  }
}

template <int V>
vq_status dispatch_x(const ProductArgs& a, hipStream_t s) {
  return a.x_dtype == VQ_BF16 ? dispatch_books<V, 1>(a, s) : dispatch_books<V, 0>(a, s);
}

}  // namespace

namespace vqi {

vq_status launch_gemv(const ProductArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  // The fast path: v in {6, 8, 16}; the main book either has 16-bit indices (global) or
  // at most 4096 entries (LDS, not for v = 16); the second book none, at most 4096 entries
  // (LDS), or 65536 entries (global) beside a global main book (v = 8, 16); both LDS
  // books within 160 KiB; vector-aligned codebooks and x rows, IN a multiple of 8
  // (v = 8, 16) or even (v = 6).
  const size_t align = (a.v == 6) ? 4 : 16;
  const bool v_ok = a.v == 6 || a.v == 8 || a.v == 16;
  const bool b1_ok = a.bits1 == 16 || (a.bits1 <= 12 && a.v != 16);
  const bool b2_ok = a.bits2 <= 12 || (a.bits2 == 16 && a.bits1 == 16 && a.v != 6);
  const size_t words = a.v > 8 ? 2 : 1;  // 16-byte LDS words per centroid
  const size_t lds_need = 16u * words * ((a.bits1 <= 12 ? (1u << a.bits1) : 0u) +
                                         (a.bits2 >= 1 && a.bits2 <= 12 ? (1u << a.bits2) : 0u));
  const bool fast_shape = v_ok && b1_ok && b2_ok && lds_need <= 160u * 1024u && a.in_features >= 8;
  const bool fast_align = aligned(a.cb1, align) && (!a.cb2 || aligned(a.cb2, align)) && aligned(a.x, align) &&
                          (((size_t)a.in_features * 2) % align == 0);
  if (fast_shape && fast_align) {
    if (a.v == 16) return dispatch_x<16>(a, s);
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
