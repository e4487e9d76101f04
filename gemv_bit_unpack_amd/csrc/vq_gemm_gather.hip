// vq_gemm_ws: the prefill product for the 65536-entry main codebook (v = 8, 16-bit
// indices, residual book of 0 or 8 bits), with the rebuilt weights fed to the matrix
// cores straight from the lanes that gather them.
//
// In v_mfma_f32_32x32x16_f16 each lane supplies 8 consecutive k of one column of the B
// operand, which is exactly one rebuilt weight vector (v = 8).  So a lane gathers its
// vector's main centroid (16 bytes, served by L2: the 1 MiB book does not fit in LDS),
// adds the residual centroid read from LDS in fp16 (one rounding of the exact sum, the
// same value as rounding the fp32 sum), and passes the vector to the matrix core: no
// weight tile goes through LDS and each vector is rebuilt once per batch chunk of 128
// rows.  The A operand is the activation tile (batch rows x 16 k), held in LDS and shared
// by the workgroup's 7 or 8 wavefronts.
//   - workgroup: 224 or 256 output rows (wavefront w owns rows 32w .. 32w + 31, lane l the
//     row l % 32) x one batch chunk (<= 128 rows) x one range of K-tiles (a K split);
//   - K-tile: 16 vectors (128 columns) per row; lane l supplies vectors 8 (l / 32) ..
//     8 (l / 32) + 7 of it, one per matrix step, so its 8 indices are one 16-byte load and
//     its 8 residual indices one 8-byte load;
//   - pipelining: while tile t is multiplied, the centroids of tile t + 1, the indices of
//     tile t + 2 and the activations of tile t + 1 are in flight; one barrier per tile
//     (the activation tile is double-buffered in LDS);
//   - output: with one K split the workgroup writes y (2^e of the batch row, scale, bias);
//     with several it writes fp32 partial sums, added in a fixed order by a second kernel.
// The production-VQ post ("1. Prefill vs. Decode Bottlenecks") places prefill in the
// compute-bound regime; with a 65536-entry book the bound here is the L2's rate of random
// 16-byte lookups, one per weight vector and batch chunk ("Lookup Table (LUT) Overhead vs.
// Bit-Shifting").  bf16 activations are first rewritten as fp16 times a power of two per
// batch row (the pass the codebook-sliced GEMV uses), so one fp16 matrix instruction
// serves each step.
#include "vq_device.h"

namespace {

using vqi::ProductArgs;

constexpr int kRowsWG = 256;   // output rows per workgroup at most (8 wavefronts)
constexpr int kTileV = 16;     // vectors per K-tile
constexpr int kMC = 128;       // batch rows per chunk
constexpr int kXRow = 17;      // 16-byte units per batch row of an activation tile (16 + 1 pad)
constexpr int kRes = 256;      // residual centroids (8-bit indices)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct GatherCfg {
  int32_t n_rb;         // row blocks of 32 * WV rows
  int32_t ks;           // K splits
  int32_t tps;          // K-tiles per split (even)
  int32_t n_kt;         // K-tiles of 16 vectors
  float* part;          // [ks][M][N] partial sums (ks > 1)
  const uint16_t* x16;  // fp16 activations [M][IN]
  const int32_t* xexp;  // [M] powers of two taken out of bf16 rows, or nullptr
};

// Raw buffer resource over n bytes at p: loads of dwords outside [0, n) return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ uint32_t add2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b));
}

// Byte offset (times 16) of 16-bit field h of w: one SDWA shift.
template <int H>
__device__ __forceinline__ uint32_t word_x16(uint32_t w) {
  uint32_t r;
  if constexpr (H == 0) {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_0"
        : "=v"(r) : "v"(w));
  } else {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(r) : "v"(w));
  }
  return r;
}
template <int B>
__device__ __forceinline__ uint32_t byte_x16(uint32_t w) {
  uint32_t r;
  if constexpr (B == 0) {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  } else if constexpr (B == 1) {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  } else if constexpr (B == 2) {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  } else {
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  }
  return r;
}

// The 8 main centroids of one K-tile: buffer loads at index * 16 in the book.
__device__ __forceinline__ void gather8(__amdgpu_buffer_rsrc_t bc, const uint4& iw, uint4 (&c)[8]) {
  c[0] = ld16(bc, word_x16<0>(iw.x), 0);
  c[1] = ld16(bc, word_x16<1>(iw.x), 0);
  c[2] = ld16(bc, word_x16<0>(iw.y), 0);
  c[3] = ld16(bc, word_x16<1>(iw.y), 0);
  c[4] = ld16(bc, word_x16<0>(iw.z), 0);
  c[5] = ld16(bc, word_x16<1>(iw.z), 0);
  c[6] = ld16(bc, word_x16<0>(iw.w), 0);
  c[7] = ld16(bc, word_x16<1>(iw.w), 0);
}

// WV wavefronts (7 or 8) per workgroup, one per 32 output rows: the host picks the count
// that makes row blocks x K splits fill the CUs.
template <int NB, bool RES, int WV>
__global__ __launch_bounds__(512) void gemm_gather_kernel(ProductArgs a, GatherCfg g) {
  constexpr int kThreadsW = 64 * WV;
  constexpr int kXPass = kThreadsW / 16;                // activation rows staged per pass
  constexpr int kXP = (32 * NB + kXPass - 1) / kXPass;  // passes over the chunk's 32 NB rows
  constexpr int kXBuf = 32 * NB * kXRow;  // 16-byte units per activation buffer
  constexpr int kResAt = 0;
  constexpr int kXAt = RES ? kRes : 0;
  __shared__ uint4 lds[kXAt + 2 * kXBuf];
  __shared__ int32_t sexp[kMC];
  uint4* const xt = lds + kXAt;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = lane >> 5;
  const int l32 = lane & 31;
  const int split = (int)(blockIdx.x % (unsigned)g.ks);
  const int rest = (int)(blockIdx.x / (unsigned)g.ks);
  const int rb = rest % g.n_rb;
  const int mc = rest / g.n_rb;
  const int kt0 = split * g.tps;
  const int kt1 = min(kt0 + g.tps, g.n_kt);
  const int row = rb * 32 * WV + wave * 32 + l32;
  const int m0 = mc * kMC;
  const int M = a.m, N = a.n, IN = a.in_features;
  const uint32_t s1b = (uint32_t)a.s1_words * 4u;
  const uint32_t s2b = (uint32_t)a.s2_words * 4u;

  // Rows past N and batch rows past M read as zero through the buffer bounds.
  const __amdgpu_buffer_rsrc_t b1 = span(a.packed1, (uint32_t)N * s1b);
  const __amdgpu_buffer_rsrc_t b2 = span(RES ? (const void*)a.packed2 : (const void*)a.packed1,
                                         RES ? (uint32_t)N * s2b : 0u);
  const __amdgpu_buffer_rsrc_t bc = span(a.cb1, 65536u * 16u);
  const __amdgpu_buffer_rsrc_t bx = span(g.x16, (uint32_t)M * (uint32_t)IN * 2u);
  const uint32_t v_idx = (uint32_t)row * s1b + (uint32_t)kg * 16u;
  const uint32_t v_res = (uint32_t)row * s2b + (uint32_t)kg * 8u;
  // activation staging: thread tid moves 16-byte unit tid % 16 of batch rows
  // tid / 16 + kXPass h (rows past the chunk's 32 NB are not stored)
  const int xr = tid >> 4, xu = tid & 15;
  uint32_t v_x[kXP];
#pragma unroll
  for (int h = 0; h < kXP; ++h)
    v_x[h] = ((uint32_t)(m0 + xr + kXPass * h) * (uint32_t)IN + (uint32_t)xu * 8u) * 2u;

  auto load_x = [&](int kt, uint4 (&xs)[kXP]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < kXP; ++h) xs[h] = ld16(bx, v_x[h], (uint32_t)kt * (kTileV * 16u));
  };
  // columns past IN (a ragged last tile) must be zero: they would read the next batch row.
  // A mask, not a select: a branch here would make the compiler wait for every load in
  // flight where the paths join.
  auto store_x = [&](int kt, int buf, uint4 (&xs)[kXP]) __attribute__((always_inline)) {
    const uint32_t keep = 0u - (uint32_t)(kt * (kTileV * 8) + xu * 8 < IN);
#pragma unroll
    for (int h = 0; h < kXP; ++h) {
      if (kXPass * kXP == 32 * NB || xr + kXPass * h < 32 * NB) {
        xt[buf * kXBuf + (xr + kXPass * h) * kXRow + xu] =
            make_uint4(xs[h].x & keep, xs[h].y & keep, xs[h].z & keep, xs[h].w & keep);
      }
    }
  };

  // prologue: the residual book and the batch rows' powers of two (for LDS); the first
  // tile's indices and activations; then, in the order every tile leaves them in flight,
  // the next tile's indices, the first tile's residual indices and its centroids
  const uint4 rbk = (RES && tid < kRes) ? ((const uint4*)a.cb2)[tid] : make_uint4(0u, 0u, 0u, 0u);
  const int32_t ex = (tid < kMC && g.xexp) ? g.xexp[min(m0 + tid, M - 1)] : 0;
  uint4 iwA = ld16(b1, v_idx, (uint32_t)kt0 * (kTileV * 2u));
  uint4 xs[kXP];
  load_x(kt0, xs);
  __builtin_amdgcn_sched_barrier(0);
  uint4 iwB = ld16(b1, v_idx, (uint32_t)min(kt0 + 1, kt1 - 1) * (kTileV * 2u));
  uint2 irA = RES ? ld8(b2, v_res, (uint32_t)kt0 * kTileV) : make_uint2(0u, 0u);
  uint2 irB = irA;
  uint4 cA[8], cB[8];
  gather8(bc, iwA, cA);
  __builtin_amdgcn_sched_barrier(0);
  if (RES && tid < kRes) lds[kResAt + tid] = rbk;
  if (tid < kMC) sexp[tid] = ex;
  store_x(kt0, 0, xs);
  __syncthreads();

  float16_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.0f;
  }

  // One K-tile: kt is multiplied from cur (its centroids, gathered one tile earlier) and
  // activation buffer buf; the centroids of the next tile are gathered into nxt from iwn,
  // the indices two tiles ahead are loaded into iwl, the residual indices of the next tile
  // into irn.  Prefetches past the split's last tile re-read that tile (no branch).
  auto tile = [&](int kt, int buf, uint4 (&cur)[8], uint4 (&nxt)[8], const uint4& iwn, uint4& iwl, const uint2& irc,
                  uint2& irn) __attribute__((always_inline)) {
    const int kn = min(kt + 1, kt1 - 1);
    const int kn2 = min(kt + 2, kt1 - 1);
    __builtin_amdgcn_sched_barrier(0);  // nothing of this tile moves into the previous one
    load_x(kn, xs);
    iwl = ld16(b1, v_idx, (uint32_t)kn2 * (kTileV * 2u));
    if constexpr (RES) irn = ld8(b2, v_res, (uint32_t)kn * kTileV);
    gather8(bc, iwn, nxt);
    __builtin_amdgcn_sched_barrier(0);
    const uint4* xb = xt + buf * kXBuf + l32 * kXRow + kg * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 w = cur[s];
      if constexpr (RES) {
        const uint32_t rw = s < 4 ? irc.x : irc.y;
        uint32_t ra;
        switch (s & 3) {
          case 0: ra = byte_x16<0>(rw); break;
          case 1: ra = byte_x16<1>(rw); break;
          case 2: ra = byte_x16<2>(rw); break;
          default: ra = byte_x16<3>(rw); break;
        }
        const uint4 c2 = *(const uint4*)((const char*)(lds + kResAt) + ra);
        w = make_uint4(add2(w.x, c2.x), add2(w.y, c2.y), add2(w.z, c2.z), add2(w.w, c2.w));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint4 xa = xb[nb * 32 * kXRow + s];
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, xa),
                                                         __builtin_bit_cast(half8_t, w), acc[nb], 0, 0, 0);
      }
    }
    store_x(kn, buf ^ 1, xs);
    __syncthreads();
  };

  // Tiles in pairs (the two register sets in turn, no copies); an odd last tile after the
  // loop, so the loop body has no branch (a branch there makes the compiler wait at the top
  // of the loop for the centroids still in flight).
  int kt = kt0;
  for (; kt + 1 < kt1; kt += 2) {
    tile(kt, 0, cA, cB, iwB, iwA, irA, irB);
    tile(kt + 1, 1, cB, cA, iwA, iwB, irB, irA);
  }
  if (kt < kt1) tile(kt, 0, cA, cB, iwB, iwA, irA, irB);

  // Epilogue: accumulator register r of lane l holds batch row 8 (r / 4) + 4 (l / 32) +
  // r % 4 of block nb, output row `row`.
  if (row >= N) return;
  if (g.ks == 1) {
    const float sc = a.scale ? vqd::f16_to_f32(a.scale[row]) : 1.0f;
    const float bi = a.bias ? vqd::f16_to_f32(a.bias[row]) : 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mi = 32 * nb + 8 * (r >> 2) + 4 * kg + (r & 3);
        const int m = m0 + mi;
        if (m < M) {
          float out = acc[nb][r];
          if (g.xexp) out = ldexpf(out, sexp[mi]);
          if (a.scale) out = out * sc;
          if (a.bias) out = out + bi;
          vqd::store_out(a.y, (size_t)m * N + row, out, a.y_dtype);
        }
      }
    }
  } else {
    float* p = g.part + (size_t)split * M * N + row;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * nb + 8 * (r >> 2) + 4 * kg + (r & 3);
        if (m < M) p[(size_t)m * N] = acc[nb][r];
      }
    }
  }
}

struct Plan {
  GatherCfg cfg;
  int nb, wv;
  size_t x16_off, exp_off, part_off, bytes;
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Row blocks of 32 WV rows x batch chunks; the K range is split (into an even number of
// tiles per split) until about three quarters of the CUs have a workgroup, keeping at
// least two tiles per split.  WV is 8, or 7 when that fills the 256 CUs in fewer rounds'
// worth of idle CUs (the 28672-row layer: 128 blocks of 224 rows x 2 splits = 256
// workgroups, against 112 x 2 = 224 with 8).
Plan make_plan(int32_t n, int32_t in_features, int32_t m, bool bf16, bool rht = false) {
  Plan p{};
  GatherCfg& g = p.cfg;
  const int nv = in_features / 8;
  g.n_kt = (nv + kTileV - 1) / kTileV;
  const int n_mc = (m + kMC - 1) / kMC;
  long best_idle = -1;
  for (int wv = 8; wv >= 7; --wv) {
    const int n_rb = (n + 32 * wv - 1) / (32 * wv);
    const int base = n_rb * n_mc;
    int ks = 1;
    while (base * ks < 192 && ks < 16 && g.n_kt >= 4 * ks) ks *= 2;
    int tps = (g.n_kt + ks - 1) / ks;
    tps += tps & 1;
    const int ks_eff = (g.n_kt + tps - 1) / tps;
    const long units = (long)base * ks_eff;
    const long idle = (units + 255) / 256 * 256 - units;  // CU slots left empty in the last round
    if (best_idle < 0 || idle < best_idle) {
      best_idle = idle;
      p.wv = wv;
      g.n_rb = n_rb;
      g.tps = tps;
      g.ks = ks_eff;
    }
  }
  const int mr = m < kMC ? m : kMC;
  p.nb = (mr + 31) / 32;
  p.x16_off = 0;
  const bool pass = bf16 || rht;  // an x pass writes the fp16 copy and the powers of two
  p.exp_off = pass ? round256((size_t)m * in_features * 2) : 0;
  p.part_off = p.exp_off + (pass ? round256((size_t)m * sizeof(int32_t)) : 0);
  p.bytes = p.part_off + (g.ks > 1 ? round256((size_t)g.ks * m * n * sizeof(float)) : 0);
  return p;
}

template <bool RES, int WV>
vq_status launch_nb(const ProductArgs& a, const GatherCfg& g, int nb, int n_mc, hipStream_t s) {
  const unsigned grid = (unsigned)g.ks * (unsigned)g.n_rb * (unsigned)n_mc;
  const dim3 block(64 * WV);
  switch (nb) {
    case 1: hipLaunchKernelGGL((gemm_gather_kernel<1, RES, WV>), dim3(grid), block, 0, s, a, g); break;
    case 2: hipLaunchKernelGGL((gemm_gather_kernel<2, RES, WV>), dim3(grid), block, 0, s, a, g); break;
    case 3: hipLaunchKernelGGL((gemm_gather_kernel<3, RES, WV>), dim3(grid), block, 0, s, a, g); break;
    default: hipLaunchKernelGGL((gemm_gather_kernel<4, RES, WV>), dim3(grid), block, 0, s, a, g); break;
  }
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace

namespace vqi {

bool gather_gemm_shape_ok(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (d.v != 8 || d.bits1 != 16 || !(d.bits2 == 0 || d.bits2 == 8)) return false;
  if (m < 1 || !(x_dtype == VQ_F16 || x_dtype == VQ_BF16)) return false;
  if (d.in_features < 8 || d.in_features % 8 != 0 || d.out_features < 1) return false;
  // 32-bit buffer offsets: every row block's last row and every batch chunk's last row
  const uint64_t s1 = (uint64_t)row_stride(d.in_features, 8, 16);
  const uint64_t s2 = (uint64_t)row_stride(d.in_features, 8, d.bits2);
  const uint64_t rows = (uint64_t)d.out_features + kRowsWG;
  if (rows * s1 >= ((uint64_t)1 << 32) || rows * s2 >= ((uint64_t)1 << 32)) return false;
  if (((uint64_t)m + kMC + 32) * (uint64_t)d.in_features * 2u >= ((uint64_t)1 << 32)) return false;
  return true;
}

size_t gather_gemm_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (!gather_gemm_shape_ok(d, m, x_dtype)) return 0;
  return make_plan(d.out_features, d.in_features, m, x_dtype == VQ_BF16).bytes;
}

bool gather_gemm_pointers_ok(const ProductArgs& a) {
  return aligned(a.packed1, 16) && aligned(a.cb1, 16) && (a.bits2 == 0 || aligned(a.cb2, 16)) && aligned(a.x, 16);
}

size_t gather_gemm_rht_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype) {
  if (!gather_gemm_shape_ok(d, m, x_dtype) || d.in_features > kFusedRhtMaxIn || d.in_features % 16 != 0) return 0;
  return make_plan(d.out_features, d.in_features, m, x_dtype == VQ_BF16, true).bytes;
}

vq_status launch_gemm_gather(const ProductArgs& a, void* workspace, void* stream, const uint8_t* rht_signs) {
  const bool bf16 = a.x_dtype == VQ_BF16;
  Plan p = make_plan(a.n, a.in_features, a.m, bf16, rht_signs != nullptr);
  if (p.bytes > 0 && !workspace) return VQ_ERR_NULL;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  p.cfg.part = p.cfg.ks > 1 ? (float*)(ws + p.part_off) : nullptr;
  if (bf16 || rht_signs) {
    uint16_t* x16 = (uint16_t*)(ws + p.x16_off);
    int32_t* xexp = (int32_t*)(ws + p.exp_off);
    const vq_status st = rht_signs ? launch_x_rht_to_f16(a, rht_signs, x16, xexp, stream)
                                   : launch_x_to_f16(a, x16, xexp, stream);
    if (st != VQ_OK) return st;
    p.cfg.x16 = x16;
    p.cfg.xexp = xexp;
  } else {
    p.cfg.x16 = a.x;
    p.cfg.xexp = nullptr;
  }
  const int n_mc = (a.m + kMC - 1) / kMC;
  const vq_status st = a.bits2 == 8 ? (p.wv == 7 ? launch_nb<true, 7>(a, p.cfg, p.nb, n_mc, s)
                                                  : launch_nb<true, 8>(a, p.cfg, p.nb, n_mc, s))
                                     : (p.wv == 7 ? launch_nb<false, 7>(a, p.cfg, p.nb, n_mc, s)
                                                  : launch_nb<false, 8>(a, p.cfg, p.nb, n_mc, s));
  if (st != VQ_OK || p.cfg.ks == 1) return st;
  return launch_partials_finalize(a, p.cfg.part, p.cfg.xexp, p.cfg.ks, stream);
}

}  // namespace vqi
