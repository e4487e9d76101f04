// Internal declarations shared by the host and device translation units of libvq.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "vq.h"

namespace vqi {

// Number of v-wide vectors per row; the last one may be partial.
inline int64_t num_vectors(int64_t in_features, int v) { return (in_features + v - 1) / v; }

// Bytes of one row of an index stream of `bits`-bit fields: 16-byte padded.
inline int64_t row_stride(int64_t in_features, int v, int bits) {
  if (bits == 0) return 0;
  const int64_t nbits = num_vectors(in_features, v) * bits;
  return 16 * ((nbits + 127) / 128);
}

// Validates the descriptor fields (not pointers) of a row-stream layer: VQ_OK or the error
// code (any other layout is VQ_ERR_UNSUPPORTED).
vq_status check_desc(const vq_desc* d);
// The same, also accepting the slice-bucketed layout where it is defined (v = 8,
// bits1 = 16, bits2 0 or 8, IN a multiple of 8, within the 32-bit offsets of its product).
vq_status check_desc_any(const vq_desc* d);

// Slice-bucketed layout: vectors per chunk, and the bytes of its prefix table (8 * chunks
// * N + 1 uint32 bucket offsets, padded to 256 bytes) ahead of the 32-bit bucket words.
constexpr int32_t kBucketChunk = 1024;
inline int64_t bucketed_chunks(const vq_desc& d) {
  return (num_vectors(d.in_features, 8) + kBucketChunk - 1) / kBucketChunk;
}
inline size_t bucketed_header_bytes(const vq_desc& d) {
  const size_t starts = (size_t)(8 * bucketed_chunks(d)) * (size_t)d.out_features + 1;
  return (starts * 4 + 255) / 256 * 256;
}

// Packed size in bytes of a validated descriptor.
inline size_t packed_size(const vq_desc& d) {
  if (d.layout == VQ_LAYOUT_BUCKETED)
    return bucketed_header_bytes(d) + 4 * (size_t)d.out_features * (size_t)num_vectors(d.in_features, 8);
  return (size_t)d.out_features *
         (size_t)(row_stride(d.in_features, d.v, d.bits1) + row_stride(d.in_features, d.v, d.bits2));
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Arguments of every product launch (gemv and gemm), after validation.
struct ProductArgs {
  int32_t n, in_features, v, bits1, bits2, nv;
  int32_t s1_words, s2_words;  // row strides in 32-bit words
  const uint32_t* packed1;     // stream 1
  const uint32_t* packed2;     // stream 2 or nullptr
  const uint16_t* cb1;         // fp16 bits [K1][v]
  const uint16_t* cb2;         // fp16 bits [K2][v] or nullptr
  const uint16_t* scale;       // fp16 bits [n] or nullptr
  const uint16_t* bias;        // fp16 bits [n] or nullptr
  const uint16_t* x;           // [M][in] fp16 / bf16 bits
  void* y;                     // [M][n]
  int32_t m;
  vq_dtype x_dtype, y_dtype;
};

// Validates a product call; on success fills `a`.  `max_m` bounds M (0: unbounded).
vq_status prepare_product(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                          const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t m, void* y,
                          vq_dtype y_dtype, int32_t max_m, ProductArgs* a);

// Launchers (defined in the .hip units).  Return VQ_OK or VQ_ERR_HIP / VQ_ERR_UNSUPPORTED.
vq_status launch_dequant(const vq_desc& d, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         void* w, vq_dtype w_dtype, void* stream);
vq_status launch_gemv(const ProductArgs& a, void* stream);
// The codebook-sliced GEMV (65536-entry main book, v = 8, 1 <= M <= 16) that runs with a
// caller-owned workspace: whether the shape has that path and the workspace it needs (0:
// none), whether the pointers allow it, and the launch.
bool sliced_gemv_shape_ok(const vq_desc& d, int32_t m, vq_dtype x_dtype);
size_t sliced_gemv_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype);
bool sliced_gemv_pointers_ok(const ProductArgs& a);
// rht_signs: also the randomized Hadamard transform of x (forward, blocks of rht_block(IN))
// in the x pass; then the workspace is sliced_gemv_rht_workspace(...) bytes.
vq_status launch_gemv_sliced(const ProductArgs& a, void* workspace, void* stream, const uint8_t* rht_signs = nullptr);
size_t sliced_gemv_rht_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype);
// The product over the slice-bucketed layout (M = 1): whether the descriptor's sizes fit
// its 32-bit offsets, its workspace bytes, and the launch (packed1 = the prefix table,
// packed2 = the bucket words, nv = IN / 8).
bool bucketed_gemv_shape_ok(const vq_desc& d);
size_t bucketed_gemv_workspace(const vq_desc& d);
vq_status launch_gemv_bucketed(const ProductArgs& a, void* workspace, void* stream);
// The fixed device workspace of vq_gemv_noalloc: its size, and this GPU's copy (looked up
// on the first call on each device; no allocation).
size_t static_scratch_bytes();
vq_status static_scratch(void** ptr);
vq_status launch_gemm(const ProductArgs& a, void* stream);
// The prefill product for the same 65536-entry book (vq_gemm_ws): shape test, workspace
// bytes (0: none needed), pointer test and launch.
bool gather_gemm_shape_ok(const vq_desc& d, int32_t m, vq_dtype x_dtype);
size_t gather_gemm_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype);
bool gather_gemm_pointers_ok(const ProductArgs& a);
vq_status launch_gemm_gather(const ProductArgs& a, void* workspace, void* stream, const uint8_t* rht_signs = nullptr);
size_t gather_gemm_rht_workspace(const vq_desc& d, int32_t m, vq_dtype x_dtype);
// Passes shared by the workspace products: bf16 activations rewritten as fp16 times a
// power of two per batch row (x16 [M][IN], xexp [M]); and y = 2^e * scale * (sum of
// `nparts` fp32 partial sums [nparts][M][N], in order) + bias.
vq_status launch_x_to_f16(const ProductArgs& a, uint16_t* x16, int32_t* xexp, void* stream);
// The same pass with the forward randomized Hadamard transform first (IN a multiple of 16,
// at most 32768; VQ_ERR_UNSUPPORTED otherwise).
vq_status launch_x_rht_to_f16(const ProductArgs& a, const uint8_t* signs, uint16_t* x16, int32_t* xexp, void* stream);
constexpr int32_t kFusedRhtMaxIn = 32768;
vq_status launch_partials_finalize(const ProductArgs& a, const float* part, const int32_t* xexp, int nparts,
                                   void* stream);

// Affine-lattice layers (v = 4, one 8-bit field of four 2-bit codes per vector), after
// validation.
struct SvqArgs {
  int32_t n, in_features, nv, stride;  // stride: bytes per row of the code stream
  const uint8_t* packed;
  const uint16_t* a;      // fp16 bits [4][4], A[t][u]
  const uint16_t* b;      // fp16 bits [4]
  const uint16_t* scale;  // fp16 bits [n] or nullptr
  const uint16_t* bias;   // fp16 bits [n] or nullptr
  const uint16_t* x;      // [M][in] fp16 / bf16 bits
  void* y;                // [M][n]
  int32_t m;
  vq_dtype x_dtype, y_dtype;
  int32_t x_vec4;  // IN % 4 == 0 and x 8-byte aligned: x read one 4-vector per load
};
vq_status launch_svq_gemv(const SvqArgs& p, void* stream);
vq_status launch_svq_gemm(const SvqArgs& p, void* stream);
// Randomized Hadamard transform (validated arguments; n a multiple of 16, m >= 1).
int32_t rht_block(int32_t n);
vq_status launch_rht(int32_t m, int32_t n, const void* x, vq_dtype x_dtype, const uint8_t* signs, int32_t transpose,
                     void* y, vq_dtype y_dtype, void* stream);
vq_status launch_svq_dequant(const SvqArgs& p, void* w, vq_dtype w_dtype, void* stream);
// Residual VQ encode (validated arguments: IN % v == 0, N * IN / v >= 1, workspace of at
// least assign_workspace(d) bytes, 256-byte aligned).
size_t assign_workspace(const vq_desc& d);
vq_status launch_assign(const vq_desc& d, const void* w, vq_dtype w_dtype, const uint16_t* cb1, const uint16_t* cb2,
                        uint32_t* idx1, uint32_t* idx2, void* workspace, void* stream);

}  // namespace vqi
