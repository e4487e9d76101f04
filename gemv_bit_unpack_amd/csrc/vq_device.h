// Device helpers shared by the gfx950 kernels of libvq: index bit-unpacking, 16-bit
// float conversions and output stores.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "vq_internal.h"

namespace vqd {

constexpr int kWave = 64;

// Field j (bits [j*bits, (j+1)*bits), LSB-first) of a row of 32-bit words.  The field
// always lies inside the row; the second word is read only when it exists, so the last
// field of the last row never reads past the buffer.  One funnel shift and one mask.
__device__ __forceinline__ uint32_t extract_index(const uint32_t* __restrict__ row, int32_t row_words, uint32_t j,
                                                  uint32_t bits) {
  const uint32_t bitpos = j * bits;
  const uint32_t w = bitpos >> 5;
  const uint32_t lo = row[w];
  const uint32_t hi = ((int32_t)w + 1 < row_words) ? row[w + 1] : 0u;
  return __builtin_amdgcn_alignbit(hi, lo, bitpos & 31u) & ((1u << bits) - 1u);
}

// Exact widening of IEEE binary16 bits.
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xFFFFu));
}
// Exact widening of bfloat16 bits (bfloat16 is the upper half of a binary32).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __builtin_bit_cast(float, bits16 << 16); }

template <int XT>  // 0: fp16, 1: bf16
__device__ __forceinline__ float x_to_f32(uint32_t bits16) {
  if constexpr (XT == 0) {
    return f16_to_f32(bits16);
  } else {
    return bf16_to_f32(bits16);
  }
}

// Round-to-nearest-even fp32 -> bfloat16 bits (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
// Round-to-nearest-even fp32 -> binary16 bits (hardware conversion, RNE mode).
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}

__device__ __forceinline__ void store_out(void* y, size_t i, float r, vq_dtype t) {
  if (t == VQ_F32) {
    ((float*)y)[i] = r;
  } else if (t == VQ_F16) {
    ((uint16_t*)y)[i] = f32_to_f16_rne(r);
  } else {
    ((uint16_t*)y)[i] = f32_to_bf16_rne(r);
  }
}

}  // namespace vqd
