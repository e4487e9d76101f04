// vq_dequant: writes the rebuilt weight matrix W^ [N][IN] (diagnostic, untimed).
//
// Decode as in the VPTQ guide's residual formula ("2. Multi-Stage Residual Vector
// Quantization (RVQ)") and its "Step 2" dequantize: per vector, the main centroid plus
// the residual centroid, summed in fp32 (round to nearest even), then multiplied by the
// output channel's scale in fp32.  No fused multiply-add is formed (the unit is built
// with -ffp-contract=off), fp32 subnormals are kept, so the fp32 result is unique and
// fp16 / bf16 outputs are its nearest-even rounding.
#include "vq_device.h"

namespace {

struct DequantArgs {
  int32_t n, in_features, v, bits1, bits2, nv, s1_words, s2_words;
  const uint32_t* packed1;
  const uint32_t* packed2;
  const uint16_t* cb1;
  const uint16_t* cb2;
  const uint16_t* scale;
  void* w;
  vq_dtype w_dtype;
};

// One thread per (row, vector) slot; grid-stride over all N * nv slots.  Consecutive
// threads take consecutive vectors of a row, so the index reads and the v-wide output
// writes of a wavefront are contiguous.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const size_t total = (size_t)a.n * (size_t)a.nv;
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t slot = (size_t)blockIdx.x * blockDim.x + threadIdx.x; slot < total; slot += step) {
    const int32_t row = (int32_t)(slot / (size_t)a.nv);
    const uint32_t j = (uint32_t)(slot - (size_t)row * (size_t)a.nv);
    const uint32_t i1 = vqd::extract_index(a.packed1 + (size_t)row * a.s1_words, a.s1_words, j, a.bits1);
    uint32_t i2 = 0;
    if (a.bits2) i2 = vqd::extract_index(a.packed2 + (size_t)row * a.s2_words, a.s2_words, j, a.bits2);
    const float s = a.scale ? vqd::f16_to_f32(a.scale[row]) : 1.0f;
    const int32_t col0 = (int32_t)j * a.v;
    const int32_t nt = min(a.v, a.in_features - col0);
    for (int32_t t = 0; t < nt; ++t) {
      float w = vqd::f16_to_f32(a.cb1[(size_t)i1 * a.v + t]);
      if (a.bits2) w = w + vqd::f16_to_f32(a.cb2[(size_t)i2 * a.v + t]);
      if (a.scale) w = w * s;
      vqd::store_out(a.w, (size_t)row * a.in_features + col0 + t, w, a.w_dtype);
    }
  }
}

}  // namespace

namespace vqi {

vq_status launch_dequant(const vq_desc& d, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         void* w, vq_dtype w_dtype, void* stream) {
  DequantArgs a;
  a.n = d.out_features;
  a.in_features = d.in_features;
  a.v = d.v;
  a.bits1 = d.bits1;
  a.bits2 = d.bits2;
  a.nv = (int32_t)num_vectors(d.in_features, d.v);
  const int64_t s1 = row_stride(d.in_features, d.v, d.bits1);
  a.s1_words = (int32_t)(s1 / 4);
  a.s2_words = (int32_t)(row_stride(d.in_features, d.v, d.bits2) / 4);
  a.packed1 = (const uint32_t*)packed;
  a.packed2 = d.bits2 ? (const uint32_t*)((const uint8_t*)packed + (size_t)d.out_features * (size_t)s1) : nullptr;
  a.cb1 = (const uint16_t*)cb1;
  a.cb2 = (const uint16_t*)cb2;
  a.scale = (const uint16_t*)scale;
  a.w = w;
  a.w_dtype = w_dtype;
  const size_t total = (size_t)a.n * (size_t)a.nv;
  const size_t blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
