// Hardware ceilings that bound the VQ kernels on one GPU, measured with plain kernels:
//   - streaming read bandwidth from HBM (4 GiB buffer, 16-byte loads);
//   - random 16-byte gathers from a table in global memory (table sizes from L1-resident
//     to larger than one XCD's L2), the operation behind every centroid lookup of a
//     65536-entry codebook;
//   - random 16-byte gathers from LDS tables (the small-codebook path);
//   - the LDS read rate with little VALU work per read (addresses held in registers,
//     constant offsets), for four address patterns of a 64-lane 16-byte read: random,
//     7 of 8 lanes on one address, 1 of 8 lanes active, and conflict-free;
//   - the issue rate of the matrix instructions the products use (16x16x32, 32x32x16,
//     4x4x4 with 16 blocks, fp16) and of the packed fp16 dot (v_dot2_f32_f16), and whether
//     VALU and matrix instructions overlap on one SIMD;
//   - the rate at which 8 workgroups on one XCD can all read the same stream (each
//     byte fetched once from HBM, then served 7 more times by the XCD's L2), against
//     each workgroup reading its own stream.
// Every index is masked into its table.  Prints one JSON object; with --stream, only the
// streaming read.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#define CHECK(x)                                                                                   \
  do {                                                                                             \
    hipError_t e_ = (x);                                                                           \
    if (e_ != hipSuccess) {                                                                        \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__);      \
      exit(1);                                                                                     \
    }                                                                                              \
  } while (0)

__global__ void stream_read(const uint4* __restrict__ p, size_t n16, unsigned* out) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n16; i += stride) acc ^= p[i].x;
  if (acc == 0x12345678u) out[0] = acc;
}

__global__ void gather_global(const uint4* __restrict__ tab, unsigned mask, int iters, unsigned* out) {
  unsigned s = (blockIdx.x * blockDim.x + threadIdx.x) * 2654435761u + 12345u;
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s = s * 1664525u + 1013904223u;
      v[k] = tab[(s >> 7) & mask];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;  // all four words: full 16-byte loads
  }
  if (acc == 0x12345678u) out[0] = acc;
}

extern __shared__ uint4 lds_tab[];
__global__ void gather_lds(const uint4* __restrict__ tab, unsigned entries, int iters, unsigned* out) {
  for (unsigned e = threadIdx.x; e < entries; e += blockDim.x) lds_tab[e] = tab[e];
  __syncthreads();
  const unsigned mask = entries - 1;
  unsigned s = (blockIdx.x * blockDim.x + threadIdx.x) * 2654435761u + 12345u;
  unsigned acc = 0;
  for (int it = 0; it < iters; ++it) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      s = s * 1664525u + 1013904223u;
      v[k] = lds_tab[(s >> 7) & mask];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;  // all four words: full 16-byte loads
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// LDS read rate.  Each lane holds 8 table offsets in registers; the loop reads 4
// consecutive entries from each (constant instruction offsets: no address VALU) and
// folds the 16 bytes with two 3-input adds, so the SIMDs issue 2 VALU per read.
//   MODE 0: random entries of a 128 KiB table;
//   MODE 1: lanes 1..7 of every 8 read entry kLdsEntries - 4, lane 0 a random one;
//   MODE 2: only lanes 0, 8, ..., 56 run the loop (7 of 8 lanes masked off);
//   MODE 3: lane l reads entry l + 64 k (each group of 16 lanes covers all 64 banks);
//   MODE 4: lane l reads a random row of the table at column l mod 16 (column = entry
//           mod 16), so lanes 4q .. 4q + 3 of each 16-lane group stay in columns
//           4q .. 4q + 3;
//   MODE 5: random rows at column 5 l mod 16: still 16 distinct columns per group of 16
//           lanes, but a lane's column lies outside its group of four.
// Modes 4 and 5 step the 4 reads of an offset by 16 entries (same column).
constexpr unsigned kLdsEntries = 8192;
template <int MODE>
__global__ __launch_bounds__(512) void lds_rate(const uint4* __restrict__ tab, int iters, unsigned* out) {
  __shared__ uint4 t[kLdsEntries];
  for (unsigned e = threadIdx.x; e < kLdsEntries; e += blockDim.x) t[e] = tab[e];
  __syncthreads();
  const unsigned lane = threadIdx.x & 63;
  unsigned h = (blockIdx.x * blockDim.x + threadIdx.x) * 2654435761u + 12345u;
  unsigned a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    h = h * 1664525u + 1013904223u;
    unsigned e = (h >> 9) % (kLdsEntries - 4);  // entries e .. e + 3 stay in the table
    if (MODE == 1 && (lane & 7)) e = kLdsEntries - 4;
    if (MODE == 3) e = lane + 64 * k;
    if (MODE == 4) e = ((h >> 9) % (kLdsEntries / 16 - 4)) * 16 + (lane & 15);
    if (MODE == 5) e = ((h >> 9) % (kLdsEntries / 16 - 4)) * 16 + ((lane * 5) & 15);
    a[k] = e;
  }
  constexpr unsigned kStep = MODE >= 4 ? 16 : 1;
  unsigned acc0 = 0, acc1 = 0;
  if (MODE != 2 || (lane & 7) == 0) {
    for (int it = 0; it < iters; ++it) {
      asm volatile("" ::: "memory");  // the table may have changed: read it again every pass
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint4 v = t[a[k] + j * kStep];
          acc0 = acc0 + v.x + v.y;  // v_add3_u32
          acc1 = acc1 + v.z + v.w;
        }
      }
    }
  }
  if ((acc0 ^ acc1) == 0x12345678u) out[0] = acc0;
}

typedef _Float16 mr_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 mr_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 mr_half2 __attribute__((ext_vector_type(2)));
typedef float mr_float4 __attribute__((ext_vector_type(4)));
typedef float mr_float16 __attribute__((ext_vector_type(16)));

// Matrix-instruction issue rate: 4 independent accumulator chains per wavefront.
//   KIND 0: v_mfma_f32_16x16x32_f16; KIND 1: v_mfma_f32_32x32x16_f16;
//   KIND 2: v_mfma_f32_4x4x4_16b_f16 (16 blocks).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate(int iters, float* out) {
  const float s = (float)(threadIdx.x & 7) * 0.001f;
  float sum = 0.0f;
  if constexpr (KIND == 0) {
    const mr_half8 a = {(_Float16)s, 1, 2, 3, 4, 5, 6, 7}, b = {1, 1, 1, 1, 1, 1, 1, (_Float16)s};
    mr_float4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c3, 0, 0, 0);
    }
    sum = c0[0] + c1[1] + c2[2] + c3[3];
  } else if constexpr (KIND == 1) {
    const mr_half8 a = {(_Float16)s, 1, 2, 3, 4, 5, 6, 7}, b = {1, 1, 1, 1, 1, 1, 1, (_Float16)s};
    mr_float16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    sum = c0[0] + c1[5] + c2[10] + c3[15];
  } else {
    const mr_half4 a = {(_Float16)s, 1, 2, 3}, b = {1, 1, 1, (_Float16)s};
    mr_float4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c3, 0, 0, 0);
    }
    sum = c0[0] + c1[1] + c2[2] + c3[3];
  }
  if (sum == 1234.5f) out[0] = sum;
}

// Packed fp16 dot (v_dot2_f32_f16) issue rate: 8 independent chains per lane.
__global__ __launch_bounds__(256) void dot2_rate(int iters, float* out) {
  const mr_half2 a = {(_Float16)((threadIdx.x & 7) * 0.001f), (_Float16)1}, b = {(_Float16)1, (_Float16)0.5f};
  float c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = (float)k;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_fdot2(a, b, c[k], false);
  }
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += c[k];
  if (sum == 1234.5f) out[0] = sum;
}

// Whether VALU and matrix instructions overlap on one SIMD: per iteration a wavefront
// issues 4 independent v_mfma_f32_16x16x32_f16 (MODE 0), 16 independent v_dot2_f32_f16
// (MODE 1), or both (MODE 2); 4 wavefronts per SIMD.  With full overlap MODE 2 would take
// the longer of MODE 0 and MODE 1, without any the sum.
template <int MODE>
__global__ __launch_bounds__(256) void issue_overlap(int iters, float* out) {
  const float s = (float)(threadIdx.x & 7) * 0.001f;
  const mr_half8 a = {(_Float16)s, 1, 2, 3, 4, 5, 6, 7}, b = {1, 1, 1, 1, 1, 1, 1, (_Float16)s};
  const mr_half2 p = {(_Float16)s, (_Float16)1}, q = {(_Float16)1, (_Float16)0.5f};
  mr_float4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
  float d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) d[j] = (float)j;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE != 1) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c3, 0, 0, 0);
    }
    if constexpr (MODE != 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = __builtin_amdgcn_fdot2(p, q, d[j], false);
      }
    }
  }
  float sum = c0[0] + c1[1] + c2[2] + c3[3];
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += d[j];
  if (sum == 1234.5f) out[0] = sum;
}

// Shared-stream read: 256 workgroups of 512 threads as 32 groups of 8 (the 8 workgroups of
// a group have consecutive ids above the XCD bits, so they land on one XCD).  SHARED: the 8
// read the same `per` bytes of their group's region; otherwise each reads its own.
template <bool SHARED>
__global__ __launch_bounds__(512) void group_stream(const uint4* __restrict__ p, size_t per16, unsigned* out) {
  const int xcd = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int s = rest & 7;
  const int grp = (rest >> 3) * 8 + xcd;
  const uint4* q = p + (SHARED ? (size_t)grp : (size_t)grp * 8 + s) * per16;
  unsigned acc = 0;
  size_t i = threadIdx.x;
  for (; i + 7 * 512 < per16; i += 8 * 512) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = q[i + k * 512];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].w;
  }
  for (; i < per16; i += 512) acc ^= q[i].x;
  if (acc == 0x12345678u) out[0] = acc;
}

int main(int argc, char** argv) {
  const bool stream_only = argc > 1 && std::string(argv[1]) == "--stream";
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int ncu = prop.multiProcessorCount;
  const double clk = prop.clockRate * 1e3;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  unsigned* dout;
  CHECK(hipMalloc(&dout, 64));
  const size_t bytes = (size_t)4 << 30;
  uint4* buf;
  CHECK(hipMalloc(&buf, bytes));
  CHECK(hipMemset(buf, 1, bytes));
  auto timed = [&](auto launch, int reps) {
    launch();
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    return ms * 1e-3 / reps;
  };
  printf("{\"device\": \"%s\", \"cus\": %d, \"clock_ghz\": %.3f", prop.gcnArchName, ncu, clk / 1e9);
  double best = 0;
  for (int per_cu : {4, 8, 16}) {
    const int grid = ncu * per_cu;
    const double t = timed([&] { hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, 0, buf, bytes / 16, dout); }, 5);
    best = std::max(best, bytes / t / 1e9);
  }
  printf(", \"stream_read_GBps\": %.1f", best);
  if (stream_only) {  // just the HBM read rate
    printf("}\n");
    CHECK(hipFree(buf));
    return 0;
  }
  printf(", \"gather_global\": {");
  bool first = true;
  for (unsigned entries : {2048u, 8192u, 65536u, 262144u}) {
    double g = 0;
    for (int per_cu : {8, 16}) {
      const int grid = ncu * per_cu, iters = 64;
      const double t = timed([&] { hipLaunchKernelGGL(gather_global, dim3(grid), dim3(256), 0, 0, buf, entries - 1, iters, dout); }, 3);
      g = std::max(g, (double)grid * 256 * iters * 8 / t);
    }
    printf("%s\"table_%uKiB\": {\"gathers_per_s\": %.4g, \"per_clk_per_cu\": %.3f}", first ? "" : ", ", entries * 16 / 1024,
           g, g / (ncu * clk));
    first = false;
  }
  printf("}, \"gather_lds\": {");
  first = true;
  for (unsigned entries : {256u, 4096u, 8192u}) {
    const size_t lds = entries * 16;
    CHECK(hipFuncSetAttribute((const void*)gather_lds, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    double g = 0;
    for (int bs : {256, 1024}) {
      const int grid = ncu * 4, iters = 256;
      const double t = timed([&] { hipLaunchKernelGGL(gather_lds, dim3(grid), dim3(bs), lds, 0, buf, entries, iters, dout); }, 3);
      g = std::max(g, (double)grid * bs * iters * 8 / t);
    }
    printf("%s\"table_%uKiB\": {\"gathers_per_s\": %.4g, \"per_clk_per_cu\": %.3f}", first ? "" : ", ", entries * 16 / 1024,
           g, g / (ncu * clk));
    first = false;
  }
  printf("}");

  // LDS read rate at 512 threads (one workgroup per CU: the 128 KiB table), 6 patterns.
  printf(", \"lds_read_b128\": {");
  const char* lds_modes[6] = {"random", "seven_of_eight_one_address", "one_of_eight_active", "conflict_free",
                              "random_rows_column_in_lane_quad", "random_rows_distinct_columns_across_quads"};
  for (int mode = 0; mode < 6; ++mode) {
    const int grid = ncu, iters = 512;
    auto launch = [&] {
      switch (mode) {
        case 0: hipLaunchKernelGGL(lds_rate<0>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
        case 1: hipLaunchKernelGGL(lds_rate<1>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
        case 2: hipLaunchKernelGGL(lds_rate<2>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
        case 3: hipLaunchKernelGGL(lds_rate<3>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
        case 4: hipLaunchKernelGGL(lds_rate<4>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
        default: hipLaunchKernelGGL(lds_rate<5>, dim3(grid), dim3(512), 0, 0, buf, iters, dout); break;
      }
    };
    const double t = timed(launch, 3);
    const double instr = (double)grid * (512 / 64) * iters * 32;  // 64-lane read instructions
    printf("%s\"%s\": {\"clk_per_instr_per_cu\": %.3f, \"active_lanes_per_clk_per_cu\": %.3f}", mode ? ", " : "",
           lds_modes[mode], t * clk * ncu / instr, instr * (mode == 2 ? 8 : 64) / (t * clk * ncu));
  }
  printf("}");

  // Matrix and dot instruction issue rates at 4 wavefronts per SIMD.
  printf(", \"issue\": {");
  const char* mnames[3] = {"mfma_f32_16x16x32_f16", "mfma_f32_32x32x16_f16", "mfma_f32_4x4x4_16b_f16"};
  float* fout = (float*)dout;
  for (int kind = 0; kind < 3; ++kind) {
    const int grid = ncu * 4, iters = 4096;
    auto launch = [&] {
      if (kind == 0) hipLaunchKernelGGL(mfma_rate<0>, dim3(grid), dim3(256), 0, 0, iters, fout);
      else if (kind == 1) hipLaunchKernelGGL(mfma_rate<1>, dim3(grid), dim3(256), 0, 0, iters, fout);
      else hipLaunchKernelGGL(mfma_rate<2>, dim3(grid), dim3(256), 0, 0, iters, fout);
    };
    const double t = timed(launch, 3);
    const double instr = (double)grid * 4 * iters * 4;  // per wavefront: 4 chains x iters
    printf("%s\"%s\": {\"clk_per_instr_per_simd\": %.2f}", kind ? ", " : "", mnames[kind],
           t * clk * ncu * 4 / instr);
  }
  {
    const int grid = ncu * 4, iters = 4096;
    const double t = timed([&] { hipLaunchKernelGGL(dot2_rate, dim3(grid), dim3(256), 0, 0, iters, fout); }, 3);
    const double instr = (double)grid * 4 * iters * 8;
    printf(", \"v_dot2_f32_f16\": {\"clk_per_instr_per_simd\": %.2f}", t * clk * ncu * 4 / instr);
  }
  printf("}");

  // VALU / matrix-core overlap on one SIMD.
  printf(", \"valu_mfma_overlap\": {");
  {
    const char* onames[3] = {"mfma_only", "dot2_only", "both_in_one_wave"};
    for (int mode = 0; mode < 3; ++mode) {
      const int grid = ncu * 4, iters = 2048;
      auto launch = [&] {
        if (mode == 0) hipLaunchKernelGGL(issue_overlap<0>, dim3(grid), dim3(256), 0, 0, iters, fout);
        else if (mode == 1) hipLaunchKernelGGL(issue_overlap<1>, dim3(grid), dim3(256), 0, 0, iters, fout);
        else hipLaunchKernelGGL(issue_overlap<2>, dim3(grid), dim3(256), 0, 0, iters, fout);
      };
      const double t = timed(launch, 3);
      printf("%s\"%s\": {\"simd_clk_per_iteration_4_waves\": %.1f}", mode ? ", " : "", onames[mode],
             t * clk / iters);
    }
  }
  printf("}");

  // Eight workgroups of one XCD reading one stream vs their own streams.
  {
    const size_t per = (size_t)8 << 20;  // bytes per stream
    const int grid = 256;
    const double ts = timed([&] { hipLaunchKernelGGL(group_stream<true>, dim3(grid), dim3(512), 0, 0, buf, per / 16, dout); }, 3);
    const double td = timed([&] { hipLaunchKernelGGL(group_stream<false>, dim3(grid), dim3(512), 0, 0, buf, per / 16, dout); }, 3);
    const double delivered = (double)grid * per;
    printf(", \"group_stream\": {\"bytes_per_workgroup\": %zu, \"shared_by_8_delivered_GBps\": %.1f, "
           "\"shared_B_per_clk_per_cu\": %.2f, \"own_stream_GBps\": %.1f}",
           per, delivered / ts / 1e9, delivered / ts / clk / grid, delivered / td / 1e9);
  }
  printf("}\n");
  CHECK(hipFree(buf));
  return 0;
}
