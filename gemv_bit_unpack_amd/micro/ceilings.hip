// Hardware ceilings that bound the VQ kernels on one GPU, measured with plain kernels:
//   - streaming read bandwidth from HBM (4 GiB buffer, 16-byte loads);
//   - random 16-byte gathers from a table in global memory (table sizes from L1-resident
//     to larger than one XCD's L2), the operation behind every centroid lookup of a
//     65536-entry codebook;
//   - random 16-byte gathers from LDS tables (the small-codebook path).
// Every index is masked into its table.  Prints one JSON object.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
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

int main() {
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
  printf("}}\n");
  CHECK(hipFree(buf));
  return 0;
}
