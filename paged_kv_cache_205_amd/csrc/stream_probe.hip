// A plain streaming read, timed by the benchmark as the bandwidth this GPU
// actually delivers to a read-only scan (the reference beside the decode
// kernel's KV bandwidth).  Not part of the paged-attention library: it is
// built into its own libpa_probe.so.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16, unsigned* sink) {
  size_t i = (size_t)blockIdx.x * 256 * kUnroll + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256 * kUnroll;
  unsigned acc = 0;
  for (; i + 256 * (kUnroll - 1) < n16; i += stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // keeps the loads; practically never stored
}

}  // namespace

// Reads bytes (a multiple of 16 * 256 * 8) from p once; sink is a device word.
extern "C" int pa_probe_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t stream) {
  if (!p || !sink || bytes % (16 * 256 * kUnroll) != 0) return -1;
  int cus = 256, dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    cus = n;
  hipLaunchKernelGGL(stream_read_kernel, dim3(cus * 32), dim3(256), 0, stream, static_cast<const u32x4*>(p),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
