// Measurement utilities beside the layer kernel: HBM read-stream ceiling,
// cache-evicting fill, empty launch.  Declarations: include/moe_bench.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_bench.h"
#include "../../include/moe_decode.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Each thread streams 16-byte units with four loads in flight per
// iteration; workgroups take 64 KiB blocks (256 threads x 16 B x 16) in a
// grid-stride loop.
__global__ __launch_bounds__(256) void k_read_stream(const uint8_t* buf, size_t blocks, unsigned* sink) {
  unsigned acc = 0u;
  for (size_t b = blockIdx.x; b < blocks; b += gridDim.x) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(buf + b * 65536) + threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const u32x4_t v0 = __builtin_nontemporal_load(p + (i + 0) * 256);
      const u32x4_t v1 = __builtin_nontemporal_load(p + (i + 1) * 256);
      const u32x4_t v2 = __builtin_nontemporal_load(p + (i + 2) * 256);
      const u32x4_t v3 = __builtin_nontemporal_load(p + (i + 3) * 256);
      acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
      acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void k_fill(u32x4_t* buf, size_t n, unsigned v) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) buf[i] = u32x4_t{v, v, v, v};
}

__global__ __launch_bounds__(256) void k_empty() {}

int cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

}  // namespace

extern "C" {

int moe_bench_read_stream(const void* buf, size_t bytes, unsigned* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 65536 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return MOE_ERR_INVALID_ARG;
  const int n = cus();
  if (n <= 0) return MOE_ERR_LAUNCH;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_read_stream, dim3(4 * n), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(buf), bytes / 65536, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_bench_fill(void* buf, size_t bytes, unsigned value, void* stream) {
  if (buf == nullptr || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return MOE_ERR_INVALID_ARG;
  const int n = cus();
  if (n <= 0) return MOE_ERR_LAUNCH;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_fill, dim3(8 * n), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<u32x4_t*>(buf), bytes / 16, value);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

int moe_bench_empty(int workgroups, void* stream) {
  if (workgroups <= 0) return MOE_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_empty, dim3(workgroups), dim3(256), 0, reinterpret_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // extern "C"
