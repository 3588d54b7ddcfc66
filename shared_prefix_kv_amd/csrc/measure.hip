// Streaming-read probe (gfx950): the HBM read rate a plain kernel reaches on
// this device, measured next to the 8 TB/s published peak that the decode
// kernels' roofline fractions are quoted against.
//
// Each thread reads 16-byte pieces in a grid-stride loop, four loads in
// flight per iteration, and folds them into a running XOR; the XOR is stored
// only if it equals a value no input produces in practice, so the loads
// cannot be dropped and nothing is written.

#include "fca_internal.h"

namespace fca {

// Externally visible, so that the store that keeps the loads alive is not
// dropped as dead code.
__device__ uint32_t g_read_sink;

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 512;

__global__ __launch_bounds__(kReadThreads) void fca_stream_read_kernel(const u32x4* __restrict__ src, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) g_read_sink = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, int n_cu, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int grid = std::max(1, n_cu * 4);
  hipLaunchKernelGGL(fca_stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

}  // namespace fca
