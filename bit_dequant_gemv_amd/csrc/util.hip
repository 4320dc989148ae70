// Status strings and the two measurement kernels (streaming read, copy)
// used to put the decode path next to the achievable HBM rate.
#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Each thread reads 16-byte vectors at a grid stride and folds them into a
// checksum so the loads cannot be elided; one float per block is written.
__global__ void __launch_bounds__(256)
stream_read_kernel(const u32x4* __restrict__ buf, int64_t n_vec, float* __restrict__ sink) {
  __shared__ float red[4];
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n_vec; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  float v = (float)(acc & 0xFFFFu);
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

__global__ void __launch_bounds__(256)
stream_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n_vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec; i += stride) dst[i] = src[i];
}

}  // namespace bdg

using namespace bdg;

extern "C" int bdg_stream_read(const void* buf, int64_t bytes, float* sink, int32_t n_blocks, void* stream) {
  if (!buf || !sink || bytes < 0 || (bytes % 16) != 0) return BDG_E_INVALID;
  if (!aligned16(buf)) return BDG_E_ALIGN;
  if (n_blocks <= 0) n_blocks = 256 * 8;
  hipLaunchKernelGGL(stream_read_kernel, dim3(n_blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return launch_status();
}

extern "C" int bdg_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes < 0 || (bytes % 16) != 0) return BDG_E_INVALID;
  if (!aligned16(src) || !aligned16(dst)) return BDG_E_ALIGN;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(256 * 8), dim3(256), 0, as_stream(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return launch_status();
}

extern "C" const char* bdg_strerror(int32_t status) {
  switch (status) {
    case BDG_OK: return "ok";
    case BDG_E_INVALID: return "invalid argument (shape, dtype, flag, count or NULL pointer)";
    case BDG_E_ALIGN: return "a code buffer or stride is not 16-byte aligned";
    case BDG_E_UNSUPPORTED: return "outside the shapes the kernels cover";
    case BDG_E_HIP: return "HIP runtime or kernel launch error";
    case BDG_E_NOMEM: return "device allocation failed";
    case BDG_E_TOO_LARGE: return "request needs more than the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

extern "C" const char* bdg_version(void) { return "libbdg 0.1.0 gfx950"; }
