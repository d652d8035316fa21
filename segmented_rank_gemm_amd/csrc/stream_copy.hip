// Measurement aids: a plain device-to-device copy, and an in-place update of
// one buffer (read each 16-byte piece, change it, write it back), both with
// 16-byte vector accesses, four per lane per step.  They give the practical
// read+write HBM ceilings that the kernels of this library are measured
// against; the update is the access pattern of the expand's output.

#include "device_common.hpp"
#include "lora_measure.h"

namespace lora {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                                   u32x4* __restrict__ dst,
                                                                   int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads * kCopyUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * kCopyThreads;
      if (j < n16) v[i] = src[j];
    }
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * kCopyThreads;
      if (j < n16) dst[j] = v[i];
    }
  }
}

__global__ __launch_bounds__(kCopyThreads) void stream_update_kernel(u32x4* __restrict__ buf,
                                                                     int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads * kCopyUnroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
       base < n16; base += stride) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * kCopyThreads;
      if (j < n16) v[i] = load16_stream(buf + j);
    }
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      const int64_t j = base + static_cast<int64_t>(i) * kCopyThreads;
      if (j < n16) store16_stream(buf + j, v[i] ^ u32x4{1u, 1u, 1u, 1u});
    }
  }
}

hipError_t launch_stream_update(void* buf, int64_t bytes, int num_cus, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = static_cast<int64_t>(kCopyThreads) * kCopyUnroll;
  int64_t grid = (n16 + per_block - 1) / per_block;
  const int64_t cap = static_cast<int64_t>(num_cus) * 16;
  grid = grid < cap ? grid : cap;
  grid = grid < 1 ? 1 : grid;
  hipLaunchKernelGGL(stream_update_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), 0,
                     stream, static_cast<u32x4*>(buf), n16);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int num_cus,
                              hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = static_cast<int64_t>(kCopyThreads) * kCopyUnroll;
  int64_t grid = (n16 + per_block - 1) / per_block;
  const int64_t cap = static_cast<int64_t>(num_cus) * 16;
  grid = grid < cap ? grid : cap;
  grid = grid < 1 ? 1 : grid;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kCopyThreads), 0,
                     stream, static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace lora

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
lora_status_t launch_status(hipError_t e) { return e == hipSuccess ? LORA_OK : LORA_ERR_LAUNCH; }
}  // namespace

extern "C" {

lora_status_t lora_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return LORA_ERR_INVALID_ARGUMENT;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + static_cast<uintptr_t>(bytes) && d < s + static_cast<uintptr_t>(bytes))
    return LORA_ERR_INVALID_ARGUMENT;
  return launch_status(lora::launch_stream_copy(src, dst, bytes, lora::kCus, stream));
}

lora_status_t lora_stream_update(void* buf, int64_t bytes, hipStream_t stream) {
  if (!buf || bytes <= 0 || bytes % 16 != 0 || !aligned16(buf)) return LORA_ERR_INVALID_ARGUMENT;
  return launch_status(lora::launch_stream_update(buf, bytes, lora::kCus, stream));
}

}  // extern "C"
