// Metadata upload on the call's stream as a kernel.
//
// The metadata a call builds on a cache miss (aiter PR 6912, Changes: one non-blocking
// upload from pinned memory) sits in the context's pinned staging arena, which the device
// can read directly. A copy engine transfer would put a hand-off between the copy queue and
// the compute queue in front of the call's first kernel; this kernel copies the buffer on
// the compute queue itself, reading host memory over the bus.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {
namespace {

// Buffer-load cache policy: system scope (sc0 | sc1), so the loads bypass the GPU caches.
// A staging range is reused once its upload has completed, with new contents the host
// wrote; a cached line of the previous contents must never be read.
constexpr int kSystemScope = 1 | 16;

// src and dst are 16-byte aligned; n16 (16-byte words) fits a 32-bit byte range.
__global__ __launch_bounds__(256) void meta_copy_kernel(const void* src, int4* __restrict__ dst, int n16) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), (short)0, n16 * 16, 0x00020000);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
    dst[i] = __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, kSystemScope));
}

}  // namespace

int launch_meta_copy(const void* host_src, void* dst, size_t bytes, void* stream, void* done) {
  if (bytes % 16 != 0 || (uintptr_t)host_src % 16 != 0 || (uintptr_t)dst % 16 != 0 || bytes > (size_t)INT32_MAX)
    return (int)hipErrorInvalidValue;
  const int n16 = (int)(bytes / 16);
  const int want = (n16 + 255) / 256;
  const int grid = want < 1 ? 1 : (want < 64 ? want : 64);
  hipExtLaunchKernelGGL(meta_copy_kernel, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), nullptr,
                        reinterpret_cast<hipEvent_t>(done), 0, host_src, reinterpret_cast<int4*>(dst), n16);
  return (int)hipGetLastError();
}

}  // namespace kda
