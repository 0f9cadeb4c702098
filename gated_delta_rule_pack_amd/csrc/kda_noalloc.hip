// Fixed workspace of the allocation-free forward call (kda_chunk_fwd_noalloc).
//
// Some callers cannot allocate memory around a call: code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc. For them the library carries one
// fixed-size device array, `scratch`, in its own code object: every GPU the library runs
// on holds a copy of it, at its own address, until the process ends. It stands in for
// the caller's workspace (the chunk records prep writes and the scan reads, and the
// segment maps and start states of a segmented call); every byte of it that a call reads
// is written earlier in that call, so nothing needs clearing between calls. All calls on
// one GPU share it: calls that overlap in time on one GPU race on it.
//
// In host code the array's name is only a host-side stand-in for the symbol, never a
// device address: each context resolves the device copy's address once per device, with
// that device current, and the launches receive that address.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "kda_internal.h"

static __device__ __align__(256) char scratch[kda::kScratchBytes];

namespace kda {

int scratch_address(int device, void** ptr) {
  static std::mutex mu;
  static std::vector<void*> by_device;  // resolved address per device ordinal (null: not yet)
  std::lock_guard<std::mutex> lock(mu);
  if (device < 0) return (int)hipErrorInvalidDevice;
  if ((size_t)device < by_device.size() && by_device[device]) {
    *ptr = by_device[device];
    return 0;
  }
  int current = 0;
  hipError_t e = hipGetDevice(&current);
  if (e != hipSuccess) return (int)e;
  if (current != device && (e = hipSetDevice(device)) != hipSuccess) return (int)e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (current != device) {
    const hipError_t r = hipSetDevice(current);
    if (e == hipSuccess) e = r;
  }
  if (e != hipSuccess) return (int)e;
  if (!p) return (int)hipErrorInvalidSymbol;
  if (by_device.size() <= (size_t)device) by_device.resize(device + 1, nullptr);
  by_device[device] = p;
  *ptr = p;
  return 0;
}

}  // namespace kda
