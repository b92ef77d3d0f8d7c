// noalloc.hip -- the library-owned packet workspace behind
// mrr_allreduce_packet_noalloc, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// The workspace is one statically sized device array: a flag area of
// kMaxRanks x kFlagSlots uint32 (every rank count's flag slots, so calls of
// different rank counts continue one flag sequence), then kNoAllocPacketBytes
// of packet scratch.  Each GPU holds its own copy of the array, at its own
// address, from the time the library's code is loaded on it until the process
// ends.  In host code `scratch` names a host-side stand-in, not the device
// memory: the device address is fetched once per device with
// hipGetSymbolAddress and only that address is ever handed to a kernel.
#include <mutex>

#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

static_assert(kNoAllocFlagBytes % 256 == 0, "the packet area must start 256-byte aligned");

static __device__ __align__(256) uint8_t scratch[kNoAllocFlagBytes + kNoAllocPacketBytes];

// Zero fill of n16 16-byte vectors.
__global__ void __launch_bounds__(256) noalloc_clear_k(u32x4* p, uint64_t n16) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = z;
}

// Device address of the current device's workspace.  The first call on a
// device looks the address up and clears the whole array on `stream` (the
// packet protocol needs every flag slot equal and no packet carrying a flag
// the sequence has not reached yet), stream-ordered before the caller's
// kernel.  That first call must not run under stream capture, or the clear
// would only run when the graph does: it then returns
// hipErrorStreamCaptureUnsupported and sets nothing up.
hipError_t noalloc_workspace(hipStream_t stream, uint8_t** base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::mutex mu;
  static uint8_t* ptr[64] = {nullptr};
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (uintptr_t)p % 256 != 0) return hipErrorInvalidSymbol;
    const uint64_t n16 = (kNoAllocFlagBytes + kNoAllocPacketBytes) / 16;
    hipLaunchKernelGGL(noalloc_clear_k, dim3(1024), dim3(256), 0, stream, (u32x4*)p, n16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ptr[dev] = (uint8_t*)p;
  }
  *base = ptr[dev];
  return hipSuccess;
}

}  // namespace mrr
