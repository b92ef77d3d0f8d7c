// calib.hip -- plain device copy with the RS/AG launch scheme: the copy-kernel
// calibration measured beside the reductions.
//
// A reduction's HBM traffic is a 1:1 mix of streaming reads and writes; a copy
// of the same bytes is that mix with no arithmetic, so its bandwidth on the
// same launch scheme (one single-wave workgroup per tile, residency capped
// through an unused LDS reservation, non-temporal 16-byte accesses) is the
// practical ceiling the reductions are read against.
#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

// Units (16-byte vectors) per lane and workgroups per CU, from a sweep on
// MI355X copying 512 MiB (U in {1,2,4} x 2-16 workgroups per CU): U=4 at 12
// per CU moved 0.83 of the 8 TB/s HBM peak; the best persistent grid (cap
// 8-32, U 1-4) reached 0.77.
constexpr int kCopyU = 4;
constexpr int kCopyThreads = 64;
constexpr int kCopyWpc = 12;
constexpr uint64_t kCopyMaxGrid = 1u << 24;

__global__ void __launch_bounds__(kCopyThreads)
stream_copy_k(const void* src, void* dst, uint64_t nvec, uint64_t tiles, uint64_t nbytes) {
  for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint64_t v0 = t * (kCopyThreads * kCopyU) + threadIdx.x;
    u32x4 r[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint64_t v = v0 + (uint64_t)u * kCopyThreads;
      if (v < nvec) r[u] = ld_stream(src, v);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint64_t v = v0 + (uint64_t)u * kCopyThreads;
      if (v < nvec) st_stream(dst, v, r[u]);
    }
  }
  // The last nbytes % 16 bytes, one per lane, by the last workgroup.
  if (blockIdx.x == gridDim.x - 1) {
    const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
    uint8_t* d = reinterpret_cast<uint8_t*>(dst);
    for (uint64_t i = nvec * 16 + threadIdx.x; i < nbytes; i += kCopyThreads) d[i] = s[i];
  }
}

// src and dst 16-byte aligned, not overlapping (checked by the caller).
hipError_t launch_stream_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream) {
  const uint64_t nvec = nbytes / 16;
  const uint64_t tiles = (nvec + kCopyThreads * kCopyU - 1) / (kCopyThreads * kCopyU);
  const bool capped = lds_cap_enabled();
  uint64_t max_grid = kCopyMaxGrid;
  const uint32_t g_env = max_grid_override();
  if (g_env > 0 && g_env < max_grid) max_grid = g_env;
  if (!capped) {  // persistent grid, no LDS reservation
    const uint64_t p = (uint64_t)device_cu_count(-1) * kCopyWpc;
    if (p > 0 && p < max_grid) max_grid = p;
  }
  uint64_t blocks = tiles < max_grid ? tiles : max_grid;
  if (blocks == 0) blocks = 1;  // a tail-only copy
  const size_t lds = capped ? occupancy_lds_bytes(kCopyWpc) : 0;
  hipLaunchKernelGGL(stream_copy_k, dim3((uint32_t)blocks), dim3(kCopyThreads), lds, stream, src, dst,
                     nvec, tiles, (uint64_t)nbytes);
  return hipGetLastError();
}

}  // namespace mrr
