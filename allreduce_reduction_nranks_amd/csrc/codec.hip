// codec.hip -- standalone FP8 E4M3B15 <-> f16 / f32 conversion kernels.
//
// Format: MSCCL++ commit history for /src, entry adding the fp8_e4m3b15
// datatype (4 exponent bits, 3 mantissa bits, bias 15, largest finite value
// 0.9375, converted through fp16 as intermediate); ROCm support entry.
// Decoding is exact; encoding is one round-to-nearest-even, saturating.
//
// Elementwise and HBM-bound.  A lane handles a unit of 16 elements: 16 bytes
// of FP8, 32 bytes of f16 or 64 bytes of f32, all moved with non-temporal
// 16-byte accesses; the last n % 16 elements go element by element.
#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

enum : int { kDecF16 = 0, kDecF32 = 1, kEncF16 = 2, kEncF32 = 3 };

template <int Dir> __device__ __forceinline__ void codec_unit(const void* in, void* out, uint64_t u) {
  if constexpr (Dir == kDecF16 || Dir == kDecF32) {
    const u32x4 c = ld_stream(in, u);
    if constexpr (Dir == kDecF16) {
      u32x4 o[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = c[j];
        const uint32_t lo = fp8_to_f16(w & 0xFFu) | (fp8_to_f16((w >> 8) & 0xFFu) << 16);
        const uint32_t hi = fp8_to_f16((w >> 16) & 0xFFu) | (fp8_to_f16(w >> 24) << 16);
        o[j / 2][(j % 2) * 2] = lo;
        o[j / 2][(j % 2) * 2 + 1] = hi;
      }
      st_stream(out, 2 * u, o[0]);
      st_stream(out, 2 * u + 1, o[1]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) o[b] = __float_as_uint(fp8_to_f32((c[j] >> (8 * b)) & 0xFFu));
        st_stream(out, 4 * u + j, o);
      }
    }
  } else {
    u32x4 o;
    if constexpr (Dir == kEncF16) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 h = ld_stream(in, 2 * u + q);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t w0 = h[2 * j], w1 = h[2 * j + 1];
          o[2 * q + j] = f16_to_fp8(w0 & 0xFFFFu) | (f16_to_fp8(w0 >> 16) << 8) |
                         (f16_to_fp8(w1 & 0xFFFFu) << 16) | (f16_to_fp8(w1 >> 16) << 24);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 f = ld_stream(in, 4 * u + q);
        o[q] = f32_to_fp8(__uint_as_float(f[0])) | (f32_to_fp8(__uint_as_float(f[1])) << 8) |
               (f32_to_fp8(__uint_as_float(f[2])) << 16) | (f32_to_fp8(__uint_as_float(f[3])) << 24);
      }
    }
    st_stream(out, u, o);
  }
}

template <int Dir> __device__ __forceinline__ void codec_elem(const void* in, void* out, uint64_t i) {
  if constexpr (Dir == kDecF16)
    reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)fp8_to_f16(reinterpret_cast<const uint8_t*>(in)[i]);
  else if constexpr (Dir == kDecF32)
    reinterpret_cast<float*>(out)[i] = fp8_to_f32(reinterpret_cast<const uint8_t*>(in)[i]);
  else if constexpr (Dir == kEncF16)
    reinterpret_cast<uint8_t*>(out)[i] = (uint8_t)f16_to_fp8(reinterpret_cast<const uint16_t*>(in)[i]);
  else
    reinterpret_cast<uint8_t*>(out)[i] = (uint8_t)f32_to_fp8(reinterpret_cast<const float*>(in)[i]);
}

// Vector path: units [0, n / 16) then the tail, both grid-stride.
template <int Dir>
__global__ void __launch_bounds__(256) codec_vec_k(const void* in, void* out, uint64_t n) {
  const uint64_t units = n / 16;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (uint64_t u = tid; u < units; u += stride) codec_unit<Dir>(in, out, u);
  for (uint64_t i = units * 16 + tid; i < n; i += stride) codec_elem<Dir>(in, out, i);
}

template <int Dir>
__global__ void __launch_bounds__(256) codec_scalar_k(const void* in, void* out, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    codec_elem<Dir>(in, out, i);
}

hipError_t launch_codec(int dir, const void* in, void* out, size_t n, bool vector,
                        hipStream_t stream) {
  const uint64_t work = vector ? (n / 16 > 0 ? n / 16 : 1) : n;
  uint64_t blocks = (work + 255) / 256;
  const uint64_t cap = (uint64_t)device_cu_count(-1) * 16;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) blocks = 1;
  const dim3 grid((uint32_t)blocks), block(256);
  switch (dir) {
#define MRR_DIR(D)                                                                          \
  case D:                                                                                   \
    if (vector) hipLaunchKernelGGL(codec_vec_k<D>, grid, block, 0, stream, in, out, (uint64_t)n); \
    else hipLaunchKernelGGL(codec_scalar_k<D>, grid, block, 0, stream, in, out, (uint64_t)n); \
    break;
    MRR_DIR(kDecF16) MRR_DIR(kDecF32) MRR_DIR(kEncF16) MRR_DIR(kEncF32)
#undef MRR_DIR
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mrr
