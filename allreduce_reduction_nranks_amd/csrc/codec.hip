// codec.hip -- standalone FP8 E4M3B15 <-> f16 / f32 conversion kernels.
//
// Format: MSCCL++ commit history for /src, entry adding the fp8_e4m3b15
// datatype (4 exponent bits, 3 mantissa bits, bias 15, largest finite value
// 0.9375, converted through fp16 as intermediate); ROCm support entry.
// Decoding is exact; encoding is one round-to-nearest-even, saturating.
//
// Elementwise and HBM-bound.  A lane converts units of V elements, where the
// wider side of a unit is one 16-byte vector and the narrower side 4 or 8
// bytes; consecutive lanes take consecutive units, so every load and every
// store instruction of a wave covers one contiguous span (1 KiB on the wide
// side, 256 or 512 B on the narrow side) and writes whole cache lines.  Each
// lane keeps U units in flight; the last n % V elements go one by one.
// One workgroup per tile, dispatched in order, with residency capped by an
// unused LDS reservation (as for the RS/AG kernels): a persistent grid that
// strides over the tiles was measured 7-18 % slower on MI355X.
#include <cstdlib>

#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

enum : int { kDecF16 = 0, kDecF32 = 1, kEncF16 = 2, kEncF32 = 3 };

// V elements per unit; DI input words and DO output words per unit.
template <int Dir> struct CodecShape;
template <> struct CodecShape<kDecF16> { static constexpr int V = 8, DI = 2, DO = 4; };
template <> struct CodecShape<kDecF32> { static constexpr int V = 4, DI = 1, DO = 4; };
template <> struct CodecShape<kEncF16> { static constexpr int V = 8, DI = 4, DO = 2; };
template <> struct CodecShape<kEncF32> { static constexpr int V = 4, DI = 4, DO = 1; };

template <int Dir> __device__ __forceinline__ void convert_unit(const uint32_t* in, uint32_t* out) {
  if constexpr (Dir == kDecF16) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w = in[j];
      out[2 * j] = fp8_to_f16(w & 0xFFu) | (fp8_to_f16((w >> 8) & 0xFFu) << 16);
      out[2 * j + 1] = fp8_to_f16((w >> 16) & 0xFFu) | (fp8_to_f16(w >> 24) << 16);
    }
  } else if constexpr (Dir == kDecF32) {
#pragma unroll
    for (int b = 0; b < 4; ++b) out[b] = __float_as_uint(fp8_to_f32((in[0] >> (8 * b)) & 0xFFu));
  } else if constexpr (Dir == kEncF16) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w0 = in[2 * j], w1 = in[2 * j + 1];
      out[j] = f16_to_fp8(w0 & 0xFFFFu) | (f16_to_fp8(w0 >> 16) << 8) |
               (f16_to_fp8(w1 & 0xFFFFu) << 16) | (f16_to_fp8(w1 >> 16) << 24);
    }
  } else {
    out[0] = f32_to_fp8(__uint_as_float(in[0])) | (f32_to_fp8(__uint_as_float(in[1])) << 8) |
             (f32_to_fp8(__uint_as_float(in[2])) << 16) | (f32_to_fp8(__uint_as_float(in[3])) << 24);
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

constexpr int kCodecThreads = 64;  // one wave per workgroup, as the RS/AG kernels

// Vector path: tiles of kCodecThreads * U units, grid-stride, then the tail.
template <int Dir, int U>
__global__ void __launch_bounds__(kCodecThreads) codec_vec_k(const void* in, void* out, uint64_t n) {
  using S = CodecShape<Dir>;
  const uint64_t units = n / S::V;
  const uint64_t tile = (uint64_t)kCodecThreads * U;
  for (uint64_t t0 = (uint64_t)blockIdx.x * tile; t0 < units; t0 += (uint64_t)gridDim.x * tile) {
    const uint64_t v0 = t0 + threadIdx.x;
    if (t0 + tile <= units) {
      uint32_t w[U][S::DI];
#pragma unroll
      for (int u = 0; u < U; ++u) ld_words<S::DI>(in, v0 + (uint64_t)u * kCodecThreads, w[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t o[S::DO];
        convert_unit<Dir>(w[u], o);
        st_words<S::DO>(out, v0 + (uint64_t)u * kCodecThreads, o);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t v = v0 + (uint64_t)u * kCodecThreads;
        if (v < units) {
          uint32_t w[S::DI], o[S::DO];
          ld_words<S::DI>(in, v, w);
          convert_unit<Dir>(w, o);
          st_words<S::DO>(out, v, o);
        }
      }
    }
  }
  const uint64_t stride = (uint64_t)gridDim.x * kCodecThreads;
  for (uint64_t i = units * S::V + (uint64_t)blockIdx.x * kCodecThreads + threadIdx.x; i < n; i += stride)
    codec_elem<Dir>(in, out, i);
}

template <int Dir>
__global__ void __launch_bounds__(kCodecThreads) codec_scalar_k(const void* in, void* out, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    codec_elem<Dir>(in, out, i);
}

// Units in flight per lane and single-wave workgroups per CU, per direction,
// measured on MI355X over 268,435,456 elements (U in {1,2,4,8} x 4-32
// workgroups per CU, one workgroup per tile, two runs each), fractions of the
// HBM peak: E4M3B15 -> f16 U=4 x16 (0.81), -> f32 U=4 x16 (0.82); f16 ->
// E4M3B15 U=4 x24 (0.81), f32 -> E4M3B15 U=2 x24 (0.85).  A second session
// moved two caps (E4M3B15 -> f16 x24 -> x16: 0.807 -> 0.813; f32 -> E4M3B15
// x32 -> x24: 0.842 -> 0.853, mean of two A/B runs each).  256-lane
// workgroups (U=4 at 4 per CU for the decodes, 6 for the encodes; U=2 for the
// f32 encode) ran 0.77 / 0.82 / 0.80 / 0.79 in the first session.  Stores at
// device scope (written through the L2, as some RS/AG shapes use) were 0.5-1 %
// slower in every direction, so the codec keeps plain streaming stores.
// MRR_CODEC_U / MRR_CODEC_WPC override.
constexpr int codec_unroll(int dir) { return dir == kEncF32 ? 2 : 4; }
constexpr int codec_wg_per_cu(int dir) {
  return dir == kDecF32 || dir == kDecF16 ? 16 : 24;
}
// At most 2^22 workgroups of 64 lanes (2^28 work-items); past that a workgroup
// walks several tiles.
constexpr uint64_t kCodecMaxGrid = 1u << 22;
template <int Dir, int U>
static void launch_vec_u(dim3 grid, size_t lds, const void* in, void* out, uint64_t n,
                         hipStream_t s) {
  hipLaunchKernelGGL((codec_vec_k<Dir, U>), grid, dim3(kCodecThreads), lds, s, in, out, n);
}

template <int Dir>
static hipError_t launch_codec_dir(const void* in, void* out, uint64_t n, bool vector,
                                   hipStream_t stream) {
  const int u_env = codec_u_override();
  const int wpc_env = codec_wpc_override();
  const int U = (u_env == 1 || u_env == 2 || u_env == 4 || u_env == 8) ? u_env : codec_unroll(Dir);
  const uint64_t wpc = wpc_env > 0 ? (uint64_t)wpc_env : (uint64_t)codec_wg_per_cu(Dir);
  const uint64_t units = n / CodecShape<Dir>::V;
  const uint64_t work = vector ? (units + (uint64_t)kCodecThreads * U - 1) / ((uint64_t)kCodecThreads * U)
                               : (n + kCodecThreads - 1) / kCodecThreads;
  // Vector path: one workgroup per tile, residency capped through LDS.  The
  // element-wise path (unaligned pointers), and the vector path with
  // MRR_LDS_CAP=0, keep a grid of wpc workgroups per CU striding over the
  // work.
  uint64_t blocks = work;
  const uint64_t g_env = max_grid_override();
  const bool capped = vector && lds_cap_enabled();
  uint64_t cap = capped ? (g_env > 0 && g_env < kCodecMaxGrid ? g_env : kCodecMaxGrid)
                        : (uint64_t)device_cu_count(-1) * wpc;
  if (!capped && g_env > 0 && g_env < cap) cap = g_env;
  if (cap == 0) cap = 2048;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) blocks = 1;  // tail only
  const dim3 grid((uint32_t)blocks);
  if (!vector) {
    hipLaunchKernelGGL(codec_scalar_k<Dir>, grid, dim3(kCodecThreads), 0, stream, in, out, n);
  } else {
    const size_t lds = capped ? occupancy_lds_bytes((int)wpc) : 0;
    switch (U) {
      case 1: launch_vec_u<Dir, 1>(grid, lds, in, out, n, stream); break;
      case 2: launch_vec_u<Dir, 2>(grid, lds, in, out, n, stream); break;
      case 4: launch_vec_u<Dir, 4>(grid, lds, in, out, n, stream); break;
      default: launch_vec_u<Dir, 8>(grid, lds, in, out, n, stream); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_codec(int dir, const void* in, void* out, size_t n, bool vector,
                        hipStream_t stream) {
  switch (dir) {
    case kDecF16: return launch_codec_dir<kDecF16>(in, out, n, vector, stream);
    case kDecF32: return launch_codec_dir<kDecF32>(in, out, n, vector, stream);
    case kEncF16: return launch_codec_dir<kEncF16>(in, out, n, vector, stream);
    case kEncF32: return launch_codec_dir<kEncF32>(in, out, n, vector, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mrr
