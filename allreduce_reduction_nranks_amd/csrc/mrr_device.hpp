// mrr_device.hpp -- element types, 16-byte vectors and conversions for gfx950.
//
// Type ids equal the public mrr_dtype values.  Every conversion here is exact
// (widening) or a single round-to-nearest-even (narrowing); FP8 E4M3B15
// narrowing saturates at +-0.9375.  The FP8 format (4 exponent bits, bias 15,
// 3 mantissa bits, largest finite 0.9375) is the one defined in the MSCCL++
// commit history entry adding the fp8_e4m3b15 datatype; since 0.9375 is the
// largest finite value, exponent field 15 encodes inf (mantissa 0) and NaN.
//
// Kernels are compiled without fast-math and with f32/f16 denormals kept, so
// f32 adds are IEEE binary32 adds and hardware converts honour denormals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mrr {

enum : int { kF32 = 1, kF16 = 2, kBF16 = 3, kFP8 = 4, kFP8FN = 5 };

// 1-byte floating-point types.
constexpr bool is_fp8(int t) { return t == kFP8 || t == kFP8FN; }

template <int T> struct Ty;
template <> struct Ty<kF32> { static constexpr int size = 4; };
template <> struct Ty<kF16> { static constexpr int size = 2; };
template <> struct Ty<kBF16> { static constexpr int size = 2; };
template <> struct Ty<kFP8> { static constexpr int size = 1; };
template <> struct Ty<kFP8FN> { static constexpr int size = 1; };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Memory access helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 ld_stream(const void* base, uint64_t vec) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + vec);
}
__device__ __forceinline__ void st_stream(void* base, uint64_t vec, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(base) + vec);
}
// 64-bit packet access, coherent across the XCDs of one device.
__device__ __forceinline__ uint64_t ld_pkt(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_pkt(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// FP8 E4M3B15 -> f32.  Moving the code's exponent and mantissa into the top of
// an f32's fields gives 2^(e-127) * (1.m) (or the f32 denormal m * 2^-129 for
// e = 0); multiplying by 2^112 rebiases to 2^(e-15) exactly.
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  float v = __uint_as_float((c & 0x7Fu) << 20) * 0x1p112f;
  uint32_t u = __float_as_uint(v);
  if ((c & 0x78u) == 0x78u) u = (c & 7u) ? 0x7FC00000u : 0x7F800000u;
  return __uint_as_float(u | sign);
}

// FP8 E4M3B15 -> f16 bits: both formats have exponent bias 15, so the fields
// line up after a shift.
__device__ __forceinline__ uint32_t fp8_to_f16(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 8;
  uint32_t mag = (c & 0x7Fu) << 7;
  if ((c & 0x78u) == 0x78u) mag = (c & 7u) ? 0x7E00u : 0x7C00u;
  return sign | mag;
}

// f32 -> FP8 E4M3B15, one round-to-nearest-even, saturating.
//  |x| >= 2^-14: rebias the exponent by -112 in the bit pattern, then round
//   the 23-bit mantissa to 3 bits by adding 2^19 - 1 plus the kept lsb; a
//   carry rolls into the exponent.  Anything past 0x77 (including inf)
//   clamps to 0x77.
//  |x| <  2^-14: the subnormal step is 2^-17, so the code is rint(|x| * 2^17)
//   (exact scaling, RNE), which reaches 8 = the first normal code.
__device__ __forceinline__ uint32_t f32_to_fp8(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  uint32_t q;
  if (a >= 0x38800000u) {
    const uint32_t r = a - (112u << 23);
    q = (r + 0x7FFFFu + ((r >> 20) & 1u)) >> 20;
    q = q < 0x77u ? q : 0x77u;
  } else {
    q = (uint32_t)__builtin_rintf(__uint_as_float(a) * 0x1p17f);
  }
  return sign | q;
}

// f16 bits -> FP8 E4M3B15: drop 7 mantissa bits with round-to-nearest-even
// (the biases agree, f16 subnormals land on FP8 subnormals), then saturate.
__device__ __forceinline__ uint32_t f16_to_fp8(uint32_t h) {
  const uint32_t sign = (h >> 8) & 0x80u;
  const uint32_t mag = h & 0x7FFFu;
  if (mag > 0x7C00u) return sign | 0x7Fu;
  uint32_t q = (mag + 0x3Fu + ((mag >> 7) & 1u)) >> 7;
  q = q < 0x77u ? q : 0x77u;
  return sign | q;
}

// OCP FP8 E4M3FN (bias 7, largest finite 448, S.1111.111 NaN, no infinity)
// -> f32: the gfx950 convert is exact for every code.
__device__ __forceinline__ float fp8fn_to_f32(uint32_t c) {
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(c, false);
  return v.x;
}

// Two f32 -> two OCP FP8 E4M3FN codes in bytes 2*HI and 2*HI+1 of `old`:
// one round-to-nearest-even each (the hardware convert), saturating at +-448
// (also for +-inf); NaN gives 0x7F with the input's sign.
template <bool HI>
__device__ __forceinline__ uint32_t encode2_fp8fn(float a, float b, uint32_t old) {
  const float ya = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float yb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, (int)old, HI);
  constexpr int sh = HI ? 16 : 0;
  if (a != a) w = (w & ~(0xFFu << sh)) | ((((__float_as_uint(a) >> 24) & 0x80u) | 0x7Fu) << sh);
  if (b != b)
    w = (w & ~(0xFFu << (sh + 8))) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7Fu) << (sh + 8));
  return w;
}

__device__ __forceinline__ uint32_t f32_to_fp8fn(float f) {
  return encode2_fp8fn<false>(f, f, 0u) & 0xFFu;
}

// ---------------------------------------------------------------------------
// Generic element access by type id (T)
// ---------------------------------------------------------------------------
template <int T> __device__ __forceinline__ float to_f32(uint32_t bits);
template <> __device__ __forceinline__ float to_f32<kF32>(uint32_t b) { return __uint_as_float(b); }
template <> __device__ __forceinline__ float to_f32<kF16>(uint32_t b) { return f16_to_f32(b); }
template <> __device__ __forceinline__ float to_f32<kBF16>(uint32_t b) { return bf16_to_f32(b); }
template <> __device__ __forceinline__ float to_f32<kFP8>(uint32_t b) { return fp8_to_f32(b); }
template <> __device__ __forceinline__ float to_f32<kFP8FN>(uint32_t b) { return fp8fn_to_f32(b); }

template <int T> __device__ __forceinline__ uint32_t from_f32(float f);
template <> __device__ __forceinline__ uint32_t from_f32<kF32>(float f) { return __float_as_uint(f); }
template <> __device__ __forceinline__ uint32_t from_f32<kF16>(float f) { return f32_to_f16(f); }
template <> __device__ __forceinline__ uint32_t from_f32<kBF16>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ uint32_t from_f32<kFP8>(float f) { return f32_to_fp8(f); }
template <> __device__ __forceinline__ uint32_t from_f32<kFP8FN>(float f) { return f32_to_fp8fn(f); }

// Rounds an f32 partial sum to the accumulator type.  The f32 add before it is
// itself rounded, but f32 carries at least 2p+2 bits for p = 11 (f16), 8 (bf16)
// and 4 (FP8), so the two roundings equal one correct rounding of the exact
// sum.  FP8 sums of two FP8 values are exact in f32 in any case.
template <int A> __device__ __forceinline__ float round_acc(float s);
template <> __device__ __forceinline__ float round_acc<kF32>(float s) { return s; }
template <> __device__ __forceinline__ float round_acc<kF16>(float s) { return (float)(_Float16)s; }
template <> __device__ __forceinline__ float round_acc<kBF16>(float s) {
  return bf16_to_f32(f32_to_bf16(s));
}
template <> __device__ __forceinline__ float round_acc<kFP8>(float s) {
  return fp8_to_f32(f32_to_fp8(s));
}
template <> __device__ __forceinline__ float round_acc<kFP8FN>(float s) {
  return s != s ? s : fp8fn_to_f32(f32_to_fp8fn(s));
}

// Element i of a buffer of type T, widened to f32.
template <int T> __device__ __forceinline__ float load_elem(const void* p, uint64_t i) {
  if constexpr (T == kF32) return __uint_as_float(reinterpret_cast<const uint32_t*>(p)[i]);
  else if constexpr (Ty<T>::size == 2) return to_f32<T>(reinterpret_cast<const uint16_t*>(p)[i]);
  else return to_f32<T>(reinterpret_cast<const uint8_t*>(p)[i]);
}
template <int T> __device__ __forceinline__ void store_elem(void* p, uint64_t i, float v) {
  if constexpr (T == kF32) reinterpret_cast<uint32_t*>(p)[i] = __float_as_uint(v);
  else if constexpr (Ty<T>::size == 2) reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)from_f32<T>(v);
  else reinterpret_cast<uint8_t*>(p)[i] = (uint8_t)from_f32<T>(v);
}

// ---------------------------------------------------------------------------
// FP8 E4M3B15 through the gfx950 OCP FP8 converts.
//
// The hardware converts between f32 and OCP FP8 E4M3 (bias 7) exactly
// (decode) and with round-to-nearest-even (encode), subnormals included.  For
// exponent fields 0..14 an E4M3B15 code has the bit layout of the E4M3 code
// of 2^8 times its value, subnormals included, so
//   decode_b15(c) = decode_e4m3(c) * 2^-8       (one scaled convert)
//   encode_b15(x) = encode_e4m3(clamp(x * 2^8, -240, 240))
// where 240 = 0.9375 * 2^8 is the largest E4M3B15 value, so the clamp is the
// saturation.  Exponent field 15 differs (inf / NaN here, finite or NaN in
// E4M3): codes with it are detected per word and fixed up, and values
// derived from them take the exact bit-arithmetic path above.
// ---------------------------------------------------------------------------
// Finite f32 -> E4M3B15 bits of a pair, packed into the low (HI = false) or
// high (HI = true) 16 bits of `old`; the other half of `old` is kept.
template <bool HI>
__device__ __forceinline__ uint32_t encode2_fp8_hw(float a, float b, uint32_t old) {
  const float ya = __builtin_amdgcn_fmed3f(a * 256.0f, -240.0f, 240.0f);
  const float yb = __builtin_amdgcn_fmed3f(b * 256.0f, -240.0f, 240.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, (int)old, HI);
}

// 16 finite f32 values -> one 16-byte vector of E4M3B15 codes.
__device__ __forceinline__ u32x4 encode16_fp8_hw(const float* x) {
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = encode2_fp8_hw<false>(x[4 * j], x[4 * j + 1], 0u);
    v[j] = encode2_fp8_hw<true>(x[4 * j + 2], x[4 * j + 3], w);
  }
  return v;
}

// Rounds a finite f32 sum to the E4M3B15 grid (native FP8 accumulation).
__device__ __forceinline__ float round_fp8_hw(float s) {
  const uint32_t c = encode2_fp8_hw<false>(s, s, 0u);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 0x1p-8f, false);
  return d.x;
}

// ---------------------------------------------------------------------------
// Word-level access: a lane's share of one rank is D 32-bit words (D = 1, 2
// or 4), loaded with one non-temporal D-word load.
// ---------------------------------------------------------------------------
template <int D> struct WordsT;
template <> struct WordsT<1> { typedef uint32_t type; };
template <> struct WordsT<2> { typedef uint32_t type __attribute__((ext_vector_type(2))); };
template <> struct WordsT<4> { typedef uint32_t type __attribute__((ext_vector_type(4))); };

// Loads unit `unit` (D words) of a buffer.
template <int D> __device__ __forceinline__ void ld_words(const void* base, uint64_t unit, uint32_t* w) {
  typedef typename WordsT<D>::type V;
  const V v = __builtin_nontemporal_load(reinterpret_cast<const V*>(base) + unit);
  if constexpr (D == 1) {
    w[0] = v;
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) w[j] = v[j];
  }
}

// Stores D words as unit `unit` of a buffer (D-word units), non-temporal.
template <int D> __device__ __forceinline__ void st_words(void* base, uint64_t unit, const uint32_t* w) {
  typedef typename WordsT<D>::type V;
  V v;
  if constexpr (D == 1) {
    v = w[0];
  } else {
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] = w[j];
  }
  __builtin_nontemporal_store(v, reinterpret_cast<V*>(base) + unit);
}

// Elements of type T in one 32-bit word, widened to f32.
template <int T> __device__ __forceinline__ void decode_word(uint32_t w, float* x) {
  if constexpr (T == kF32) {
    x[0] = __uint_as_float(w);
  } else if constexpr (T == kF16) {
    const f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
    x[0] = p.x;
    x[1] = p.y;
  } else if constexpr (T == kBF16) {
    x[0] = __uint_as_float(w << 16);
    x[1] = __uint_as_float(w & 0xFFFF0000u);
  } else if constexpr (T == kFP8FN) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    x[0] = lo.x;
    x[1] = lo.y;
    x[2] = hi.x;
    x[3] = hi.y;
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) x[b] = fp8_to_f32((w >> (8 * b)) & 0xFFu);
  }
}

// Four FP8 E4M3B15 codes through the hardware converts (exact for exponent
// fields <= 14), see the FP8 section above.
__device__ __forceinline__ void decode_word_fp8_hw(uint32_t w, float* x) {
  const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 0x1p-8f, false);
  const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 0x1p-8f, true);
  x[0] = lo.x;
  x[1] = lo.y;
  x[2] = hi.x;
  x[3] = hi.y;
}

// Bit 7 of byte b of the result is set exactly when byte b of w has
// exponent field 15 (inf or NaN in E4M3B15): (b & 0x78) + 8 reaches 0x80 only
// from 0x78, and no byte carries into the next.  The marks of many words are
// OR-ed together and tested once against kFp8E15Bits.
__device__ __forceinline__ uint32_t fp8_e15_marks(uint32_t w) { return (w & 0x78787878u) + 0x08080808u; }
constexpr uint32_t kFp8E15Bits = 0x80808080u;

// ---------------------------------------------------------------------------
// 16-byte vector decode / encode.  An input vector holds VW = 16 / size(In)
// elements; its output holds VW * size(Out) bytes = OV 16-byte vectors.
// ---------------------------------------------------------------------------
template <int T> struct Vec {
  static constexpr int VW = 16 / Ty<T>::size;
};

template <int T> __device__ __forceinline__ void decode16(const u32x4 v, float* x) {
  if constexpr (T == kF32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __uint_as_float(v[j]);
  } else if constexpr (T == kF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // copy the lane out first: a bit_cast applied to a vector element
      // expression reads element 0 whatever the index
      const uint32_t w = v[j];
      const f32x2 p = __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
      x[2 * j] = p.x;
      x[2 * j + 1] = p.y;
    }
  } else if constexpr (T == kBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(v[j] << 16);
      x[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) x[4 * j + b] = fp8_to_f32((v[j] >> (8 * b)) & 0xFFu);
    }
  }
}

// Packs n = 16 / size(T) f32 values (already members of T, or to be rounded
// into T) into one 16-byte vector of type T.
template <int T> __device__ __forceinline__ u32x4 encode16(const float* x) {
  u32x4 v;
  if constexpr (T == kF32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __float_as_uint(x[j]);
  } else if constexpr (T == kF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x2 p;
      p.x = x[2 * j];
      p.y = x[2 * j + 1];
      v[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, f16x2));
    }
  } else if constexpr (T == kBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x2 p;
      p.x = x[2 * j];
      p.y = x[2 * j + 1];
      v[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2));
    }
  } else if constexpr (T == kFP8FN) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = encode2_fp8fn<false>(x[4 * j], x[4 * j + 1], 0u);
      v[j] = encode2_fp8fn<true>(x[4 * j + 2], x[4 * j + 3], w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= from_f32<T>(x[4 * j + b]) << (8 * b);
      v[j] = w;
    }
  }
  return v;
}

// 8 f32 values -> two words of FP8 codes of type T (E4M3B15 or E4M3FN), one
// rounding each.  For E4M3B15, `exact` selects the bit-arithmetic encoder
// (units holding inf / NaN); otherwise the hardware converts.
template <int T> __device__ __forceinline__ void encode8_fp8(const float* x, bool exact, uint32_t* w) {
  static_assert(T == kFP8 || T == kFP8FN, "FP8 output types only");
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (T == kFP8FN) {
      w[j] = encode2_fp8fn<true>(x[4 * j + 2], x[4 * j + 3], encode2_fp8fn<false>(x[4 * j], x[4 * j + 1], 0u));
    } else {
      if (exact) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= f32_to_fp8(x[4 * j + b]) << (8 * b);
        w[j] = v;
      } else {
        w[j] = encode2_fp8_hw<true>(x[4 * j + 2], x[4 * j + 3],
                                    encode2_fp8_hw<false>(x[4 * j], x[4 * j + 1], 0u));
      }
    }
  }
}

}  // namespace mrr
