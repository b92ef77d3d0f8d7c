// rsag.hip -- RS/AG zero-copy N-rank reduction kernels for gfx950.
//
// Operation ("Support 2 ranks in AllreduceRsAgZeroCopy", MSCCL++ PR #948,
// sections "why" and "what changed"): rank r reads chunk r of every rank's
// input, reduces it, and writes the reduced chunk into every rank's output.
// One kernel instance is compiled per rank count (2, 4, 8, 16 and 32), each
// with its loops over the ranks fully unrolled.
//
// MI355X mapping.  All N rank buffers live in this GPU's HBM, so one launch
// performs every rank's share (or one chosen rank's share).  The work is
// HBM-bound (N*S bytes read, N*S written, ~N VALU adds per element); what
// decides the bandwidth is how many bytes are in flight and how the 2N
// same-offset streams hit the DRAM banks:
//   - the reduce-scatter partition is kept at tile granularity: chunks are
//     ceil(count / N) elements rounded up to 256 bytes of input (so every
//     chunk starts on the cache-line grid), tile i of the launch is tile
//     (i % tiles_per_chunk) of chunk first_chunk + i / tiles_per_chunk, and
//     no tile straddles two chunks;
//   - one single-wave (64-lane) workgroup per tile, so the hardware
//     dispatcher hands tiles out in launch order as workgroups retire and the
//     2N active address windows stay as narrow as the resident workgroups;
//     each lane owns U units of a tile, a unit being one 16-byte output
//     vector and its 4 to 16 input bytes per rank (lane-contiguous, so every
//     store instruction covers 1 KiB of one buffer), issues the loads of a
//     rank group together (non-temporal: the data is touched once),
//     accumulates in rank order 0..N-1, narrows once and stores the result
//     to all N outputs (the all-gather) with non-temporal 16-byte stores,
//     written through to HBM at device scope where that measured faster
//     (rsag_dev_stores);
//   - few waves per CU stream best (two to twelve single-wave workgroups
//     per CU, see the launch-shape table below): more loads in flight thrash
//     DRAM rows across the 2N same-offset buffers, fewer leave HBM latency
//     exposed.  The cap is enforced by giving each workgroup an LDS
//     reservation of 1/cap of the CU's LDS, which the kernels never touch.
//   - A persistent grid that strides over the tiles was measured slower on
//     MI355X, increasingly so the more tiles each workgroup walks (8 x 256 MiB
//     bf16: 0.69 of the HBM peak against 0.77; 2 x 2 GiB: 0.66 against 0.74):
//     workgroups drift apart over a long launch and the active windows widen.
// No __restrict__: an output may be its own rank's input (in place); a lane
// reads every element it writes before writing it.
#include <stdlib.h>

#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

constexpr int kRsagThreads = 64;  // one wave per workgroup (all kernels but one shape below)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Fourth word of a raw buffer descriptor on gfx9-family GPUs: 32-bit data
// format, no swizzle, no index stride.
constexpr uint32_t kBufferWord3 = 0x00020000u;

// Streaming store at device scope (sc1 nt): written through to memory rather
// than held in the XCD's L2 until evicted.  Issued as a buffer store whose
// descriptor starts at the unit of the wave's first active lane and spans 64
// units, so the active lanes must hold consecutive units from that lane on
// (lane-contiguous tiles, or a prefix of one); a store outside the span is
// dropped by the range check, never written elsewhere.  B = 16 or 8 bytes.
template <int B, typename V>
__device__ __forceinline__ void st_stream_dev(void* base, uint64_t unit, V v) {
  static_assert(B == 16 || B == 8, "16- or 8-byte units");
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)unit);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(unit >> 32));
  const uint64_t first = ((uint64_t)hi << 32) | lo;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<char*>(base) + first * B, (short)0, 64 * B, kBufferWord3);
  constexpr int kDevNt = 18;  // cache policy: sc1 (device scope) | nt
  if constexpr (B == 16)
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (uint32_t)(unit - first) * 16u, 0, kDevNt);
  else
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (uint32_t)(unit - first) * 8u, 0, kDevNt);
}
// Streaming 16-byte store, device scope or not.
template <bool kDev>
__device__ __forceinline__ void st_out(void* base, uint64_t vec, u32x4 v) {
  if constexpr (kDev) st_stream_dev<16>(base, vec, v);
  else st_stream(base, vec, v);
}

// Launch shape, from sweeps of (units per lane U) x (workgroups per CU) of
// this kernel on MI355X at 64 MiB and 256 MiB per rank (16- and 32-bit
// inputs) and 32 MiB per rank (FP8 inputs at 8 ranks).  Streaming bandwidth is
// bumpy in both knobs -- the 2N same-offset streams interact with the DRAM
// channel and bank mapping -- so each entry is the setting that stayed near
// the best across buffer sizes rather than a formula.
//   16-bit and 32-bit inputs: N=2 U=2 x12, N=4 U=1 x8, N=8 U=1 x6 (x8
//                             before; three alternating runs of the
//                             benchmark each, one session: 8 x 64 MiB f16
//                             164.6 against 164.9 us, 8 x 32 MiB f16 84.6
//                             against 88.7 us, 8 x 256 MiB bf16 691.4
//                             against 687.5 us; f32 data 0.82 against
//                             0.78),
//                             N=16 U=1 x4, N=32 U=1 x4 with loads in groups of
//                             8 ranks (fractions of the HBM peak at 64 / 256 MiB
//                             per rank, with the store policy of
//                             rsag_dev_stores: N=2 0.81 / 0.83, N=4 0.83 / 0.81,
//                             N=8 0.82 (f16) / 0.78, N=16 0.79 / 0.76-0.77,
//                             N=32 0.74 / 0.78; with groups of 16 ranks at 8
//                             per CU, N=32 ran 0.70 / 0.70)
//   FP8 inputs (E4M3B15 and OCP E4M3FN), N>2: U=1 for FP8 and f16 outputs
//                             (U=2 for E4M3B15 at N=4: at its best cap, x6,
//                             0.77-0.78 / 0.77 to FP8 / f16 against 0.77 /
//                             0.76 for U=1 at x12 / x16; E4M3FN loses 4-5 %
//                             with U=2),
//                             U=2 (128-lane tiles, below) x2 for f32 outputs,
//                             which at most rank counts take
//                             rsag_wide_f32_kernel instead (rsag_wide_wg_per_cu);
//                             N=2: U=4 times 2 for f16 and 4 for f32 outputs
//                             (a lane loads 16 bytes per rank).  Workgroups per
//                             CU, swept 4-16 at 32 MiB per rank with the store
//                             policy of rsag_dev_stores (fractions of the HBM
//                             peak at the chosen cap, E4M3B15 / E4M3FN, two
//                             sessions):
//                               FP8 out: N=2 x10 (0.78 / 0.76), N=4 x6 (U=2) / x10
//                                 (0.77 / 0.79), N=8 x6 (0.82 / 0.82),
//                                 N=16 x4 (0.77 / 0.80), N=32 x4 (0.75 / 0.74);
//                               f16 out: N=2 x8 / x4 (0.79 / 0.76), N=4 x6 (U=2) / x10
//                                 (0.77 / 0.81), N=8 x6 (0.82 / 0.82),
//                                 N=16 x4 (0.75 / 0.77), N=32 x6 (0.71 / 0.71).
//                             A paired sweep (every cap timed in turn on the
//                             same buffers, three processes) put this table
//                             within 0.6 % of the best cap at every FP8 shape
//                             and 16-bit shape at 2-32 ranks, after moving
//                             E4M3FN -> f16 at 32 ranks from x4 to x6 (+1.4 %).
//                             At 4 ranks fewer than 8 workgroups per CU starve
//                             the memory system (E4M3B15 -> f16 0.39 at 4,
//                             0.59 at 8).
//   One-pass FP8 -> f16 + FP8 (rsag_dual_kernel): U=2 x4 (U=8 x4 at N=2; 2-8
//                             swept at 8 x 32 MiB and 2 x 32 MiB).
//   Workgroup width: 64 lanes, except FP8 inputs with f32 outputs above two
//   ranks, which run two-wave (128-lane) tiles at 2 workgroups per CU:
//   8 x 32 MiB E4M3B15 0.69 -> 0.74 of the HBM peak, E4M3FN 0.68 -> 0.75.
//   Wider tiles lost elsewhere (FP8 and one-pass outputs, 16-bit data at 2,
//   8 and 32 ranks).
constexpr int rsag_threads(int n, int tin, int tout) {
  return is_fp8(tin) && tout == kF32 && n > 2 ? 128 : kRsagThreads;
}
constexpr int rsag_unroll(int n, int tin, int tout) {
  if (is_fp8(tin)) {
    if (n == 2) return 4 * (tout == kF32 ? 4 : tout == kF16 ? 2 : 1);
    if (n == 4 && tin == kFP8 && tout != kF32) return 2;
    return tout == kF32 ? 2 : 1;
  }
  return n == 2 ? 2 : 1;
}
constexpr int rsag_wg_per_cu(int n, int tin, int tout) {
  if (is_fp8(tin)) {
    const bool fn = tin == kFP8FN;
    const bool f16 = tout == kF16;
    if (tout == kF32) return n == 2 && !fn ? 8 : 2;  // 128-lane workgroups above 2 ranks
    switch (n) {
      case 2: return f16 ? (fn ? 4 : 8) : 10;
      case 4: return fn ? 10 : 6;  // E4M3B15: two units per lane
      case 16: return 4;
      case 32: return f16 ? 6 : 4;
      default: return 6;
    }
  }
  return n == 2 ? 12 : n == 4 ? 8 : n == 8 ? 6 : 4;
}
// Output stores at device scope (sc1 nt, st_stream_dev) or plain streaming
// (nt).  Device-scope stores are written through to HBM instead of waiting in
// the XCD's L2 for eviction.  Measured on MI355X (two sessions, each kernel at
// its best cap under either policy, fractions of the HBM peak, nt -> sc1 nt):
//   16-bit data: N=2 0.81 -> 0.78 at 64 MiB per rank (kept nt), N=4 0.81-0.82
//     -> 0.81-0.84, N=8 0.815-0.825 -> 0.811-0.825 (f16 a tie, bf16 1 % down:
//     kept nt), N=16 0.74-0.78 -> 0.76-0.79, N=32 0.73-0.78 -> 0.74-0.78;
//   f32 data (64 / 256 MiB per rank): N=2 0.80 / 0.83 -> 0.78 / 0.84 (kept
//     nt), N=4 0.83 / 0.82 -> 0.83 / 0.83, N=8 0.82 / 0.78 -> 0.82 / 0.80
//     (kept nt), N=16 0.77 / 0.77 -> 0.79 / 0.81,
//     N=32 0.73 / 0.77 -> 0.74 / 0.78;
//   FP8 data (E4M3B15 / E4M3FN, 32 MiB per rank) to FP8 or f16: +2 to +4 % at
//     N=2 (E4M3FN -> f16 a tie), -1 to -3 % at N=4 (kept nt), +0 to +3 % at
//     N=8, +1 to +3 % at 16 and +0 to +3 % at 32 ranks;
//   FP8 to f32 (128-lane tiles at N=8): 0.72-0.73 -> 0.77 at N=8; E4M3FN at
//     N=2 (64-lane, 16 codes per lane) 0.765 -> 0.741 (kept nt).
// The wide FP8 -> f32 kernel and the one-pass FP8 -> f16 + FP8 kernel always
// store at device scope (see them below).
constexpr bool rsag_dev_stores(int n, int tin, int tout) {
  if (!is_fp8(tin)) return n == 4 || n >= 16;
  if (tout == kF32) return n != 2;
  return n != 4;
}
// Large buffers of 16- or 32-bit data at 8 ranks (from 128 MiB of input per
// rank) and 2 ranks (from 256 MiB): a second instance of the kernel stores at
// device scope, at 4 (8 ranks) or 8 (2 ranks) workgroups per CU.  Measured on
// MI355X with three alternating runs of the benchmark per setting in one
// session (us per call):
//   8 ranks, plain stores at 6 per CU / device scope at 6 / device scope at
//   4: 8 x 256 MiB bf16 689.7 / 693.0 / 683.3, 8 x 128 MiB 331.8 / 333.4 /
//   327.2, 8 x 64 MiB f16 165.3 / 166.5 / 165.6;
//   2 ranks, plain stores at 12 per CU / device scope at 12 / device scope
//   at 8: 2 x 512 MiB bf16 333.0 / 326.4 / 324.2, 2 x 256 MiB 165.0 / 162.2
//   / 161.8, 2 x 128 MiB 82.3 / 83.3 / 85.2.
constexpr bool rsag_large_dev(int n, int tin, uint64_t bytes_per_rank) {
  if (is_fp8(tin)) return false;
  if (n == 8) return bytes_per_rank >= ((uint64_t)128 << 20);
  if (n == 2) return bytes_per_rank >= ((uint64_t)256 << 20);
  return false;
}
constexpr int rsag_large_dev_wg_per_cu(int n) { return n == 8 ? 4 : 8; }
// FP8 -> f32: workgroups per CU of rsag_wide_f32_kernel (16-value units,
// stores through LDS), or 0 where the general kernel above stays faster.
// Measured on MI355X, 32 MiB of codes per rank, fractions of the HBM peak,
// general kernel -> wide kernel at its best cap (2-12 swept):
//   E4M3B15: N=2 0.68 -> 0.74 (x12), N=4 0.67 -> 0.72 (x6), N=8 0.71 -> 0.72
//            (x4, a tie: kept general), N=16 0.69 -> 0.70 (x2), N=32 0.63 -> 0.66 (x2);
//   E4M3FN:  N=2 0.76 -> 0.75 (kept general), N=4 0.62 -> 0.73 (x6), N=8 0.74 -> 0.71
//            (kept general), N=16 0.69 -> 0.71 (x2), N=32 0.65 -> 0.67 (x2).
// With the one-branch exponent-15 check the general kernel at 8 ranks runs
// 0.74 for both formats at 2 per CU, against 0.71 for this one.  Its stores
// are at device scope: E4M3B15 N=2 0.75 -> 0.78 (x12), N=4 0.75 -> 0.76 (x8
// instead of x6), N=16 0.59-0.67 -> 0.71-0.73, N=32 0.65 -> 0.68.
constexpr int rsag_wide_wg_per_cu(int n, int tin) {
  return n == 2 ? (tin == kFP8 ? 12 : 0) : n == 4 ? 8 : (n == 16 || n == 32) ? 2 : 0;
}
// One-pass FP8 -> f16 + FP8: device-scope stores for both outputs (8 x 32 MiB
// E4M3B15 0.751 -> 0.759, E4M3FN 0.757 -> 0.772, 2 x 32 MiB 0.722 -> 0.742).
constexpr int rsag_dual_unroll(int n) { return n == 2 ? 8 : 2; }
constexpr int rsag_dual_wg_per_cu(int) { return 4; }
// Ranks whose vectors are loaded together before they are added: all of them
// up to 16 ranks; groups of 8 above that (measured on MI355X at 32 ranks:
// groups of 8 at 4 workgroups per CU 0.72-0.77 of the HBM peak at 32-256 MiB
// per rank, against 0.66-0.70 for groups of 16 at 8 per CU and 0.54-0.57 at
// 4 per CU), and groups of 8 for FP8 inputs or an FP8 accumulator (16 values
// per vector and two decode paths make the unrolled body large).
constexpr int rsag_group(int n, int tin, int tacc) {
  return (is_fp8(tin) || is_fp8(tacc)) ? (n < 8 ? n : 8) : (n <= 16 ? n : 8);
}

// Out2 != 0: the same sum is also written, as type Out2, to out2[0..n-1].
template <int In, int Acc, int Out, int Out2 = 0>
__device__ __forceinline__ void reduce_elem(const void* const* in, void* const* out, int n,
                                            uint64_t i, void* const* out2 = nullptr) {
  float acc = round_acc<Acc>(load_elem<In>(in[0], i));
  for (int r = 1; r < n; ++r) acc = round_acc<Acc>(acc + load_elem<In>(in[r], i));
  for (int k = 0; k < n; ++k) store_elem<Out>(out[k], i, acc);
  if constexpr (Out2 != 0)
    for (int k = 0; k < n; ++k) store_elem<Out2>(out2[k], i, acc);
}

// A unit is one 16-byte output vector: UE = 16 / size(Out) elements, whose
// inputs are D = UE * size(In) / 4 words per rank (4, 2 or 1).  Keeping the
// output side at 16 bytes per lane makes every store instruction write 1 KiB
// of contiguous memory, whatever the input width.
template <int In, int Out> struct Unit {
  static constexpr int UE = 16 / Ty<Out>::size;
  static constexpr int D = UE * Ty<In>::size / 4;
  static constexpr int EPW = 4 / Ty<In>::size;  // elements per input word
};

// E4M3B15 units holding an exponent-15 code (inf / NaN) are reduced again
// here, from memory: the exact decode, every partial sum rounded exactly to
// Acc (the hardware converts the fast path uses are exact for finite data
// only).  unit indexes D-word units of every input.
template <int D, int Acc>
__device__ __forceinline__ void fp8_unit_exact(const void* const* in, int n, uint64_t unit,
                                               float* acc) {
#pragma unroll 1
  for (int r = 0; r < n; ++r) {
    uint32_t w[D];
    ld_words<D>(in[r], unit, w);
#pragma unroll
    for (int j = 0; j < D; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float x = fp8_to_f32((w[j] >> (8 * b)) & 0xFFu);
        acc[4 * j + b] = round_acc<Acc>(r == 0 ? x : acc[4 * j + b] + x);
      }
    }
  }
}

// Reduces UU units v0 + u * T (u < UU; T lanes per workgroup) over the N ranks and stores
// each result to all N outputs.  The first partial sum is x_0 rounded to the
// accumulator type (the identity except for an FP8 accumulator, which
// saturates an infinite x_0 like any later sum).  Ranks are taken in groups
// of G: the group's UU * G loads are all issued before the first add of the
// group, then the adds run in rank order.
//
// FP8 inputs decode through the hardware E4M3 converts.  For E4M3B15 every
// loaded word also adds to the unit's exponent-15 marks; a unit that holds an
// exponent-15 code (inf / NaN) is `special`: after the rank loop it is
// reduced again by fp8_unit_exact and encoded with the exact bit arithmetic.
// One branch per unit, taken only for such data.
//
// Out2 != 0 (FP8 types only, with Out = f16): each unit's 8 sums are also
// encoded to Out2 and stored, 8 bytes per lane, to out2[0..N-1].
// kLarge: the instance for large buffers at 2 and 8 ranks (rsag_large_dev),
// which stores at device scope.
template <int N, int In, int Acc, int Out, int UU, int G, int Out2 = 0, int T = kRsagThreads,
          bool kLarge = false>
__device__ __forceinline__ void reduce_store(const RsagArgs& a, uint64_t v0,
                                             void* const* out2 = nullptr) {
  constexpr int UE = Unit<In, Out>::UE;
  constexpr int D = Unit<In, Out>::D;
  constexpr int EPW = Unit<In, Out>::EPW;
  static_assert(N % G == 0, "rank group must divide N");
  float acc[UU][UE];
  bool special[UU];
  uint32_t marks[UU];
#pragma unroll
  for (int u = 0; u < UU; ++u) marks[u] = 0;
  constexpr int kGroupUnroll = N / G <= 2 ? N / G : 1;
#pragma unroll kGroupUnroll
  for (int g = 0; g < N; g += G) {
    uint32_t raw[UU][G][D];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
#pragma unroll
      for (int r = 0; r < G; ++r) ld_words<D>(a.in[g + r], v0 + (uint64_t)u * T, raw[u][r]);
    }
#pragma unroll
    for (int u = 0; u < UU; ++u) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float x[UE];
#pragma unroll
        for (int j = 0; j < D; ++j) {
          if constexpr (In == kFP8) {
            decode_word_fp8_hw(raw[u][r][j], x + j * EPW);
            marks[u] |= fp8_e15_marks(raw[u][r][j]);
          } else {
            decode_word<In>(raw[u][r][j], x + j * EPW);
          }
        }
#pragma unroll
        for (int j = 0; j < UE; ++j) {
          const float s = g + r == 0 ? x[j] : acc[u][j] + x[j];
          if constexpr (Acc == kFP8) acc[u][j] = round_fp8_hw(s);
          else acc[u][j] = round_acc<Acc>(s);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    special[u] = (marks[u] & kFp8E15Bits) != 0u;
    if constexpr (In == kFP8) {
      if (special[u]) fp8_unit_exact<D, Acc>(a.in, N, v0 + (uint64_t)u * T, acc[u]);
    }
  }
  // Store order: at 16 ranks each workgroup starts its N stores at output
  // blockIdx % 16, so the workgroups in flight spread their writes over all
  // output buffers instead of all writing output 0 first.  Measured on MI355X
  // (16 x 256 MiB bf16, four alternating A/B pairs): 1365-1368 us against
  // 1385-1387 us in output order; at 8 and 32 ranks the rotation was 0.5-1 %
  // slower, so they keep output order, as do FP8 inputs (not measured).
  constexpr bool kRotate = N == 16 && !is_fp8(In);
  constexpr bool kDev = Out2 != 0 || kLarge || rsag_dev_stores(N, In, Out);
  const int k0 = kRotate ? (int)(blockIdx.x & (N - 1)) : 0;
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    const uint64_t v = v0 + (uint64_t)u * T;
    u32x4 o;
    if constexpr (Out == kFP8) o = special[u] ? encode16<kFP8>(acc[u]) : encode16_fp8_hw(acc[u]);
    else o = encode16<Out>(acc[u]);
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if constexpr (kRotate) st_out<kDev>(a.out[(k + k0) & (N - 1)], v, o);
      else st_out<kDev>(a.out[k], v, o);
    }
    if constexpr (Out2 != 0) {
      static_assert(UE == 8, "second FP8 output needs 8-element units");
      uint32_t w2[2];
      encode8_fp8<Out2>(acc[u], special[u], w2);
      u32x2 o2;
      o2[0] = w2[0];
      o2[1] = w2[1];
#pragma unroll
      for (int k = 0; k < N; ++k) st_stream_dev<8>(out2[k], v, o2);
    }
  }
}

// The persistent tile loop shared by the single- and dual-output kernels.
template <int N, int In, int Acc, int Out, int U, int Out2, int T = kRsagThreads, bool kLarge = false>
__device__ __forceinline__ void rsag_vec_body(const RsagArgs& a, void* const* out2) {
  constexpr int G = rsag_group(N, In, Acc);
  for (uint32_t i = blockIdx.x; i < a.launch_tiles; i += gridDim.x) {
    const uint32_t chunk_rel = i / a.tiles_per_chunk;
    const uint32_t tile = i - chunk_rel * a.tiles_per_chunk;
    const uint64_t v_lo = (uint64_t)(a.first_chunk + chunk_rel) * a.chunk_vecs;
    const uint64_t v_hi = v_lo + a.chunk_vecs < a.total_vecs ? v_lo + a.chunk_vecs : a.total_vecs;
    const uint64_t v0 = v_lo + (uint64_t)tile * (T * U) + threadIdx.x;
    if (v0 + (uint64_t)(U - 1) * T < v_hi) {
      reduce_store<N, In, Acc, Out, U, G, Out2, T, kLarge>(a, v0, out2);
    } else {  // the last, partial tile of a chunk: unit by unit
#pragma nounroll
      for (int u = 0; u < U; ++u) {
        const uint64_t v = v0 + (uint64_t)u * T;
        if (v < v_hi) reduce_store<N, In, Acc, Out, 1, G, Out2, T, kLarge>(a, v, out2);
      }
    }
  }
  // Elements past the last whole unit (count % UE of them, fewer than one
  // wave) go to the last workgroup, one per lane.
  if (a.tail_count != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < a.tail_count)
    reduce_elem<In, Acc, Out, Out2>(a.in, a.out, N, a.tail_begin + threadIdx.x, out2);
}

template <int N, int In, int Acc, int Out, int U, int T, bool kLarge>
__global__ void __launch_bounds__(T) rsag_vec_kernel(const RsagArgs a) {
  rsag_vec_body<N, In, Acc, Out, U, 0, T, kLarge>(a, nullptr);
}

// FP8 inputs, f16 outputs plus the FP8 re-encode of the same sums.
template <int N, int In, int Acc, int U>
__global__ void __launch_bounds__(kRsagThreads) rsag_dual_kernel(const RsagDualArgs d) {
  rsag_vec_body<N, In, Acc, kF16, U, In>(d.base, d.out2);
}

// FP8 inputs, f32 outputs: a 1:4 read:write mix.  Here a unit is 16 input
// bytes per rank (16 FP8 values, one 16-byte load) and 64 output bytes per
// rank.  A lane sums its 16 values in rank order; the wave then passes its
// 64 x 16 sums through 4 KiB of LDS so that lane l holds output vector l of
// each of the tile's four 1 KiB output blocks, and every store instruction
// writes 1 KiB contiguous -- with 4-value units (the general kernel) a lane
// loads only 4 bytes per rank.  Chunks are whole 256-element blocks, so a
// tile's store blocks are whole or empty except at the end of the buffer,
// where lanes past the last whole unit store nothing.
constexpr int kWideUE = 16;  // elements per unit
constexpr size_t kWideLds = 4 * kRsagThreads * sizeof(u32x4);

template <int N, int In, int Acc>
__global__ void __launch_bounds__(kRsagThreads) rsag_wide_f32_kernel(const RsagArgs a) {
  constexpr int G = rsag_group(N, In, Acc);
  __shared__ u32x4 tr[4 * kRsagThreads];
  const uint32_t lane = threadIdx.x;
  for (uint32_t i = blockIdx.x; i < a.launch_tiles; i += gridDim.x) {
    const uint32_t chunk_rel = i / a.tiles_per_chunk;
    const uint32_t tile = i - chunk_rel * a.tiles_per_chunk;
    const uint64_t v_lo = (uint64_t)(a.first_chunk + chunk_rel) * a.chunk_vecs;
    const uint64_t v_hi = v_lo + a.chunk_vecs < a.total_vecs ? v_lo + a.chunk_vecs : a.total_vecs;
    const uint64_t u_base = v_lo + (uint64_t)tile * kRsagThreads;
    if (u_base >= v_hi) continue;  // a tile past the buffer's last whole unit (wave-uniform)
    // Lanes past the end load unit u_base instead (in range), so no load waits on a branch.
    const uint64_t u = u_base + lane < v_hi ? u_base + lane : u_base;
    float acc[kWideUE];
    uint32_t marks = 0;
#pragma unroll 1
    for (int g = 0; g < N; g += G) {
      u32x4 raw[G];
#pragma unroll
      for (int r = 0; r < G; ++r) raw[r] = ld_stream(a.in[g + r], u);
#pragma unroll
      for (int r = 0; r < G; ++r) {
        float x[kWideUE];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = raw[r][j];
          if constexpr (In == kFP8) {
            decode_word_fp8_hw(w, x + 4 * j);
            marks |= fp8_e15_marks(w);
          } else {
            decode_word<In>(w, x + 4 * j);
          }
        }
#pragma unroll
        for (int j = 0; j < kWideUE; ++j) {
          const float s = g + r == 0 ? x[j] : acc[j] + x[j];
          if constexpr (Acc == kFP8) acc[j] = round_fp8_hw(s);
          else acc[j] = round_acc<Acc>(s);
        }
      }
    }
    if constexpr (In == kFP8) {
      if ((marks & kFp8E15Bits) != 0u) fp8_unit_exact<4, Acc>(a.in, N, u, acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(acc[4 * j + e]);
      tr[4 * lane + j] = o;
    }
    __syncthreads();
    const uint64_t w_base = u_base * 4;  // first 16-byte f32 output vector of the tile
    const uint64_t w_hi = v_hi * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t w = w_base + (uint64_t)j * kRsagThreads + lane;
      const u32x4 o = tr[j * kRsagThreads + lane];
      if (w < w_hi) {
#pragma unroll
        for (int k = 0; k < N; ++k) st_stream_dev<16>(a.out[k], w, o);
      }
    }
    __syncthreads();  // the next tile rewrites tr
  }
  if (a.tail_count != 0 && blockIdx.x == gridDim.x - 1 && lane < a.tail_count)
    reduce_elem<In, Acc, kF32>(a.in, a.out, N, a.tail_begin + lane);
}

// Runtime rank count (1..32): the fallback for counts without a compiled
// kernel.  Ranks are taken in groups of G behind wavefront-uniform bounds, in
// rank order, with the same unit structure as reduce_store: all loads of a
// group are issued before its first add.  G is 16 for 9 to 20 ranks of 16- or
// 32-bit data and 8 otherwise (FP8 data or accumulator, up to 8 ranks, above
// 20 ranks).  Measured on MI355X, 64 MiB of bf16 per rank at 4 workgroups
// per CU, groups of 16 -> 8: 24 ranks 0.727 -> 0.748, 28 ranks 0.713 ->
// 0.733, 31 ranks 0.699 -> 0.721; at 12 and 20 ranks groups of 8 were
// 1-2 % slower in an earlier session and equal in this one.
constexpr int kAnyGroup = 8;
constexpr int kAnyGroupWide = 16;
constexpr int kAnyGroupWideMaxRanks = 20;

// kDev: device-scope output stores (st_stream_dev); the launcher picks them
// per rank count (rsag_any_dev_stores).
template <int In, int Acc, int Out, int UU, int G, bool kDev>
__device__ __forceinline__ void reduce_store_any(const RsagArgs& a, int n, uint64_t v0) {
  constexpr int UE = Unit<In, Out>::UE;
  constexpr int D = Unit<In, Out>::D;
  constexpr int EPW = Unit<In, Out>::EPW;
  float acc[UU][UE];
  bool special[UU];
  uint32_t marks[UU];
#pragma unroll
  for (int u = 0; u < UU; ++u) marks[u] = 0;
  for (int g = 0; g < n; g += G) {
    uint32_t raw[UU][G][D];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
#pragma unroll
      for (int r = 0; r < G; ++r)
        if (g + r < n) ld_words<D>(a.in[g + r], v0 + (uint64_t)u * kRsagThreads, raw[u][r]);
    }
#pragma unroll
    for (int u = 0; u < UU; ++u) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        if (g + r >= n) break;
        float x[UE];
#pragma unroll
        for (int j = 0; j < D; ++j) {
          if constexpr (In == kFP8) {
            decode_word_fp8_hw(raw[u][r][j], x + j * EPW);
            marks[u] |= fp8_e15_marks(raw[u][r][j]);
          } else {
            decode_word<In>(raw[u][r][j], x + j * EPW);
          }
        }
#pragma unroll
        for (int j = 0; j < UE; ++j) {
          const float s = g + r == 0 ? x[j] : acc[u][j] + x[j];
          if constexpr (Acc == kFP8) acc[u][j] = round_fp8_hw(s);
          else acc[u][j] = round_acc<Acc>(s);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    special[u] = (marks[u] & kFp8E15Bits) != 0u;
    if constexpr (In == kFP8) {
      if (special[u]) fp8_unit_exact<D, Acc>(a.in, n, v0 + (uint64_t)u * kRsagThreads, acc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < UU; ++u) {
    const uint64_t v = v0 + (uint64_t)u * kRsagThreads;
    u32x4 o;
    if constexpr (Out == kFP8) o = special[u] ? encode16<kFP8>(acc[u]) : encode16_fp8_hw(acc[u]);
    else o = encode16<Out>(acc[u]);
    if constexpr (G == kAnyGroupWide) {
      // Above 8 ranks, four output pointers per step: their kernel-argument
      // loads are issued together and waited for once, instead of one
      // dependent load per store.  Measured on MI355X, 64 MiB per rank:
      // 12 ranks 295 -> 283 us, 20 ranks 509 -> 489 us.  At 5 to 8 ranks the
      // same batching was 2-3 % slower at some counts, so the narrow-group
      // kernels keep the plain loop.
      int k = 0;
      for (; k + 4 <= n; k += 4) {
        void* const p0 = a.out[k];
        void* const p1 = a.out[k + 1];
        void* const p2 = a.out[k + 2];
        void* const p3 = a.out[k + 3];
        st_out<kDev>(p0, v, o);
        st_out<kDev>(p1, v, o);
        st_out<kDev>(p2, v, o);
        st_out<kDev>(p3, v, o);
      }
      for (; k < n; ++k) st_out<kDev>(a.out[k], v, o);
    } else {
      for (int k = 0; k < n; ++k) st_out<kDev>(a.out[k], v, o);
    }
  }
}

template <int In, int Acc, int Out, int U, int G, bool kDev>
__global__ void __launch_bounds__(kRsagThreads) rsag_any_kernel(const RsagArgs a) {
  const int n = (int)a.nranks;
  for (uint32_t i = blockIdx.x; i < a.launch_tiles; i += gridDim.x) {
    const uint32_t chunk_rel = i / a.tiles_per_chunk;
    const uint32_t tile = i - chunk_rel * a.tiles_per_chunk;
    const uint64_t v_lo = (uint64_t)(a.first_chunk + chunk_rel) * a.chunk_vecs;
    const uint64_t v_hi = v_lo + a.chunk_vecs < a.total_vecs ? v_lo + a.chunk_vecs : a.total_vecs;
    const uint64_t v0 = v_lo + (uint64_t)tile * (kRsagThreads * U) + threadIdx.x;
    if (v0 + (uint64_t)(U - 1) * kRsagThreads < v_hi) {
      reduce_store_any<In, Acc, Out, U, G, kDev>(a, n, v0);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint64_t v = v0 + (uint64_t)u * kRsagThreads;
        if (v < v_hi) reduce_store_any<In, Acc, Out, 1, G, kDev>(a, n, v);
      }
    }
  }
  if (a.tail_count != 0 && blockIdx.x == gridDim.x - 1 && threadIdx.x < a.tail_count)
    reduce_elem<In, Acc, Out>(a.in, a.out, n, a.tail_begin + threadIdx.x);
}

// Element-wise variant for buffers that are not 16-byte aligned.
template <int In, int Acc, int Out>
__global__ void __launch_bounds__(256) rsag_scalar_kernel(const RsagScalarArgs a) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = a.begin + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.end; i += stride)
    reduce_elem<In, Acc, Out>(a.in, a.out, a.nranks, i);
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
#define MRR_RSAG_TRIPLES(X)                                                              \
  X(kF32, kF32, kF32) X(kF16, kF32, kF16) X(kF16, kF16, kF16) X(kBF16, kF32, kBF16)      \
  X(kBF16, kBF16, kBF16) X(kFP8, kF32, kFP8) X(kFP8, kF32, kF16) X(kFP8, kF32, kF32)     \
  X(kFP8, kF16, kFP8) X(kFP8, kF16, kF16) X(kFP8, kF16, kF32) X(kFP8, kFP8, kFP8)        \
  X(kFP8, kFP8, kF16) X(kFP8, kFP8, kF32) X(kFP8FN, kF32, kFP8FN) X(kFP8FN, kF32, kF16)     \
  X(kFP8FN, kF32, kF32) X(kFP8FN, kF16, kFP8FN) X(kFP8FN, kF16, kF16) X(kFP8FN, kF16, kF32) \
  X(kFP8FN, kFP8FN, kFP8FN) X(kFP8FN, kFP8FN, kF16) X(kFP8FN, kFP8FN, kF32)

static bool valid_nranks(int n) { return n == 2 || n == 4 || n == 8 || n == 16 || n == 32; }

bool rsag_compiled_nranks(int n) { return valid_nranks(n); }

bool rsag_types_supported(int tin, int tacc, int tout) {
#define MRR_MATCH(I, A, O) if (tin == I && tacc == A && tout == O) return true;
  MRR_RSAG_TRIPLES(MRR_MATCH)
#undef MRR_MATCH
  return false;
}

bool rsag_supported(int nranks, int tin, int tacc, int tout) {
  return valid_nranks(nranks) && rsag_types_supported(tin, tacc, tout);
}

// Launch shape: one workgroup per tile (at most kMaxGrid; past that each
// workgroup walks several tiles) and a dynamic LDS reservation that lets at
// most `wpc` workgroups share a CU (occupancy_lds_bytes; MRR_RSAG_WPC
// overrides the table).  With MRR_LDS_CAP=0, a persistent grid of wpc
// workgroups per CU and no reservation.
struct RsagShape {
  dim3 grid;
  size_t lds;
};
constexpr uint32_t kMaxGrid = 1u << 24;

static RsagShape rsag_shape(int wpc, uint32_t launch_tiles) {
  const int wpc_env = rsag_wpc_override();
  if (wpc_env > 0) wpc = wpc_env;
  RsagShape sh;
  const bool capped = lds_cap_enabled();
  const uint32_t g_env = max_grid_override();
  uint32_t max_grid = g_env > 0 && g_env < kMaxGrid ? g_env : kMaxGrid;
  if (!capped) {  // persistent grid: wpc workgroups per CU stride over the tiles
    const uint64_t p = (uint64_t)device_cu_count(-1) * (uint64_t)(wpc > 0 ? wpc : 1);
    if (p > 0 && p < max_grid) max_grid = (uint32_t)p;
  }
  const uint32_t blocks = launch_tiles < max_grid ? launch_tiles : max_grid;
  sh.grid = dim3(blocks ? blocks : 1);  // at least one: a tail-only launch
  sh.lds = capped ? occupancy_lds_bytes(wpc) : 0;
  return sh;
}

template <int In, int Acc>
static void launch_wide_typed(int nranks, const RsagShape& sh, const RsagArgs& a, hipStream_t s) {
  switch (nranks) {
#define MRR_CASE(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((rsag_wide_f32_kernel<N, In, Acc>), sh.grid, dim3(kRsagThreads), sh.lds, \
                       s, a);                                                                \
    break;
    MRR_CASE(2) MRR_CASE(4) MRR_CASE(16) MRR_CASE(32)
#undef MRR_CASE
    default: break;
  }
}

template <int In, int Acc, int Out>
static void launch_vec_typed(int nranks, bool large, const RsagShape& sh, const RsagArgs& a,
                             hipStream_t s) {
  switch (nranks) {
#define MRR_CASE(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((rsag_vec_kernel<N, In, Acc, Out, rsag_unroll(N, In, Out),            \
                                        rsag_threads(N, In, Out), false>),                   \
                       sh.grid, dim3(rsag_threads(N, In, Out)), sh.lds, s, a);               \
    break;
    MRR_CASE(4) MRR_CASE(16) MRR_CASE(32)
#undef MRR_CASE
// 2 and 8 ranks: a second instance for large buffers (rsag_large_dev).
#define MRR_CASE_LARGE(N)                                                                    \
  case N:                                                                                    \
    if constexpr (!is_fp8(In)) {                                                             \
      if (large) {                                                                           \
        hipLaunchKernelGGL((rsag_vec_kernel<N, In, Acc, Out, rsag_unroll(N, In, Out),        \
                                            rsag_threads(N, In, Out), true>),                \
                           sh.grid, dim3(rsag_threads(N, In, Out)), sh.lds, s, a);           \
        break;                                                                               \
      }                                                                                      \
    }                                                                                        \
    hipLaunchKernelGGL((rsag_vec_kernel<N, In, Acc, Out, rsag_unroll(N, In, Out),            \
                                        rsag_threads(N, In, Out), false>),                   \
                       sh.grid, dim3(rsag_threads(N, In, Out)), sh.lds, s, a);               \
    break;
    MRR_CASE_LARGE(2) MRR_CASE_LARGE(8)
#undef MRR_CASE_LARGE
    default: break;
  }
}

// The runtime-N kernel loads 16 bytes per lane per rank like the compiled
// ones at N = 8, times a multiplier M of units per lane for 16- and 32-bit
// inputs (MRR_RSAG_ANY_M = 1, 2 or 4; the table uses 1).  Measured on MI355X
// at 64 MiB per rank of bf16, M in {1,2,4} x 4-16 workgroups per CU (one per
// tile, capped as for the compiled kernels): M=1 with 16 per CU for N <= 4
// (3 ranks 0.81 of the HBM peak; the persistent-grid table, M=4 at 12 per
// CU, gave 0.76), 8 per CU for N <= 8 (5, 6, 7 ranks 0.81, 0.80, 0.80,
// against 0.74-0.77 at M=2 and 4 per CU), 4 per CU above (12 x f16 0.78,
// 24 x bf16 0.73).  FP8 inputs keep M=1, at 8 workgroups per CU (6, 12 and
// 24 ranks to E4M3B15 0.72 / 0.74 / 0.72, against 0.72 / 0.74 / 0.70 at 12
// per CU; E4M3FN 0.74 / 0.74 at 6 and 12 ranks).
// MRR_RSAG_ANY_M and MRR_RSAG_WPC override.
constexpr int rsag_any_unroll(int tin, int tout) {
  return is_fp8(tin) ? (tout == kF32 ? 4 : tout == kF16 ? 2 : 1) : 1;
}
static int rsag_any_multiplier(int) { return 1; }
static int rsag_any_wg_per_cu(int n, int tin) {
  if (is_fp8(tin)) return n <= 4 ? 16 : 8;
  return n <= 4 ? 16 : n <= 8 ? 8 : 4;
}
// Output store scope of the runtime-N kernel, measured on MI355X at each
// policy's best cap (two sessions; nt -> device scope): 16-bit data 3 x 64 MiB
// 0.807 -> 0.800 (-2.6 % at the table's x16), 5 ranks a tie, 7 ranks +1.0 %,
// 12 x 64 MiB f16 +1.0 %, 24 x 64 MiB bf16 +0.5 %; FP8 data 3 x 32 MiB -0.9 %
// (E4M3FN -4.9 %), 5 ranks -0.5 %, 6 and 7 ranks +0.9 to +1.2 %.  So device
// scope from 5 ranks of 16- and 32-bit data, plain stores for FP8 data.
// (The FP8 cap at up to 4 ranks: 3 x 32 MiB E4M3B15 0.645 at x8 -> 0.780 at
// x16, E4M3FN 0.659 -> 0.773.)
constexpr int kAnyNtMaxRanks = 4;
static bool rsag_any_dev_stores(int n, int tin) { return !is_fp8(tin) && n > kAnyNtMaxRanks; }
// Groups of 8 ranks, M = mult units per lane.
template <int In, int Acc, int Out, int U, bool kDev>
static void launch_any_g8(int mult, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                          const RsagArgs& a) {
  if (mult == 4)
    hipLaunchKernelGGL((rsag_any_kernel<In, Acc, Out, 4 * U, kAnyGroup, kDev>), grid, block, lds, s, a);
  else if (mult == 2)
    hipLaunchKernelGGL((rsag_any_kernel<In, Acc, Out, 2 * U, kAnyGroup, kDev>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((rsag_any_kernel<In, Acc, Out, U, kAnyGroup, kDev>), grid, block, lds, s, a);
}
template <int In, int Acc, int Out>
static void launch_any_typed(int n, int mult, const RsagShape& sh, const RsagArgs& a,
                             hipStream_t s) {
  const dim3 grid = sh.grid;
  const size_t lds = sh.lds;
  constexpr int U = rsag_any_unroll(In, Out);
  const dim3 block(kRsagThreads);
  // FP8 data or accumulators keep groups of 8 (as the compiled kernels do):
  // their per-rank decode state for 16 ranks no longer stays in registers.
  constexpr bool wide_ok = !is_fp8(In) && !is_fp8(Acc);
  if constexpr (wide_ok) {
    if (n > kAnyGroup && n <= kAnyGroupWideMaxRanks) {
      hipLaunchKernelGGL((rsag_any_kernel<In, Acc, Out, U, kAnyGroupWide, true>), grid, block, lds,
                         s, a);
      return;
    }
  }
  if constexpr (is_fp8(In)) {
    hipLaunchKernelGGL((rsag_any_kernel<In, Acc, Out, U, kAnyGroup, false>), grid, block, lds, s, a);
  } else if (rsag_any_dev_stores(n, In)) {
    launch_any_g8<In, Acc, Out, U, true>(mult, grid, block, lds, s, a);
  } else {
    launch_any_g8<In, Acc, Out, U, false>(mult, grid, block, lds, s, a);
  }
}

// Plans and launches one type triple.  The chunk and unit geometry comes from
// the same compile-time element sizes the kernels index with (Ty, Unit), so
// the host plan and the kernel cannot disagree on how many elements a unit
// or an input vector holds.
// Chunk widths are rounded up to 256 bytes of input, so every chunk after the
// first starts on a cache-line boundary and each wave's 1 KiB loads and
// stores cover whole lines.  With the 16-byte rounding of the plain
// definition, rank counts that do not divide the buffer into line multiples
// (3, 6, 12, 24, ...) put most chunks off the line grid: measured on MI355X,
// 6 x 64 MiB f16 157 -> 138 us, 12 x 64 MiB 342 -> 295 us, 24 x 64 MiB
// 714 -> 608 us; power-of-two counts are unchanged.
constexpr uint64_t kChunkAlignBytes = 256;

// Chunk and tile geometry of a launch: chunks of ceil(count / N) elements
// rounded up to vw, units of ue elements, tiles of tile_units units; every
// chunk (rank < 0) or chunk `rank` only.
static void rsag_geometry(const RsagPlan& p, uint64_t vw, uint64_t ue, uint64_t tile_units,
                          RsagArgs& a) {
  const uint64_t n = (uint64_t)p.nranks;
  const uint64_t per = (p.count + n - 1) / n;
  const uint64_t chunk_elems = (per + vw - 1) / vw * vw;
  a.chunk_vecs = chunk_elems / ue;
  a.total_vecs = p.count / ue;
  a.tail_begin = a.total_vecs * ue;
  const uint32_t tail = (uint32_t)(p.count - a.tail_begin);
  const uint64_t tail_chunk = a.chunk_vecs ? a.total_vecs / a.chunk_vecs : 0;
  a.nranks = (uint32_t)n;
  a.tiles_per_chunk = (uint32_t)((a.chunk_vecs + tile_units - 1) / tile_units);
  if (p.rank < 0) {
    a.first_chunk = 0;
    a.tail_count = tail;
    a.launch_tiles = (uint32_t)n * a.tiles_per_chunk;
  } else {
    a.first_chunk = (uint32_t)p.rank;
    a.tail_count = tail_chunk == (uint64_t)p.rank ? tail : 0;
    a.launch_tiles = a.tiles_per_chunk;
  }
}

template <int In, int Acc, int Out>
static hipError_t launch_rsag_typed(const RsagPlan& p, const void* const* inputs,
                                    void* const* outputs, hipStream_t stream) {
  const int n = p.nranks;
  constexpr uint64_t vw = kChunkAlignBytes / Ty<In>::size;  // chunk granularity, elements
  constexpr uint64_t ue = Unit<In, Out>::UE;  // elements per unit (16-byte output vector)
  static_assert(vw % ue == 0, "a unit must divide the chunk granularity");
  const uint64_t count = p.count;
  // Chunk width: ceil(count / N) rounded up to whole 256-byte input blocks.
  const uint64_t per = (count + n - 1) / n;
  const uint64_t chunk_elems = (per + vw - 1) / vw * vw;

  if (p.vector) {
    RsagArgs a = {};
    for (int r = 0; r < n; ++r) {
      a.in[r] = inputs[r];
      a.out[r] = outputs[r];
    }
    rsag_geometry(p, vw, ue, (uint64_t)rsag_threads(n, In, Out) * rsag_unroll(n, In, Out), a);
    // Small calls: when the table's U would leave fewer than 2 tiles per CU,
    // CUs sit idle; the runtime-N kernel at one unit group per lane spreads
    // the same work over U times more workgroups (measured under HIP-graph
    // replay: 2 x 1 MiB bf16 2.44 -> 2.27 us, 4 x 256 KiB f16 2.39 -> 2.19 us).
    // Only while its ranks fit one load group (N <= 8): at N = 16 the split
    // into two dependent groups costs more than it gains (3.14 -> 3.44 us).
    // MRR_RSAG_SMALL=0 disables.
    const bool small_ok = rsag_small_enabled();
    bool small = false;
    if (valid_nranks(n) && n <= kAnyGroup && small_ok &&
        rsag_unroll(n, In, Out) > rsag_any_unroll(In, Out))
      small = a.launch_tiles < 2 * (uint64_t)(device_cu_count(-1) > 0 ? device_cu_count(-1) : 256);
    const bool any_n = !valid_nranks(n) || small;
    int mult = 1;
    if (any_n && !small && !is_fp8(In) && n <= kAnyGroup) {  // the wide-group kernel runs M = 1
      const int m_env = rsag_any_m_override();
      mult = (m_env == 1 || m_env == 2 || m_env == 4) ? m_env : rsag_any_multiplier(n);
    }
    if (any_n)
      rsag_geometry(p, vw, ue, (uint64_t)kRsagThreads * rsag_any_unroll(In, Out) * mult, a);
    constexpr bool wide_types = is_fp8(In) && Out == kF32;
    if (wide_types && !any_n && rsag_wide_wg_per_cu(n, In) > 0) {  // rsag_wide_f32_kernel
      rsag_geometry(p, vw, kWideUE, kRsagThreads, a);
      if (a.launch_tiles == 0 && a.tail_count == 0) return hipSuccess;
      RsagShape sh = rsag_shape(rsag_wide_wg_per_cu(n, In), a.launch_tiles);
      sh.lds = sh.lds > kWideLds ? sh.lds - kWideLds : 0;  // the kernel's own 4 KiB counts too
      launch_wide_typed<In, Acc>(n, sh, a, stream);
      return hipGetLastError();
    }
    if (a.launch_tiles == 0 && a.tail_count == 0) return hipSuccess;
    const bool large = !any_n && rsag_large_dev(n, In, count * (uint64_t)Ty<In>::size);
    const RsagShape sh = rsag_shape(small   ? 8
                                    : any_n ? rsag_any_wg_per_cu(n, In)
                                    : large ? rsag_large_dev_wg_per_cu(n)
                                            : rsag_wg_per_cu(n, In, Out),
                                    a.launch_tiles);
    if (any_n)
      launch_any_typed<In, Acc, Out>(n, mult, sh, a, stream);
    else
      launch_vec_typed<In, Acc, Out>(n, large, sh, a, stream);
  } else {
    RsagScalarArgs a = {};
    for (int r = 0; r < n; ++r) {
      a.in[r] = inputs[r];
      a.out[r] = outputs[r];
    }
    a.nranks = n;
    if (p.rank < 0) {
      a.begin = 0;
      a.end = count;
    } else {
      a.begin = chunk_elems * (uint64_t)p.rank;
      a.end = a.begin + chunk_elems < count ? a.begin + chunk_elems : count;
      if (a.begin > count) a.begin = count;
    }
    const uint64_t work = a.end - a.begin;
    uint64_t blocks = (work + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((rsag_scalar_kernel<In, Acc, Out>), dim3((uint32_t)blocks), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_rsag(const RsagPlan& p, const void* const* inputs, void* const* outputs,
                       hipStream_t stream) {
#define MRR_DISPATCH(I, A, O) \
  if (p.tin == I && p.tacc == A && p.tout == O) return launch_rsag_typed<I, A, O>(p, inputs, outputs, stream);
  MRR_RSAG_TRIPLES(MRR_DISPATCH)
#undef MRR_DISPATCH
  return hipErrorInvalidValue;  // callers check rsag_types_supported first
}

#define MRR_RSAG_DUAL_PAIRS(X) \
  X(kFP8, kF32) X(kFP8, kF16) X(kFP8, kFP8) X(kFP8FN, kF32) X(kFP8FN, kF16) X(kFP8FN, kFP8FN)

bool rsag_dual_supported(int tin, int tacc) {
#define MRR_MATCH(I, A) if (tin == I && tacc == A) return true;
  MRR_RSAG_DUAL_PAIRS(MRR_MATCH)
#undef MRR_MATCH
  return false;
}

// Dual output: units of 8 elements (one 16-byte f16 vector and 8 FP8 codes
// per lane), with the FP8 -> f16 launch shape.
template <int In, int Acc>
static hipError_t launch_rsag_dual_typed(const RsagPlan& p, const void* const* inputs,
                                         void* const* outputs, void* const* outputs2,
                                         hipStream_t stream) {
  const int n = p.nranks;
  RsagDualArgs d = {};
  for (int r = 0; r < n; ++r) {
    d.base.in[r] = inputs[r];
    d.base.out[r] = outputs[r];
    d.out2[r] = outputs2[r];
  }
  constexpr uint64_t vw = kChunkAlignBytes / Ty<In>::size;
  constexpr uint64_t ue = Unit<In, kF16>::UE;
  rsag_geometry(p, vw, ue, (uint64_t)kRsagThreads * rsag_dual_unroll(n), d.base);
  if (d.base.launch_tiles == 0 && d.base.tail_count == 0) return hipSuccess;
  const RsagShape sh = rsag_shape(rsag_dual_wg_per_cu(n), d.base.launch_tiles);
  const dim3 block(kRsagThreads);
  switch (n) {
#define MRR_CASE(N)                                                                          \
  case N:                                                                                    \
    hipLaunchKernelGGL((rsag_dual_kernel<N, In, Acc, rsag_dual_unroll(N)>), sh.grid, block,    \
                       sh.lds, stream, d);                                                   \
    break;
    MRR_CASE(2) MRR_CASE(4) MRR_CASE(8) MRR_CASE(16) MRR_CASE(32)
#undef MRR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rsag_dual(const RsagPlan& p, const void* const* inputs, void* const* outputs,
                            void* const* outputs2, hipStream_t stream) {
  if (!p.vector || !valid_nranks(p.nranks)) return hipErrorInvalidValue;
#define MRR_DISPATCH(I, A) \
  if (p.tin == I && p.tacc == A) return launch_rsag_dual_typed<I, A>(p, inputs, outputs, outputs2, stream);
  MRR_RSAG_DUAL_PAIRS(MRR_DISPATCH)
#undef MRR_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace mrr
