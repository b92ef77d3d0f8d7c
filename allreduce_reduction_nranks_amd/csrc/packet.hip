// packet.hip -- LL-packet (data + flag) allreduce kernels for gfx950.
//
// Protocol (MSCCL++ commit history for /src, entry fixing the
// allreduce_allpair_packet algorithm; entry on the default flag buffer):
// every rank sends its data as low-latency packets to every peer's scratch
// area, never overwriting the input; the same workgroup sends, waits for its
// peers' packets, reduces and writes back; the launch geometry is validated;
// the flag update must cover every flag slot even when a workgroup has fewer
// threads than slots; one flag buffer can be shared by calls of different
// sizes and algorithms.
//
// A packet is 8 bytes: payload word k (bytes [4k, 4k+4) of the rank's
// buffer, little-endian, zero past the end) in the low half, the call's flag
// in the high half.  64-bit packet loads/stores are single-copy atomic, so a
// reader that sees the flag also sees the payload written with it; they use
// agent scope so the data is coherent across the 8 XCDs (each has its own
// L2).  Readers poll a whole wavefront at a time and leave the loop together
// once every lane's packets carry the flag (__all vote); the poll is bounded
// by max_spins so a missing sender ends in an error word, not a hang.
//
// On one MI355X the N ranks are N groups of workgroups of one launch:
// workgroup g is (rank d = g % N, block b = g / N).  Every workgroup waits
// for its N-1 peers of the same slice, so the host checks that all N * B
// workgroups fit on the GPU at once before launching.
#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

// Payload word k of a byte buffer of nbytes bytes (4-byte aligned).
__device__ __forceinline__ uint32_t load_word(const void* src, uint64_t nbytes, uint64_t k) {
  const uint64_t at = 4 * k;
  if (at + 4 <= nbytes) return reinterpret_cast<const uint32_t*>(src)[k];
  const uint8_t* b = reinterpret_cast<const uint8_t*>(src);
  uint32_t w = 0;
  for (uint64_t i = at; i < nbytes; ++i) w |= (uint32_t)b[i] << (8 * (i - at));
  return w;
}

// Writes the bytes of word k that lie inside [0, nbytes).
__device__ __forceinline__ void store_word(void* dst, uint64_t nbytes, uint64_t k, uint32_t w) {
  const uint64_t at = 4 * k;
  if (at + 4 <= nbytes) {
    reinterpret_cast<uint32_t*>(dst)[k] = w;
    return;
  }
  uint8_t* b = reinterpret_cast<uint8_t*>(dst);
  for (uint64_t i = at; i < nbytes; ++i) b[i] = (uint8_t)(w >> (8 * (i - at)));
}

__device__ __forceinline__ uint64_t make_pkt(uint32_t word, uint32_t flag) {
  return ((uint64_t)flag << 32) | word;
}

// Element j of a payload word of type T, widened to f32.
template <int T> __device__ __forceinline__ float word_elem(uint32_t w, int j) {
  if constexpr (Ty<T>::size == 4) return __uint_as_float(w);
  else if constexpr (Ty<T>::size == 2) return to_f32<T>((w >> (16 * j)) & 0xFFFFu);
  else return to_f32<T>((w >> (8 * j)) & 0xFFu);
}

template <int T> __device__ __forceinline__ uint32_t elem_bits(float v) { return from_f32<T>(v); }

// Reduces one payload word over N ranks in rank order; rank `self` (if < N)
// contributes `own` instead of w[self].
template <int N, int T, int Acc>
__device__ __forceinline__ uint32_t reduce_word(const uint32_t* w, uint32_t self, uint32_t own) {
  constexpr int E = 4 / Ty<T>::size;
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    float acc = round_acc<Acc>(word_elem<T>(self == 0u ? own : w[0], j));
#pragma unroll
    for (int s = 1; s < N; ++s)
      acc = round_acc<Acc>(acc + word_elem<T>((uint32_t)s == self ? own : w[s], j));
    out |= elem_bits<T>(acc) << (32 / E * j);
  }
  return out;
}

__device__ __forceinline__ void report_timeout(uint32_t* dev_err) {
  if (dev_err) atomicCAS(dev_err, 0u, (uint32_t)MRR_ETIMEDOUT);
}

// Packets per lane handled in one poll round (all P x N loads in flight
// together).  The receive-only and two-phase kernels take one.  The allpair
// kernel takes one, or two for calls of at least kPktBatch2Min packets per
// rank at N <= 8: measured on MI355X, 8 ranks of f16, per call under graph
// replay, two per lane cost 16 KiB 5.7 -> 9.0 us and 64 KiB 8.7 -> 10.7 us
// (half as many workgroups share the polling), gained 256 KiB 27.2 ->
// 20.9 us (one per lane needs more workgroups than fit, so lanes poll twice
// in sequence) and tied at 1 MiB; four per lane lost at every size.
constexpr int pkt_batch(int) { return 1; }
constexpr uint64_t kPktBatch2Min = 32768;
int packet_allpair_batch(int nranks, uint64_t npkt) {
  return nranks <= 8 && npkt >= kPktBatch2Min ? 2 : 1;
}
// Largest workgroup of the allpair kernel (bounds its registers at 256).
constexpr int kPktMaxThreads = 512;
int packet_max_threads() { return kPktMaxThreads; }

template <int N>
__device__ __forceinline__ uint32_t peer_mask(uint32_t self) {
  const uint32_t all = N == 32 ? 0xFFFFFFFFu : ((1u << N) - 1u);
  return self < (uint32_t)N ? all & ~(1u << self) : all;
}

// Source s of packet k lives at addr(s) + k.
struct StridedSources {  // one scratch, sources `stride` packets apart
  const uint64_t* base;
  uint64_t stride;
  __device__ __forceinline__ const uint64_t* operator()(int s) const { return base + (uint64_t)s * stride; }
};
struct ListedSources {  // one pointer per source
  const uint64_t* const* ptr;
  __device__ __forceinline__ const uint64_t* operator()(int s) const { return ptr[s]; }
};

// Waits until every pending packet (bit s of pending[p]: source s of packet
// p) carries `flag`, filling w[p][s] with the payloads.  Each round loads
// packet kq[p] of all N sources before any flag is looked at, then waits once:
// a round costs one memory round trip, not one per source.  (Loading each
// source under the lane's pending bit made the compiler wait after every
// load: N round trips per round.)  kq[p] is the lane's packet index, or any
// in-bounds index for a lane with nothing pending; the self slot of an inbox
// exists and is loaded like the others.  Wavefront-uniform: all lanes leave
// together.  Returns false after max_spins rounds (0 = none).
template <int N, int P, typename Src>
__device__ __forceinline__ bool poll_batch(const Src& src, const uint64_t* kq, uint32_t* pending,
                                           uint32_t (*w)[N], uint32_t flag, uint32_t max_spins) {
  uint32_t spins = 0;
  while (true) {
    uint64_t pk[P][N];
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int s = 0; s < N; ++s) pk[p][s] = ld_pkt(src(s) + kq[p]);
    }
    uint32_t left = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
#pragma unroll
      for (int s = 0; s < N; ++s) {
        const bool want = (pending[p] >> s) & 1u;
        w[p][s] = want ? (uint32_t)pk[p][s] : w[p][s];
        if (want && (uint32_t)(pk[p][s] >> 32) == flag) pending[p] &= ~(1u << s);
      }
      left |= pending[p];
    }
    if (__all(left == 0u)) return true;
    if (max_spins != 0u && ++spins >= max_spins) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

template <int N, int T, int Acc, int P>
__global__ void __launch_bounds__(kPktMaxThreads) packet_allpair_k(const PacketArgs a) {
  const uint32_t d = blockIdx.x % N;
  const uint32_t b = blockIdx.x / N;
  uint32_t* const my_flags = a.flags + (uint64_t)d * kFlagSlots;
  uint32_t F = my_flags[b] + 1u;
  if (F == 0u) F = 1u;

  const uint64_t k_lo = (uint64_t)b * a.pkts_per_block;
  const uint64_t k_hi = k_lo + a.pkts_per_block < a.npkt ? k_lo + a.pkts_per_block : a.npkt;
  const void* src = a.in[d];

  // Send: slice b of rank d's input, packed once, stored to every peer.
  for (uint64_t k = k_lo + threadIdx.x; k < k_hi; k += blockDim.x) {
    const uint64_t pkt = make_pkt(load_word(src, a.nbytes, k), F);
#pragma unroll
    for (int p = 0; p < N; ++p)
      if ((uint32_t)p != d) st_pkt(a.scratch + ((uint64_t)p * N + d) * a.npkt + k, pkt);
  }

  // Receive, reduce and write back, in wavefront-uniform batches of P
  // packets per lane.
  const StridedSources inbox{a.scratch + (uint64_t)d * N * a.npkt, a.npkt};
  const uint64_t step = (uint64_t)blockDim.x * P;
  for (uint64_t kb = k_lo; kb < k_hi; kb += step) {
    uint64_t kp[P], kq[P];
    uint32_t pending[P];
    uint32_t w[P][N];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      kp[p] = kb + (uint64_t)p * blockDim.x + threadIdx.x;
      pending[p] = kp[p] < k_hi ? peer_mask<N>(d) : 0u;
      kq[p] = kp[p] < k_hi ? kp[p] : k_hi - 1;
    }
    if (!poll_batch<N, P>(inbox, kq, pending, w, F, a.max_spins)) {
      report_timeout(a.dev_err);
      break;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (kp[p] < k_hi) {
        const uint32_t own = load_word(src, a.nbytes, kp[p]);
        store_word(a.out[d], a.nbytes, kp[p], reduce_word<N, T, Acc>(w[p], d, own));
      }
    }
  }

  // Flag update: every slot j of rank d with j % B == b, by a thread loop so
  // that a workgroup with fewer threads than slots still covers them all.
  // A flag area shared by calls of several rank counts (flag_ranks > N) has
  // the slots of ranks d + N, d + 2N, ... set too, so every slot any later
  // call reads holds F; no workgroup of this launch reads those.
  __syncthreads();
  for (uint32_t r = d; r < a.flag_ranks; r += N) {
    uint32_t* const fl = a.flags + (uint64_t)r * kFlagSlots;
    for (uint32_t j = b + threadIdx.x * a.nblocks; j < (uint32_t)kFlagSlots;
         j += blockDim.x * a.nblocks)
      fl[j] = F;
  }
}

// Two-phase packet allreduce, workgroup (rank d, block b), slice b of every
// chunk (chunk c = payload words [c * cw, min((c + 1) * cw, nwords))):
//   1. reduce-scatter send: for every peer c, chunk c of rank d's input goes
//      as packets to rs[c][d] (rank c's inbox for its chunk);
//   2. reduce: poll rs[d][s] for every s != d, sum in rank order with rank
//      d's own chunk d read from its input, write the result to output d and
//      send it as packets to ag[p][d] for every peer p (all-gather send);
//   3. all-gather receive: poll ag[d][s] for every s != d and write chunk s
//      of output d.
// Each lane handles the same slice word k in all three steps, so an input
// word is read before the lane writes the output word at the same address
// (in place works).  Phase 2 depends only on phase-1 packets, phase 3 only on
// phase-2 packets, so with all N * B workgroups resident no wait is circular.
template <int N, int T, int Acc>
__global__ void __launch_bounds__(kPktMaxThreads) packet_rsag_k(const PacketRsagArgs a) {
  const uint32_t d = blockIdx.x % N;
  const uint32_t b = blockIdx.x / N;
  uint32_t* const my_flags = a.flags + (uint64_t)d * kFlagSlots;
  uint32_t F = my_flags[b] + 1u;
  if (F == 0u) F = 1u;

  const uint64_t cw = a.cw;
  const uint64_t k_lo = (uint64_t)b * a.words_per_block;
  const uint64_t k_hi = k_lo + a.words_per_block < cw ? k_lo + a.words_per_block : cw;
  uint64_t* const rs = a.scratch;
  uint64_t* const ag = a.scratch + (uint64_t)N * N * cw;
  const void* src = a.in[d];
  void* dst = a.out[d];

  // 1. reduce-scatter send
  for (uint64_t k = k_lo + threadIdx.x; k < k_hi; k += blockDim.x) {
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const uint64_t w = (uint64_t)c * cw + k;
      if ((uint32_t)c != d && w < a.nwords)
        st_pkt(rs + ((uint64_t)c * N + d) * cw + k, make_pkt(load_word(src, a.nbytes, w), F));
    }
  }

  // 2. reduce chunk d and send it to every peer
  const uint64_t wd0 = (uint64_t)d * cw;
  bool ok = true;
  for (uint64_t kb = k_lo; kb < k_hi && ok; kb += blockDim.x) {
    uint64_t kp[1] = {kb + threadIdx.x};
    const uint64_t kq[1] = {kp[0] < k_hi ? kp[0] : k_hi - 1};
    const bool active = kp[0] < k_hi && wd0 + kp[0] < a.nwords;
    uint32_t pending[1] = {active ? peer_mask<N>(d) : 0u};
    uint32_t w[1][N];
    ok = poll_batch<N, 1>(StridedSources{rs + (uint64_t)d * N * cw, cw}, kq, pending, w, F,
                          a.max_spins);
    if (!ok) {
      report_timeout(a.dev_err);
      break;
    }
    if (active) {
      const uint64_t wd = wd0 + kp[0];
      const uint32_t r = reduce_word<N, T, Acc>(w[0], d, load_word(src, a.nbytes, wd));
      store_word(dst, a.nbytes, wd, r);
      const uint64_t pkt = make_pkt(r, F);
#pragma unroll
      for (int p = 0; p < N; ++p)
        if ((uint32_t)p != d) st_pkt(ag + ((uint64_t)p * N + d) * cw + kp[0], pkt);
    }
  }

  // 3. all-gather receive
  for (uint64_t kb = k_lo; kb < k_hi && ok; kb += blockDim.x) {
    uint64_t kp[1] = {kb + threadIdx.x};
    const uint64_t kq[1] = {kp[0] < k_hi ? kp[0] : k_hi - 1};
    uint32_t pending[1] = {0u};
    if (kp[0] < k_hi) {
#pragma unroll
      for (int s = 0; s < N; ++s)
        if ((uint32_t)s != d && (uint64_t)s * cw + kp[0] < a.nwords) pending[0] |= 1u << s;
    }
    const uint32_t want = pending[0];
    uint32_t w[1][N];
    ok = poll_batch<N, 1>(StridedSources{ag + (uint64_t)d * N * cw, cw}, kq, pending, w, F,
                          a.max_spins);
    if (!ok) {
      report_timeout(a.dev_err);
      break;
    }
#pragma unroll
    for (int s = 0; s < N; ++s)
      if (want & (1u << s)) store_word(dst, a.nbytes, (uint64_t)s * cw + kp[0], w[0][s]);
  }

  __syncthreads();
  for (uint32_t j = b + threadIdx.x * a.nblocks; j < (uint32_t)kFlagSlots;
       j += blockDim.x * a.nblocks)
    my_flags[j] = F;
}

// Receive step alone: packets from N producers outside the launch.
template <int N, int T, int Acc>
__global__ void __launch_bounds__(256) packet_reduce_k(const PacketReduceArgs a) {
  constexpr int P = pkt_batch(N);
  const uint64_t step = (uint64_t)gridDim.x * blockDim.x * P;
  for (uint64_t kb = (uint64_t)blockIdx.x * blockDim.x * P; kb < a.npkts; kb += step) {
    uint64_t kp[P], kq[P];
    uint32_t pending[P];
    uint32_t w[P][N];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      kp[p] = kb + (uint64_t)p * blockDim.x + threadIdx.x;
      pending[p] = kp[p] < a.npkts ? peer_mask<N>((uint32_t)N) : 0u;
      kq[p] = kp[p] < a.npkts ? kp[p] : a.npkts - 1;
    }
    if (!poll_batch<N, P>(ListedSources{a.in}, kq, pending, w, a.flag_in, a.max_spins)) {
      report_timeout(a.dev_err);
      break;
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (kp[p] < a.npkts)
        st_pkt(a.out + kp[p], make_pkt(reduce_word<N, T, Acc>(w[p], (uint32_t)N, 0u), a.flag_out));
  }
}

__global__ void __launch_bounds__(256) pack_k(const void* src, uint64_t* pkts, uint64_t nbytes,
                                              uint32_t flag) {
  const uint64_t npkt = (nbytes + 3) / 4;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < npkt; k += stride)
    st_pkt(pkts + k, make_pkt(load_word(src, nbytes, k), flag));
}

__global__ void __launch_bounds__(256) unpack_k(const uint64_t* pkts, void* dst, uint64_t nbytes) {
  const uint64_t npkt = (nbytes + 3) / 4;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t k = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; k < npkt; k += stride)
    store_word(dst, nbytes, k, (uint32_t)pkts[k]);
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
// (type, accumulator) pairs; the output type is the input type.
#define MRR_PKT_PAIRS(X)                                                                  \
  X(kF32, kF32) X(kF16, kF32) X(kF16, kF16) X(kBF16, kF32) X(kBF16, kBF16) X(kFP8, kF32) \
  X(kFP8, kF16) X(kFP8, kFP8) X(kFP8FN, kF32) X(kFP8FN, kF16) X(kFP8FN, kFP8FN)

#define MRR_PKT_RANKS(X, T, A) X(2, T, A) X(4, T, A) X(8, T, A) X(16, T, A) X(32, T, A)

bool packet_supported(int nranks, int t, int tacc) {
  if (!(nranks == 2 || nranks == 4 || nranks == 8 || nranks == 16 || nranks == 32)) return false;
#define MRR_MATCH(T, A) if (t == T && tacc == A) return true;
  MRR_PKT_PAIRS(MRR_MATCH)
#undef MRR_MATCH
  return false;
}

// Rank counts with a two-packets-per-lane allpair kernel (packet_allpair_batch).
#define MRR_PKT_RANKS_P2(X, T, A) X(2, T, A) X(4, T, A) X(8, T, A)

const void* packet_allpair_kernel(int nranks, int t, int tacc, int batch) {
#define MRR_K(N, T, A) \
  if (nranks == N && t == T && tacc == A) return (const void*)&packet_allpair_k<N, T, A, 1>;
#define MRR_K2(N, T, A) \
  if (nranks == N && t == T && tacc == A) return (const void*)&packet_allpair_k<N, T, A, 2>;
#define MRR_ALLN(T, A) MRR_PKT_RANKS(MRR_K, T, A)
#define MRR_ALLN2(T, A) MRR_PKT_RANKS_P2(MRR_K2, T, A)
  if (batch == 2) {
    MRR_PKT_PAIRS(MRR_ALLN2)
    return nullptr;
  }
  MRR_PKT_PAIRS(MRR_ALLN)
#undef MRR_ALLN2
#undef MRR_ALLN
#undef MRR_K2
#undef MRR_K
  return nullptr;
}

hipError_t launch_packet_allpair(const PacketArgs& a, int nranks, int t, int tacc, int threads,
                                 int batch, hipStream_t stream) {
  const dim3 grid((uint32_t)nranks * a.nblocks), block((uint32_t)threads);
#define MRR_K(N, T, A)                                                               \
  if (nranks == N && t == T && tacc == A) {                                          \
    return launch_resident((const void*)&packet_allpair_k<N, T, A, 1>, grid, block,   \
    (void*)&a, stream);                                                        \
  }
#define MRR_K2(N, T, A)                                                              \
  if (nranks == N && t == T && tacc == A) {                                          \
    return launch_resident((const void*)&packet_allpair_k<N, T, A, 2>, grid, block,   \
    (void*)&a, stream);                                                        \
  }
#define MRR_ALLN(T, A) MRR_PKT_RANKS(MRR_K, T, A)
#define MRR_ALLN2(T, A) MRR_PKT_RANKS_P2(MRR_K2, T, A)
  if (batch == 2) {
    MRR_PKT_PAIRS(MRR_ALLN2)
    return hipErrorInvalidValue;
  }
  MRR_PKT_PAIRS(MRR_ALLN)
#undef MRR_ALLN2
#undef MRR_ALLN
#undef MRR_K2
#undef MRR_K
  return hipErrorInvalidValue;
}


hipError_t launch_packet_reduce(const PacketReduceArgs& a, int nranks, int t, int tacc,
                                hipStream_t stream) {
  const uint64_t per_block = 256ull * pkt_batch(nranks);
  uint64_t blocks = (a.npkts + per_block - 1) / per_block;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid((uint32_t)blocks), block(256);
#define MRR_K(N, T, A)                                                               \
  if (nranks == N && t == T && tacc == A) {                                          \
    hipLaunchKernelGGL((packet_reduce_k<N, T, A>), grid, block, 0, stream, a);       \
    return hipGetLastError();                                                        \
  }
#define MRR_ALLN(T, A) MRR_PKT_RANKS(MRR_K, T, A)
  MRR_PKT_PAIRS(MRR_ALLN)
#undef MRR_ALLN
#undef MRR_K
  return hipErrorInvalidValue;
}

const void* packet_rsag_kernel(int nranks, int t, int tacc) {
#define MRR_K(N, T, A) \
  if (nranks == N && t == T && tacc == A) return (const void*)&packet_rsag_k<N, T, A>;
#define MRR_ALLN(T, A) MRR_PKT_RANKS(MRR_K, T, A)
  MRR_PKT_PAIRS(MRR_ALLN)
#undef MRR_ALLN
#undef MRR_K
  return nullptr;
}

hipError_t launch_packet_rsag(const PacketRsagArgs& a, int nranks, int t, int tacc, int threads,
                              hipStream_t stream) {
  const dim3 grid((uint32_t)nranks * a.nblocks), block((uint32_t)threads);
#define MRR_K(N, T, A)                                                               \
  if (nranks == N && t == T && tacc == A) {                                          \
    return launch_resident((const void*)&packet_rsag_k<N, T, A>, grid, block,         \
    (void*)&a, stream);                                                        \
  }
#define MRR_ALLN(T, A) MRR_PKT_RANKS(MRR_K, T, A)
  MRR_PKT_PAIRS(MRR_ALLN)
#undef MRR_ALLN
#undef MRR_K
  return hipErrorInvalidValue;
}

hipError_t launch_pack(const void* src, uint64_t* pkts, size_t nbytes, uint32_t flag,
                       hipStream_t stream) {
  uint64_t blocks = ((nbytes + 3) / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(pack_k, dim3((uint32_t)blocks), dim3(256), 0, stream, src, pkts,
                     (uint64_t)nbytes, flag);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint64_t* pkts, void* dst, size_t nbytes, hipStream_t stream) {
  uint64_t blocks = ((nbytes + 3) / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(unpack_k, dim3((uint32_t)blocks), dim3(256), 0, stream, pkts, dst,
                     (uint64_t)nbytes);
  return hipGetLastError();
}

}  // namespace mrr
