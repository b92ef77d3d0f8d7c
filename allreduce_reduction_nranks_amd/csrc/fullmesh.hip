// fullmesh.hip -- full-mesh allreduce over plain data and semaphores, gfx950.
//
// The MSCCL++ commit history names a "fullmesh" allreduce beside the allpair
// packet one (entries adding accumDtype, and ROCm FP8 E4M3B15 support, which
// extends both kernels with wider accumulation).  The pages give no steps, so
// the kernel follows the plain reading of the name: every rank exchanges data
// directly with every peer, by writes only (a rank never reads another rank's
// memory), moving plain 16-byte vectors instead of LL packets and signalling
// each delivery with a flag written after the data:
//   1. rank d writes chunk c of its input into rank c's inbox [c][d] of the
//      scratch, for every peer c != d (the reduce-scatter push);
//   2. per block b it then sets semaphore [c][d][b] to the call's flag F,
//      with release ordering at agent scope, so a reader that sees F also
//      sees the data;
//   3. rank c waits (acquire, bounded by max_spins) until the semaphores
//      [c][s][b] of every peer s carry F, sums chunk c in rank order 0..N-1 --
//      its own contribution straight from its input, the others from its
//      inbox -- and writes the sum into chunk c of every rank's output (the
//      all-gather push);
//   4. flag slots are updated as in the packet kernels, so one flag buffer
//      serves both algorithms.
// A semaphore is a 64-bit word with the flag in its high half (a packet with
// no payload): a scratch area that packet calls used before holds packets
// whose high halves are older flags, never F.
//
// Chunks are those of the two-phase packet allreduce: C = roundup(ceil(count
// / N), 16 / e) elements.  Workgroup (rank d = g % N, block b = g / N) handles
// vectors [b * vpb, (b + 1) * vpb) of every chunk: it pushes that slice of
// each peer's chunk, then reduces that slice of its own.  Every workgroup
// waits for its N - 1 peers of the same slice, so all N * B workgroups must be
// resident at once (checked on the host).
//
// In place (outputs[k] == inputs[k]) works: the only reader of inputs[k]
// chunk c slice b other than workgroup (c, b) is workgroup (k, b), which
// reads it before it signals (c, b), and (c, b) writes outputs[k] chunk c
// slice b only after that signal; (c, b) reads its own contribution before it
// overwrites it, lane by lane.
#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

constexpr int kFmMaxThreads = 512;

__device__ __forceinline__ void fm_report_timeout(uint32_t* dev_err) {
  if (dev_err) atomicCAS(dev_err, 0u, (uint32_t)MRR_ETIMEDOUT);
}

// Elements of chunk c below count (0 for an empty trailing chunk).
__device__ __forceinline__ uint64_t chunk_elems(uint64_t count, uint64_t chunk, uint32_t c) {
  const uint64_t lo = (uint64_t)c * chunk;
  if (lo >= count) return 0;
  return count - lo < chunk ? count - lo : chunk;
}

template <int T>
__device__ __forceinline__ void copy_elems(const void* src, uint64_t si, void* dst, uint64_t di,
                                           uint64_t n) {
  const uint8_t* s = reinterpret_cast<const uint8_t*>(src) + si * Ty<T>::size;
  uint8_t* d = reinterpret_cast<uint8_t*>(dst) + di * Ty<T>::size;
  for (uint64_t i = 0; i < n * Ty<T>::size; ++i) d[i] = s[i];
}

// The 16-byte vector `v` of a buffer, widened to f32 (all 16 / e elements).
template <int T> __device__ __forceinline__ void load_vec(const void* base, uint64_t v, float* x) {
  const u32x4 w = reinterpret_cast<const u32x4*>(base)[v];
  constexpr int EPW = 4 / Ty<T>::size;
#pragma unroll
  for (int j = 0; j < 4; ++j) decode_word<T>(w[j], x + j * EPW);
}

template <int N, int T, int Acc>
__global__ void __launch_bounds__(kFmMaxThreads) fullmesh_k(const FullmeshArgs a) {
  constexpr int V = 16 / Ty<T>::size;  // elements per vector
  const uint32_t d = blockIdx.x % N;
  const uint32_t b = blockIdx.x / N;
  uint32_t* const my_flags = a.flags + (uint64_t)d * kFlagSlots;
  uint32_t F = my_flags[b] + 1u;
  if (F == 0u) F = 1u;

  const uint64_t chunk = a.chunk;
  const uint64_t cvec = chunk / V;
  const uint64_t v_lo = (uint64_t)b * a.vec_per_block;
  const uint64_t v_hi = v_lo + a.vec_per_block < cvec ? v_lo + a.vec_per_block : cvec;
  const uint64_t slot_bytes = chunk * Ty<T>::size;

  // The buffer's one partial vector (count % V elements, if any) lies at
  // vector pv of chunk pc; it is moved element by element, apart from the
  // whole vectors, by the lane of the workgroup whose slice holds it.
  const uint64_t tail_first = a.count / V * V;
  const bool has_tail = tail_first < a.count;
  const uint32_t pc = (uint32_t)(tail_first / chunk);
  const uint64_t pv = (tail_first - (uint64_t)pc * chunk) / V;
  const bool tail_lane = has_tail && pv >= v_lo && pv < v_hi &&
                         (pv - v_lo) % blockDim.x == threadIdx.x;

  // 1. push slice b of chunk c of rank d's input into inbox [c][d], peers
  // in groups of up to 8: a lane loads its vector of every chunk of a group
  // before it stores any, one memory round trip per group instead of one per
  // peer (the compiler cannot hoist a load above a store that may alias it).
  // Every lane issues all loads of a group unconditionally (a lane with
  // nothing to send for chunk c reads vector 0 of the input instead, which
  // exists whenever a whole vector does), so no load waits on a branch.
  constexpr int GP = N < 8 ? N : 8;
  if (a.count >= (uint64_t)V) {
    for (uint64_t v = v_lo + threadIdx.x; v < v_hi; v += blockDim.x) {
      const uint64_t first = v * V;
#pragma unroll 1
      for (int c0 = 0; c0 < N; c0 += GP) {
        u32x4 buf[GP];
        bool send[GP];
#pragma unroll
        for (int j = 0; j < GP; ++j) {
          const uint32_t c = (uint32_t)(c0 + j);
          send[j] = c != d && first + V <= chunk_elems(a.count, chunk, c);
          buf[j] = reinterpret_cast<const u32x4*>(a.in[d])[send[j] ? (uint64_t)c * cvec + v : 0];
        }
#pragma unroll
        for (int j = 0; j < GP; ++j) {
          uint8_t* const slot = a.inbox + ((uint64_t)(c0 + j) * N + d) * slot_bytes;
          if (send[j]) reinterpret_cast<u32x4*>(slot)[v] = buf[j];
        }
      }
    }
  }
  if (tail_lane && pc != d)
    copy_elems<T>(a.in[d], tail_first, a.inbox + ((uint64_t)pc * N + d) * slot_bytes, pv * V,
                  a.count - tail_first);
  // 2. signal: once every wave has passed the barrier, lane c stores
  // semaphore [c][d][b] with agent-scope release.  The barrier orders every
  // wave's inbox stores before that store, and a release is cumulative, so
  // one release per semaphore covers the whole workgroup's data.  (An
  // agent-scope release writes back the XCD's L2 and an acquire invalidates
  // it; measured on MI355X, an extra release fence in every wave and an
  // acquire in every wave after the wait cost 8 x 1 MiB f16 29 -> 54 us.)
  __syncthreads();
  if (threadIdx.x < (uint32_t)N && threadIdx.x != d)
    __hip_atomic_store(a.sem + ((uint64_t)threadIdx.x * N + d) * kFlagSlots + b,
                       (uint64_t)F << 32, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

  // 3. wait for every peer's slice b: wave 0 polls, one lane per peer, and
  // acquires; the barrier after it orders the other waves' inbox loads after
  // that acquire.
  __shared__ int s_ok;
  if (threadIdx.x < 64) {
    const bool mine = threadIdx.x < (uint32_t)N && threadIdx.x != d;
    const uint64_t* const p = a.sem + ((uint64_t)d * N + threadIdx.x) * kFlagSlots + b;
    uint32_t spins = 0;
    bool ok = true;
    while (true) {
      const bool done = !mine || (uint32_t)(ld_pkt(p) >> 32) == F;
      if (__all(done)) break;
      if (a.max_spins != 0u && ++spins >= a.max_spins) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (threadIdx.x == 0) s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  if (s_ok) {
    // reduce slice b of chunk d in rank order and push it to every output
    const uint64_t nd = chunk_elems(a.count, chunk, d);
    const uint8_t* const box = a.inbox + (uint64_t)d * N * slot_bytes;
    for (uint64_t v = v_lo + threadIdx.x; v < v_hi; v += blockDim.x) {
      if (v * V + V > nd) break;
      float acc[V];
#pragma unroll
      for (int s = 0; s < N; ++s) {
        float x[V];
        if ((uint32_t)s == d) load_vec<T>(a.in[d], (uint64_t)d * cvec + v, x);
        else load_vec<T>(box + (uint64_t)s * slot_bytes, v, x);
#pragma unroll
        for (int j = 0; j < V; ++j) acc[j] = round_acc<Acc>(s == 0 ? x[j] : acc[j] + x[j]);
      }
      const u32x4 o = encode16<T>(acc);
#pragma unroll
      for (int k = 0; k < N; ++k) reinterpret_cast<u32x4*>(a.out[k])[(uint64_t)d * cvec + v] = o;
    }
    if (tail_lane && pc == d) {  // the partial vector, element by element
      for (uint64_t i = tail_first; i < a.count; ++i) {
        const uint64_t j = i - (uint64_t)d * chunk;
        float acc = 0.0f;
#pragma unroll
        for (int s = 0; s < N; ++s) {
          const float x = (uint32_t)s == d ? load_elem<T>(a.in[d], i)
                                           : load_elem<T>(box + (uint64_t)s * slot_bytes, j);
          acc = round_acc<Acc>(s == 0 ? x : acc + x);
        }
#pragma unroll
        for (int k = 0; k < N; ++k) store_elem<T>(a.out[k], i, acc);
      }
    }
  } else if (threadIdx.x == 0) {
    fm_report_timeout(a.dev_err);
  }

  // 4. flag slots j of rank d with j % B == b
  __syncthreads();
  for (uint32_t j = b + threadIdx.x * a.nblocks; j < (uint32_t)kFlagSlots;
       j += blockDim.x * a.nblocks)
    my_flags[j] = F;
}

// ---------------------------------------------------------------------------
// Host-side dispatch: the packet kernels' (type, accumulator) pairs.
// ---------------------------------------------------------------------------
#define MRR_FM_PAIRS(X)                                                                   \
  X(kF32, kF32) X(kF16, kF32) X(kF16, kF16) X(kBF16, kF32) X(kBF16, kBF16) X(kFP8, kF32) \
  X(kFP8, kF16) X(kFP8, kFP8) X(kFP8FN, kF32) X(kFP8FN, kF16) X(kFP8FN, kFP8FN)
#define MRR_FM_RANKS(X, T, A) X(2, T, A) X(4, T, A) X(8, T, A) X(16, T, A) X(32, T, A)

int fullmesh_max_threads() { return kFmMaxThreads; }

const void* fullmesh_kernel(int nranks, int t, int tacc) {
#define MRR_K(N, T, A) \
  if (nranks == N && t == T && tacc == A) return (const void*)&fullmesh_k<N, T, A>;
#define MRR_ALLN(T, A) MRR_FM_RANKS(MRR_K, T, A)
  MRR_FM_PAIRS(MRR_ALLN)
#undef MRR_ALLN
#undef MRR_K
  return nullptr;
}

hipError_t launch_fullmesh(const FullmeshArgs& a, int nranks, int t, int tacc, int threads,
                           hipStream_t stream) {
  const dim3 grid((uint32_t)nranks * a.nblocks), block((uint32_t)threads);
#define MRR_K(N, T, A)                                                          \
  if (nranks == N && t == T && tacc == A) {                                     \
    return launch_resident((const void*)&fullmesh_k<N, T, A>, grid, block,       \
    (void*)&a, stream);                                                   \
  }
#define MRR_ALLN(T, A) MRR_FM_RANKS(MRR_K, T, A)
  MRR_FM_PAIRS(MRR_ALLN)
#undef MRR_ALLN
#undef MRR_K
  return hipErrorInvalidValue;
}

}  // namespace mrr
