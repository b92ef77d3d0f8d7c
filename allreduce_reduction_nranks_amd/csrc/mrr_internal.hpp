// mrr_internal.hpp -- kernel argument blocks and launcher entry points shared
// between the C-ABI layer (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mrr.h"

namespace mrr {

constexpr int kMaxRanks = MRR_MAX_RANKS;
constexpr int kFlagSlots = MRR_PKT_FLAG_SLOTS;

// ---- RS/AG ----------------------------------------------------------------
// Passed by value as the kernel argument block (< 4 KiB).
struct RsagArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t chunk_vecs;    // chunk width C in units (16-byte output vectors)
  uint64_t total_vecs;    // whole units in [0, count)
  uint64_t tail_begin;    // first element not covered by a whole unit
  uint32_t tail_count;    // elements in the tail handled by this launch (0..15)
  uint32_t first_chunk;   // first chunk of the launch
  uint32_t tiles_per_chunk;
  uint32_t launch_tiles;  // tiles of all chunks in the launch
  uint32_t nranks;        // rank count (read by the runtime-N kernel)
  uint32_t pad;
};

// RS/AG with a second output set: FP8 inputs reduced once, written as f16 to
// `base.out` and re-encoded to the input's FP8 type in `out2`.
struct RsagDualArgs {
  RsagArgs base;
  void* out2[kMaxRanks];
};

// Element-wise kernel arguments (pointers not 16-byte aligned).
struct RsagScalarArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t begin, end;  // element range
  int nranks;
};

struct RsagPlan {
  int nranks;
  int tin, tacc, tout;  // resolved type ids (no AUTO)
  size_t count;
  int rank;             // -1 = all chunks
  bool vector;          // every pointer 16-byte aligned
};

// True for the rank counts with a compile-time kernel (2, 4, 8, 16, 32); any
// other count in [1, kMaxRanks] runs the runtime-N kernel.
bool rsag_compiled_nranks(int n);
// Type combination check independent of the rank count.
bool rsag_types_supported(int tin, int tacc, int tout);

hipError_t launch_rsag(const RsagPlan& plan, const void* const* inputs, void* const* outputs,
                       hipStream_t stream);

// Dual-output RS/AG (plan.tout is F16, the second outputs take plan.tin):
// FP8 inputs only, compiled rank counts, every pointer 16-byte aligned.
bool rsag_dual_supported(int tin, int tacc);
hipError_t launch_rsag_dual(const RsagPlan& plan, const void* const* inputs, void* const* outputs,
                            void* const* outputs2, hipStream_t stream);
bool rsag_supported(int nranks, int tin, int tacc, int tout);

// ---- LL packets -------------------------------------------------------------
struct PacketArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t* scratch;       // [dst][src][npkt]
  uint32_t* flags;         // [rank][kFlagSlots]
  uint32_t* dev_err;       // may be null
  uint64_t nbytes;         // payload bytes per rank
  uint64_t npkt;           // packets per rank
  uint64_t pkts_per_block; // slice width
  uint32_t nblocks;        // B, blocks per rank
  uint32_t max_spins;      // 0 = unbounded
  uint32_t flag_ranks;     // ranks whose flag slots the call leaves at F (>= N)
};

// Two-phase (reduce-scatter then all-gather) packet allreduce.
struct PacketRsagArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t* scratch;       // rs region [dst][src][cw], then ag region [dst][src][cw]
  uint32_t* flags;         // [rank][kFlagSlots]
  uint32_t* dev_err;       // may be null
  uint64_t nbytes;         // payload bytes per rank
  uint64_t nwords;         // payload words per rank
  uint64_t cw;             // payload words per full chunk
  uint64_t words_per_block;
  uint32_t nblocks;        // B, blocks per rank
  uint32_t max_spins;
};

// Full-mesh allreduce: plain-data inboxes signalled by semaphores.
struct FullmeshArgs {
  const void* in[kMaxRanks];
  void* out[kMaxRanks];
  uint64_t* sem;            // [dst][src][kFlagSlots], flag in the high half
  uint8_t* inbox;           // [dst][src][chunk * elem_size]
  uint32_t* flags;          // [rank][kFlagSlots]
  uint32_t* dev_err;        // may be null
  uint64_t count;           // elements per rank
  uint64_t chunk;           // C, elements per chunk (a multiple of 16 / elem_size)
  uint64_t vec_per_block;   // 16-byte vectors of each chunk per block
  uint32_t nblocks;         // B, blocks per rank
  uint32_t max_spins;       // 0 = unbounded
};

struct PacketReduceArgs {
  const uint64_t* in[kMaxRanks];
  uint64_t* out;
  uint32_t* dev_err;
  uint64_t npkts;
  uint32_t flag_in, flag_out;
  uint32_t max_spins;
};

bool packet_supported(int nranks, int t, int tacc);
// Packets per lane that one poll round of the allpair kernel covers (1 or 2).
int packet_allpair_batch(int nranks, uint64_t npkt);
// Largest workgroup size the allpair kernel is built for.
int packet_max_threads();
// Pointer to the allpair kernel for (nranks, t, tacc, batch), used for occupancy.
const void* packet_allpair_kernel(int nranks, int t, int tacc, int batch);
hipError_t launch_packet_allpair(const PacketArgs& a, int nranks, int t, int tacc, int threads,
                                 int batch, hipStream_t stream);
hipError_t launch_packet_reduce(const PacketReduceArgs& a, int nranks, int t, int tacc,
                                hipStream_t stream);
const void* packet_rsag_kernel(int nranks, int t, int tacc);
hipError_t launch_packet_rsag(const PacketRsagArgs& a, int nranks, int t, int tacc, int threads,
                              hipStream_t stream);
// Full-mesh allreduce (same (type, accumulator) pairs as the packet kernels).
int fullmesh_max_threads();
const void* fullmesh_kernel(int nranks, int t, int tacc);
hipError_t launch_fullmesh(const FullmeshArgs& a, int nranks, int t, int tacc, int threads,
                           hipStream_t stream);
hipError_t launch_pack(const void* src, uint64_t* pkts, size_t nbytes, uint32_t flag,
                       hipStream_t stream);
hipError_t launch_unpack(const uint64_t* pkts, void* dst, size_t nbytes, hipStream_t stream);

// ---- Library-owned packet workspace (mrr_allreduce_packet_noalloc) ---------
// Flag slots of every rank count, then packet scratch.
constexpr size_t kNoAllocFlagBytes = (size_t)kMaxRanks * kFlagSlots * sizeof(uint32_t);
constexpr size_t kNoAllocPacketBytes = MRR_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's workspace; the first call on a
// device clears it on `stream` and must not be under stream capture.
hipError_t noalloc_workspace(hipStream_t stream, uint8_t** base);

// ---- FP8 codec ----------------------------------------------------------------
// dir: 0 fp8->f16, 1 fp8->f32, 2 f16->fp8, 3 f32->fp8
hipError_t launch_codec(int dir, const void* in, void* out, size_t n, bool vector,
                        hipStream_t stream);

// ---- device properties ---------------------------------------------------------
int device_cu_count(int device);
void device_lds_limits(size_t* per_cu, size_t* per_block);
// Dynamic LDS per workgroup that caps residency at `wpc` workgroups per CU.
size_t occupancy_lds_bytes(int wpc);
// Environment overrides (read when the library loads and by mrr_reload_env()).
// MRR_MAX_GRID, 0 when unset.
uint32_t max_grid_override();
// False when MRR_LDS_CAP=0: persistent grids, no LDS reservation.
bool lds_cap_enabled();
// MRR_RSAG_WPC, MRR_RSAG_ANY_M, MRR_CODEC_U, MRR_CODEC_WPC: 0 when unset.
int rsag_wpc_override();
int rsag_any_m_override();
int codec_u_override();
int codec_wpc_override();
// False when MRR_RSAG_SMALL=0.
bool rsag_small_enabled();
// MRR_COOPERATIVE=1: launch_resident() launches cooperatively.
bool cooperative_launch_enabled();
// Launches a kernel whose workgroups wait for each other (one argument block,
// passed by address): cooperatively when MRR_COOPERATIVE=1, else plainly.
hipError_t launch_resident(const void* kernel, dim3 grid, dim3 block, void* args,
                           hipStream_t stream);

}  // namespace mrr
