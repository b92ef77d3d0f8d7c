// api.hip -- the libmrr C ABI: argument validation, type resolution and
// dispatch to the kernel launchers.  Every check that needs no device runs
// before any HIP call, so a refused call never touches the GPU.
#include <atomic>
#include <mutex>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mrr_device.hpp"
#include "mrr_internal.hpp"

namespace mrr {

// ---------------------------------------------------------------------------
// Environment overrides: read once when the library is loaded, and again by
// mrr_reload_env().  Kept in atomics so a reload racing with calls on other
// threads is well defined (each call sees the old or the new value).
// ---------------------------------------------------------------------------
namespace {
struct EnvOverrides {
  std::atomic<int> log{0};          // MRR_LOG=1: one stderr line per refused call
  std::atomic<uint32_t> max_grid{0};  // MRR_MAX_GRID=<g>, 0 = unset
  std::atomic<int> lds_cap{1};      // MRR_LDS_CAP=0 turns the LDS reservation off
  std::atomic<int> rsag_wpc{0};     // MRR_RSAG_WPC=<w>, 0 = the launch table
  std::atomic<int> rsag_any_m{0};   // MRR_RSAG_ANY_M=1|2|4, 0 = the launch table
  std::atomic<int> rsag_small{1};   // MRR_RSAG_SMALL=0 turns the small-call route off
  std::atomic<int> codec_u{0};      // MRR_CODEC_U=<u>, 0 = the launch table
  std::atomic<int> codec_wpc{0};    // MRR_CODEC_WPC=<w>, 0 = the launch table
  std::atomic<int> cooperative{0};  // MRR_COOPERATIVE=1: cross-workgroup kernels launch cooperatively
};
EnvOverrides g_env;

int env_atoi(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

void read_env() {
  const char* lg = getenv("MRR_LOG");
  g_env.log.store(lg && lg[0] && lg[0] != '0', std::memory_order_relaxed);
  const char* mg = getenv("MRR_MAX_GRID");
  const long g = mg ? atol(mg) : 0;
  g_env.max_grid.store(g > 0 && g < (1L << 30) ? (uint32_t)g : 0u, std::memory_order_relaxed);
  const char* cap = getenv("MRR_LDS_CAP");
  g_env.lds_cap.store(!(cap && cap[0] == '0' && cap[1] == '\0'), std::memory_order_relaxed);
  g_env.rsag_wpc.store(env_atoi("MRR_RSAG_WPC"), std::memory_order_relaxed);
  g_env.rsag_any_m.store(env_atoi("MRR_RSAG_ANY_M"), std::memory_order_relaxed);
  const char* sm = getenv("MRR_RSAG_SMALL");
  g_env.rsag_small.store(!(sm && sm[0] == '0'), std::memory_order_relaxed);
  g_env.codec_u.store(env_atoi("MRR_CODEC_U"), std::memory_order_relaxed);
  g_env.codec_wpc.store(env_atoi("MRR_CODEC_WPC"), std::memory_order_relaxed);
  g_env.cooperative.store(env_atoi("MRR_COOPERATIVE") == 1, std::memory_order_relaxed);
}

struct EnvAtLoad {
  EnvAtLoad() { read_env(); }
} g_env_at_load;
}  // namespace

static bool log_enabled() { return g_env.log.load(std::memory_order_relaxed) != 0; }

static mrr_status refuse(mrr_status st, const char* fn, const char* why) {
  if (log_enabled()) fprintf(stderr, "libmrr: %s refused (%s): %s\n", fn, mrr_status_string(st), why);
  return st;
}

static int tsize(int t) {
  switch (t) {
    case kF32: return 4;
    case kF16: return 2;
    case kBF16: return 2;
    case kFP8: return 1;
    case kFP8FN: return 1;
    default: return 0;
  }
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
static bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// outputs[k] may be exactly inputs[k] (same start and length); any other
// overlap of an output with any input or output is refused.
static bool bad_overlap(const void* const* in, size_t in_bytes, void* const* out, size_t out_bytes,
                        int n) {
  for (int k = 0; k < n; ++k) {
    const Range o{(uintptr_t)out[k], (uintptr_t)out[k] + out_bytes};
    for (int r = 0; r < n; ++r) {
      const Range i{(uintptr_t)in[r], (uintptr_t)in[r] + in_bytes};
      if (!overlaps(o, i)) continue;
      if (r == k && o.lo == i.lo && out_bytes == in_bytes) continue;
      return true;
    }
    for (int j = k + 1; j < n; ++j) {
      const Range q{(uintptr_t)out[j], (uintptr_t)out[j] + out_bytes};
      if (overlaps(o, q)) return true;
    }
  }
  return false;
}

static bool valid_nranks(int n) { return n == 2 || n == 4 || n == 8 || n == 16 || n == 32; }

static mrr_status hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return MRR_OK;
  if (log_enabled()) fprintf(stderr, "libmrr: %s: HIP error %s\n", fn, hipGetErrorString(e));
  return MRR_EHIP;
}

int device_cu_count(int device) {
  static std::mutex mu;
  static int cached[64] = {0};
  if (device < 0 && hipGetDevice(&device) != hipSuccess) return 0;
  if (device < 0 || device >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[device] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
      return 0;
    cached[device] = cus;
  }
  return cached[device];
}

// LDS bytes per CU and the most one workgroup may allocate, of the current
// device (0 when unknown).
void device_lds_limits(size_t* per_cu, size_t* per_block) {
  static std::mutex mu;
  static size_t cached_cu[64] = {0}, cached_block[64] = {0};
  *per_cu = *per_block = 0;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= 64) return;
  std::lock_guard<std::mutex> lock(mu);
  if (cached_cu[device] == 0) {
    int cu = 0, blk = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, device) !=
            hipSuccess ||
        hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, device) != hipSuccess)
      return;
    cached_cu[device] = cu > 0 ? (size_t)cu : 0;
    cached_block[device] = blk > 0 ? (size_t)blk : 0;
  }
  *per_cu = cached_cu[device];
  *per_block = cached_block[device];
}

// Dynamic LDS bytes that let at most `wpc` workgroups share a CU: the CU's
// LDS divided by wpc, rounded down to 1 KiB, clamped to what one workgroup may
// allocate; 0 (no cap) when wpc <= 0 or the device reports no LDS size.  On
// MI355X (160 KiB per CU) the LDS is handed out in two halves of 80 KiB, so
// an odd cap behaves as the even cap below it (caps 2 and 3 were measured to
// time the same); the launch tables use even caps.
size_t occupancy_lds_bytes(int wpc) {
  if (wpc <= 0) return 0;
  size_t per_cu = 0, per_block = 0;
  device_lds_limits(&per_cu, &per_block);
  size_t lds = per_cu / (size_t)wpc / 1024 * 1024;
  if (lds > per_block) lds = per_block;
  return lds;
}

// MRR_MAX_GRID=<g> limits the one-workgroup-per-tile launches (RS/AG and
// codec) to g workgroups, each then walking several tiles, so that a test can
// exercise that path at small sizes.  0 when unset.
uint32_t max_grid_override() { return g_env.max_grid.load(std::memory_order_relaxed); }

// MRR_LDS_CAP=0 turns the LDS reservation off: the RS/AG and codec launches
// then use a persistent grid of wpc workgroups per CU striding over the
// tiles, which leaves the LDS free for kernels running concurrently on other
// streams, at 9-17 % lower bandwidth (measured on MI355X: 8 x 64 MiB f16 0.73
// of the HBM peak against 0.81, 8 x 256 MiB bf16 0.65 against 0.78, the f16
// decode 0.69 against 0.76).
bool lds_cap_enabled() { return g_env.lds_cap.load(std::memory_order_relaxed) != 0; }

int rsag_wpc_override() { return g_env.rsag_wpc.load(std::memory_order_relaxed); }
int rsag_any_m_override() { return g_env.rsag_any_m.load(std::memory_order_relaxed); }
bool rsag_small_enabled() { return g_env.rsag_small.load(std::memory_order_relaxed) != 0; }
int codec_u_override() { return g_env.codec_u.load(std::memory_order_relaxed); }
int codec_wpc_override() { return g_env.codec_wpc.load(std::memory_order_relaxed); }

// MRR_COOPERATIVE=1: the kernels whose workgroups wait for each other (the
// packet allreduces and the full mesh) launch through
// hipLaunchCooperativeKernel, so a grid that cannot be resident at once is a
// launch error (MRR_EHIP) instead of a wait.  Measured on MI355X, 8 ranks of
// f16: about 15 us more per eager call (16 KiB allpair 10.3 -> 24.4 us,
// full mesh 9.2 -> 25.4 us), and 4-14 us more per graph replay, so it is
// off by default; captured calls launch cooperatively too.
bool cooperative_launch_enabled() { return g_env.cooperative.load(std::memory_order_relaxed) != 0; }

hipError_t launch_resident(const void* kernel, dim3 grid, dim3 block, void* args,
                           hipStream_t stream) {
  void* params[] = {args};
  hipError_t e = cooperative_launch_enabled()
                     ? hipLaunchCooperativeKernel(kernel, grid, block, params, 0, stream)
                     : hipLaunchKernel(kernel, grid, block, params, 0, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the error is returned here; do not leave it to the next call
    return e;
  }
  return hipGetLastError();
}

// Workgroups of `kernel` at `threads` threads that fit on the device at once,
// cached per (kernel, threads, device): the occupancy query costs
// microseconds and its answer never changes within a process.
static int max_resident_blocks(const void* kernel, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  struct Entry {
    const void* kernel;
    int threads, device, blocks;
  };
  static std::mutex mu;
  static Entry cache[256];
  static int used = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].kernel == kernel && cache[i].threads == threads && cache[i].device == dev)
        return cache[i].blocks;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  const int blocks = per_cu * device_cu_count(dev);
  std::lock_guard<std::mutex> lock(mu);
  if (used < 256 && blocks > 0) cache[used++] = Entry{kernel, threads, dev, blocks};
  return blocks;
}

}  // namespace mrr

namespace mrr {
// calib.hip: plain copy on the RS/AG launch scheme; src/dst 16-byte aligned
// and disjoint (checked by mrr_stream_copy).
hipError_t launch_stream_copy(const void* src, void* dst, size_t nbytes, hipStream_t stream);
}  // namespace mrr

using namespace mrr;

extern "C" {

const char* mrr_status_string(mrr_status s) {
  switch (s) {
    case MRR_OK: return "MRR_OK: success";
    case MRR_EINVAL: return "MRR_EINVAL: invalid argument";
    case MRR_EUNSUPPORTED: return "MRR_EUNSUPPORTED: rank count or type combination not supported";
    case MRR_EALIGN: return "MRR_EALIGN: pointer misaligned";
    case MRR_EOVERLAP: return "MRR_EOVERLAP: output overlaps another buffer";
    case MRR_ESCRATCH: return "MRR_ESCRATCH: packet scratch too small";
    case MRR_ETIMEDOUT: return "MRR_ETIMEDOUT: packet poll exceeded max_spins";
    case MRR_EHIP: return "MRR_EHIP: HIP runtime error";
  }
  return "unknown mrr_status";
}

int mrr_version(void) { return 10100; }

void mrr_reload_env(void) { read_env(); }

// From 4 ranks up, buffers an odd multiple of 128 MiB long take another
// stagger: at the usual one their equal-offset streams collide (measured on
// MI355X, bf16 RS/AG, fractions of the HBM peak, usual stagger -> this one:
// 8 ranks x 128 MiB 0.74 -> 0.80, x 384 MiB 0.77 -> 0.80; 4 x 128 MiB 0.77 ->
// 0.80; 32 x 128 MiB 0.70 -> 0.74; 16 x 128 MiB unchanged at 0.77; 2 x 128
// MiB is fine at 4 KiB, 0.80, and slower at 5 KiB, 0.78).  Sizes 64, 96, 160,
// 192, 256, 320 and 512 MiB keep the usual stagger, as good or better there.
size_t mrr_rank_buffer_pitch(size_t bytes_per_rank, int nranks) {
  if (bytes_per_rank == 0 || nranks < 1) return 0;
  const size_t page = 4096;
  const size_t rounded = (bytes_per_rank + page - 1) / page * page;
  const bool odd128 = nranks >= 4 && rounded % ((size_t)256 << 20) == ((size_t)128 << 20);
  const size_t stagger = nranks >= 16 ? (odd128 ? 8192 : 3072) : (odd128 ? 5120 : 4096);
  return rounded + stagger;
}

// Shared by mrr_allreduce_rsag_ex (compiled rank counts only, as the RS/AG
// algorithm is specified) and mrr_allreduce (any count in [1, 32]).
static mrr_status rsag_call(const char* fn, const void* const* inputs, void* const* outputs,
                            size_t count, mrr_dtype in, mrr_dtype accum, mrr_dtype out, int nranks,
                            int rank, void* stream, bool any_n) {
  if (any_n ? (nranks < 1 || nranks > MRR_MAX_RANKS) : !valid_nranks(nranks))
    return refuse(MRR_EUNSUPPORTED, fn, any_n ? "nranks outside [1, 32]" : "nranks not in {2,4,8,16,32}");
  if (rank < -1 || rank >= nranks) return refuse(MRR_EINVAL, fn, "rank outside [-1, nranks)");
  if (!inputs || !outputs) return refuse(MRR_EINVAL, fn, "null pointer array");
  const int tin = (int)in;
  const int tacc = accum == MRR_AUTO ? tin : (int)accum;
  const int tout = out == MRR_AUTO ? tin : (int)out;
  if (!tsize(tin) || !rsag_types_supported(tin, tacc, tout))
    return refuse(MRR_EUNSUPPORTED, fn, "type combination");
  if (count == 0) return MRR_OK;
  const size_t ein = tsize(tin), eout = tsize(tout);
  if (count > ((uint64_t)1 << 40) / (ein > eout ? ein : eout))
    return refuse(MRR_EINVAL, fn, "count too large for one call (over 1 TiB per buffer)");
  bool vec = true;
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r]) return refuse(MRR_EINVAL, fn, "null buffer");
    if (!aligned(inputs[r], ein) || !aligned(outputs[r], eout))
      return refuse(MRR_EALIGN, fn, "buffer not aligned to its element size");
    vec = vec && aligned(inputs[r], 16) && aligned(outputs[r], 16);
  }
  if (bad_overlap(inputs, count * ein, outputs, count * eout, nranks))
    return refuse(MRR_EOVERLAP, fn, "output overlaps another buffer");
  RsagPlan plan{nranks, tin, tacc, tout, count, rank, vec};
  return hip_status(launch_rsag(plan, inputs, outputs, (hipStream_t)stream), fn);
}

mrr_status mrr_allreduce_rsag_ex(const void* const* inputs, void* const* outputs, size_t count,
                                 mrr_dtype in, mrr_dtype accum, mrr_dtype out, int nranks,
                                 int rank, void* stream) {
  return rsag_call("mrr_allreduce_rsag", inputs, outputs, count, in, accum, out, nranks, rank,
                   stream, false);
}

mrr_status mrr_allreduce_rsag_dual(const void* const* inputs, void* const* outputs,
                                   void* const* outputs2, size_t count, mrr_dtype in,
                                   mrr_dtype accum, int nranks, int rank, void* stream) {
  static const char* fn = "mrr_allreduce_rsag_dual";
  if (!valid_nranks(nranks)) return refuse(MRR_EUNSUPPORTED, fn, "nranks not in {2,4,8,16,32}");
  if (rank < -1 || rank >= nranks) return refuse(MRR_EINVAL, fn, "rank outside [-1, nranks)");
  if (!inputs || !outputs || !outputs2) return refuse(MRR_EINVAL, fn, "null pointer array");
  const int tin = (int)in;
  const int tacc = accum == MRR_AUTO ? tin : (int)accum;
  if (!rsag_dual_supported(tin, tacc)) return refuse(MRR_EUNSUPPORTED, fn, "type combination");
  if (count == 0) return MRR_OK;
  if (count > ((uint64_t)1 << 39)) return refuse(MRR_EINVAL, fn, "count too large for one call");
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r] || !outputs2[r]) return refuse(MRR_EINVAL, fn, "null buffer");
    if (!aligned(inputs[r], 16) || !aligned(outputs[r], 16) || !aligned(outputs2[r], 16))
      return refuse(MRR_EALIGN, fn, "every buffer must be 16-byte aligned");
  }
  // outputs2[k] may be exactly inputs[k] (same type and size); the f16
  // outputs may overlap nothing.
  if (bad_overlap(inputs, count, outputs2, count, nranks) ||
      bad_overlap(inputs, count, outputs, 2 * count, nranks) ||
      bad_overlap((const void* const*)outputs2, count, outputs, 2 * count, nranks))
    return refuse(MRR_EOVERLAP, fn, "an output overlaps another buffer");
  RsagPlan plan{nranks, tin, tacc, kF16, count, rank, true};
  return hip_status(launch_rsag_dual(plan, inputs, outputs, outputs2, (hipStream_t)stream), fn);
}

mrr_status mrr_allreduce_rsag(const void* const* inputs, void* const* outputs, size_t count,
                              mrr_dtype dtype, int nranks, void* stream) {
  return mrr_allreduce_rsag_ex(inputs, outputs, count, dtype, MRR_F32, MRR_AUTO, nranks, -1,
                               stream);
}

// The packet entry points refuse counts above this many bytes per rank, and
// the size helpers return 0 for them (so the products below cannot wrap).
static bool packet_count_ok(size_t count, int e) { return count <= (SIZE_MAX / 64) / (size_t)e; }

size_t mrr_packet_scratch_bytes(size_t count, mrr_dtype dtype, int nranks) {
  const int e = tsize((int)dtype);
  if (!e || nranks <= 0 || nranks > MRR_MAX_RANKS || !packet_count_ok(count, e)) return 0;
  const size_t npkt = (count * (size_t)e + 3) / 4;
  return (size_t)nranks * (size_t)nranks * npkt * 8;
}

size_t mrr_packet_flag_bytes(int nranks) {
  return (nranks <= 0 || nranks > MRR_MAX_RANKS) ? 0
                                                 : (size_t)nranks * MRR_PKT_FLAG_SLOTS * sizeof(uint32_t);
}

// Argument checks shared by the packet allreduce entry points; everything
// here runs before any HIP call.
static mrr_status packet_checks(const char* fn, const void* const* inputs, void* const* outputs,
                                void* scratch, size_t scratch_bytes, size_t scratch_need,
                                uint32_t* flags, size_t count, int t, int tacc, int nranks,
                                int blocks_per_rank, int threads) {
  if (!valid_nranks(nranks)) return refuse(MRR_EUNSUPPORTED, fn, "nranks not in {2,4,8,16,32}");
  if (!inputs || !outputs || !scratch || !flags)
    return refuse(MRR_EINVAL, fn, "null pointer argument");
  if (!tsize(t) || !packet_supported(nranks, t, tacc))
    return refuse(MRR_EUNSUPPORTED, fn, "type combination");
  if (threads != 0 && (threads < 64 || threads > packet_max_threads() || threads % 64 != 0))
    return refuse(MRR_EINVAL, fn, "threads must be a multiple of 64 in [64, 512]");
  if (blocks_per_rank < 0 || blocks_per_rank > MRR_PKT_FLAG_SLOTS)
    return refuse(MRR_EINVAL, fn, "blocks_per_rank outside [1, MRR_PKT_FLAG_SLOTS]");
  if (!aligned(scratch, 8) || !aligned(flags, 4)) return refuse(MRR_EALIGN, fn, "scratch/flags");
  if (count == 0) return MRR_OK;
  const size_t e = tsize(t);
  if (!packet_count_ok(count, e)) return refuse(MRR_EINVAL, fn, "count too large");
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r]) return refuse(MRR_EINVAL, fn, "null buffer");
    if (!aligned(inputs[r], 4) || !aligned(outputs[r], 4))
      return refuse(MRR_EALIGN, fn, "buffers must be 4-byte aligned");
  }
  const size_t nbytes = count * e;
  if (bad_overlap(inputs, nbytes, outputs, nbytes, nranks))
    return refuse(MRR_EOVERLAP, fn, "output overlaps another buffer");
  if (scratch_bytes < scratch_need) return refuse(MRR_ESCRATCH, fn, "scratch smaller than required");
  const Range sr{(uintptr_t)scratch, (uintptr_t)scratch + scratch_need};
  const Range fr{(uintptr_t)flags, (uintptr_t)flags + mrr_packet_flag_bytes(nranks)};
  if (overlaps(sr, fr)) return refuse(MRR_EOVERLAP, fn, "scratch overlaps flags");
  for (int r = 0; r < nranks; ++r) {
    const Range ir{(uintptr_t)inputs[r], (uintptr_t)inputs[r] + nbytes};
    const Range orr{(uintptr_t)outputs[r], (uintptr_t)outputs[r] + nbytes};
    if (overlaps(sr, ir) || overlaps(sr, orr) || overlaps(fr, ir) || overlaps(fr, orr))
      return refuse(MRR_EOVERLAP, fn, "scratch/flags overlap a data buffer");
  }
  return MRR_OK;
}

// Blocks per rank: the caller's, or one poll round per lane (of `batch`
// packets) over `units` words, capped by the workgroups the GPU holds at once
// and by the flag slots.
static mrr_status packet_geometry(const char* fn, const void* kernel, int nranks, uint64_t units,
                                  int threads, int batch, int blocks_per_rank, int* B) {
  const int resident = max_resident_blocks(kernel, threads);
  if (resident <= 0) return hip_status(hipErrorInvalidDevice, fn);
  const int max_b = resident / nranks;
  int b = blocks_per_rank;
  if (b == 0) {
    const uint64_t per_block = (uint64_t)threads * (uint64_t)batch;
    const uint64_t want = (units + per_block - 1) / per_block;
    b = (int)(want < 1 ? 1 : (want > (uint64_t)MRR_PKT_FLAG_SLOTS ? MRR_PKT_FLAG_SLOTS : want));
    if (b > max_b) b = max_b;
  }
  if (b < 1 || b > max_b)
    return refuse(MRR_EINVAL, fn, "nranks * blocks_per_rank workgroups do not fit on the GPU at once");
  *B = b;
  return MRR_OK;
}

mrr_status mrr_allreduce_packet_ex(const void* const* inputs, void* const* outputs, void* scratch,
                                   size_t scratch_bytes, uint32_t* flags, size_t count,
                                   mrr_dtype dtype, mrr_dtype accum, int nranks,
                                   uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                   int threads, void* stream) {
  static const char* fn = "mrr_allreduce_packet";
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  mrr_status st = packet_checks(fn, inputs, outputs, scratch, scratch_bytes,
                                mrr_packet_scratch_bytes(count, dtype, nranks), flags, count, t,
                                tacc, nranks, blocks_per_rank, threads);
  if (st != MRR_OK || count == 0) return st;
  const size_t nbytes = count * tsize(t);
  const uint64_t npkt = (nbytes + 3) / 4;
  const int T = threads ? threads : 64;
  int B = 0;
  const int batch = packet_allpair_batch(nranks, npkt);
  st = packet_geometry(fn, packet_allpair_kernel(nranks, t, tacc, batch), nranks, npkt, T, batch,
                       blocks_per_rank, &B);
  if (st != MRR_OK) return st;
  PacketArgs a = {};
  for (int r = 0; r < nranks; ++r) {
    a.in[r] = inputs[r];
    a.out[r] = outputs[r];
  }
  a.scratch = (uint64_t*)scratch;
  a.flags = flags;
  a.dev_err = dev_err;
  a.nbytes = nbytes;
  a.npkt = npkt;
  a.pkts_per_block = (npkt + (uint64_t)B - 1) / (uint64_t)B;
  a.nblocks = (uint32_t)B;
  a.max_spins = max_spins;
  a.flag_ranks = (uint32_t)nranks;
  return hip_status(launch_packet_allpair(a, nranks, t, tacc, T, batch, (hipStream_t)stream), fn);
}

mrr_status mrr_allreduce_packet_noalloc(const void* const* inputs, void* const* outputs,
                                        size_t count, mrr_dtype dtype, mrr_dtype accum,
                                        int nranks, uint32_t max_spins, uint32_t* dev_err,
                                        void* stream) {
  static const char* fn = "mrr_allreduce_packet_noalloc";
  if (!valid_nranks(nranks)) return refuse(MRR_EUNSUPPORTED, fn, "nranks not in {2,4,8,16,32}");
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  if (!inputs || !outputs) return refuse(MRR_EINVAL, fn, "null pointer array");
  if (!tsize(t) || !packet_supported(nranks, t, tacc))
    return refuse(MRR_EUNSUPPORTED, fn, "type combination");
  if (count == 0) return MRR_OK;
  const size_t need = mrr_packet_scratch_bytes(count, dtype, nranks);
  if (need == 0 || need > (size_t)MRR_NOALLOC_SCRATCH_BYTES)
    return refuse(MRR_ESCRATCH, fn,
                  "nranks^2 * ceil(count * elem_size / 4) * 8 bytes exceed MRR_NOALLOC_SCRATCH_BYTES");
  const size_t nbytes = count * tsize(t);
  for (int r = 0; r < nranks; ++r) {
    if (!inputs[r] || !outputs[r]) return refuse(MRR_EINVAL, fn, "null buffer");
    if (!aligned(inputs[r], 4) || !aligned(outputs[r], 4))
      return refuse(MRR_EALIGN, fn, "buffers must be 4-byte aligned");
  }
  if (bad_overlap(inputs, nbytes, outputs, nbytes, nranks))
    return refuse(MRR_EOVERLAP, fn, "output overlaps another buffer");
  const uint64_t npkt = (nbytes + 3) / 4;
  const int T = 64;
  const int batch = packet_allpair_batch(nranks, npkt);
  int B = 0;
  mrr_status st = packet_geometry(fn, packet_allpair_kernel(nranks, t, tacc, batch), nranks,
                                  npkt, T, batch, 0, &B);
  if (st != MRR_OK) return st;
  uint8_t* ws = nullptr;
  const hipError_t e = noalloc_workspace((hipStream_t)stream, &ws);
  if (e == hipErrorStreamCaptureUnsupported)
    return refuse(MRR_EINVAL, fn, "the first call on a device must not be under stream capture");
  if (e != hipSuccess) return hip_status(e, fn);
  PacketArgs a = {};
  for (int r = 0; r < nranks; ++r) {
    a.in[r] = inputs[r];
    a.out[r] = outputs[r];
  }
  a.flags = reinterpret_cast<uint32_t*>(ws);
  a.scratch = reinterpret_cast<uint64_t*>(ws + kNoAllocFlagBytes);
  a.dev_err = dev_err;
  a.nbytes = nbytes;
  a.npkt = npkt;
  a.pkts_per_block = (npkt + (uint64_t)B - 1) / (uint64_t)B;
  a.nblocks = (uint32_t)B;
  a.max_spins = max_spins;
  a.flag_ranks = (uint32_t)MRR_MAX_RANKS;
  return hip_status(launch_packet_allpair(a, nranks, t, tacc, T, batch, (hipStream_t)stream), fn);
}

// Payload words per full chunk of the two-phase packet allreduce: the RS/AG
// chunk C = roundup(ceil(count / N), 16 / e) elements, C * e / 4 words.
static uint64_t rsag_chunk_words(size_t count, int e, int nranks) {
  const uint64_t per = (count + (uint64_t)nranks - 1) / (uint64_t)nranks;
  const uint64_t vw = 16 / (uint64_t)e;
  return (per + vw - 1) / vw * vw * (uint64_t)e / 4;
}

size_t mrr_packet_rsag_scratch_bytes(size_t count, mrr_dtype dtype, int nranks) {
  const int e = tsize((int)dtype);
  if (!e || nranks <= 0 || nranks > MRR_MAX_RANKS || !packet_count_ok(count, e)) return 0;
  return 2 * (size_t)nranks * (size_t)nranks * rsag_chunk_words(count, e, nranks) * 8;
}

mrr_status mrr_allreduce_packet_rsag(const void* const* inputs, void* const* outputs,
                                     void* scratch, size_t scratch_bytes, uint32_t* flags,
                                     size_t count, mrr_dtype dtype, mrr_dtype accum, int nranks,
                                     uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                     int threads, void* stream) {
  static const char* fn = "mrr_allreduce_packet_rsag";
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  mrr_status st = packet_checks(fn, inputs, outputs, scratch, scratch_bytes,
                                mrr_packet_rsag_scratch_bytes(count, dtype, nranks), flags, count,
                                t, tacc, nranks, blocks_per_rank, threads);
  if (st != MRR_OK || count == 0) return st;
  const int e = tsize(t);
  const uint64_t cw = rsag_chunk_words(count, e, nranks);
  const int T = threads ? threads : 64;
  int B = 0;
  st = packet_geometry(fn, packet_rsag_kernel(nranks, t, tacc), nranks, cw, T, 1, blocks_per_rank,
                       &B);
  if (st != MRR_OK) return st;
  PacketRsagArgs a = {};
  for (int r = 0; r < nranks; ++r) {
    a.in[r] = inputs[r];
    a.out[r] = outputs[r];
  }
  a.scratch = (uint64_t*)scratch;
  a.flags = flags;
  a.dev_err = dev_err;
  a.nbytes = count * (size_t)e;
  a.nwords = (a.nbytes + 3) / 4;
  a.cw = cw;
  a.words_per_block = (cw + (uint64_t)B - 1) / (uint64_t)B;
  a.nblocks = (uint32_t)B;
  a.max_spins = max_spins;
  return hip_status(launch_packet_rsag(a, nranks, t, tacc, T, (hipStream_t)stream), fn);
}

// Chunk width of the two-phase packet and full-mesh allreduces, in elements:
// C = roundup(ceil(count / N), 16 / e).
static uint64_t chunk16_elems(size_t count, int e, int nranks) {
  const uint64_t per = (count + (uint64_t)nranks - 1) / (uint64_t)nranks;
  const uint64_t vw = 16 / (uint64_t)e;
  return (per + vw - 1) / vw * vw;
}

// Full-mesh scratch: N * N * MRR_PKT_FLAG_SLOTS semaphores of 8 bytes, then
// N * N inboxes of one chunk each.
static size_t fullmesh_sem_bytes(int nranks) {
  return (size_t)nranks * (size_t)nranks * MRR_PKT_FLAG_SLOTS * 8;
}

size_t mrr_fullmesh_scratch_bytes(size_t count, mrr_dtype dtype, int nranks) {
  const int e = tsize((int)dtype);
  if (!e || nranks <= 0 || nranks > MRR_MAX_RANKS || !packet_count_ok(count, e)) return 0;
  return fullmesh_sem_bytes(nranks) +
         (size_t)nranks * (size_t)nranks * chunk16_elems(count, e, nranks) * (size_t)e;
}

mrr_status mrr_allreduce_fullmesh(const void* const* inputs, void* const* outputs, void* scratch,
                                  size_t scratch_bytes, uint32_t* flags, size_t count,
                                  mrr_dtype dtype, mrr_dtype accum, int nranks,
                                  uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                  int threads, void* stream) {
  static const char* fn = "mrr_allreduce_fullmesh";
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  if (threads != 0 && (threads < 64 || threads > fullmesh_max_threads() || threads % 64 != 0))
    return refuse(MRR_EINVAL, fn, "threads must be a multiple of 64 in [64, 512]");
  mrr_status st = packet_checks(fn, inputs, outputs, scratch, scratch_bytes,
                                mrr_fullmesh_scratch_bytes(count, dtype, nranks), flags, count, t,
                                tacc, nranks, blocks_per_rank, 0);
  if (st != MRR_OK || count == 0) return st;
  if (!aligned(scratch, 16)) return refuse(MRR_EALIGN, fn, "scratch must be 16-byte aligned");
  for (int r = 0; r < nranks; ++r)
    if (!aligned(inputs[r], 16) || !aligned(outputs[r], 16))
      return refuse(MRR_EALIGN, fn, "inputs and outputs must be 16-byte aligned");
  const int e = tsize(t);
  const uint64_t chunk = chunk16_elems(count, e, nranks);
  const uint64_t cvec = chunk * (uint64_t)e / 16;
  // Auto geometry: 256-lane workgroups, one vector per lane per chunk, at
  // most kFmAutoWorkgroups workgroups in all.  Every workgroup pays one
  // agent-scope release (an L2 writeback) and one acquire (an L2
  // invalidate), so fewer, wider workgroups win once there is enough work:
  // measured on MI355X, 8 ranks of f16, 64-lane workgroups with one vector
  // per lane took 16.2 / 53.6 / 267 us at 256 KiB / 1 MiB / 4 MiB per rank,
  // 256 lanes 7.3 / 14.6 / 60.6 us, and 256 lanes with 16 blocks per rank
  // 8.0 / 12.9 / 30.2 us (16 MiB: 129 us; 64 blocks 116 us).
  constexpr int kFmAutoThreads = 256;
  constexpr int kFmAutoWorkgroups = 256;
  const int T = threads ? threads : kFmAutoThreads;
  int B = blocks_per_rank;
  if (B == 0) {
    const uint64_t want = (cvec + (uint64_t)T - 1) / (uint64_t)T;
    const uint64_t cap = kFmAutoWorkgroups / nranks > 1 ? kFmAutoWorkgroups / nranks : 1;
    B = (int)(want < 1 ? 1 : want > cap ? cap : want);
    const int fit = max_resident_blocks(fullmesh_kernel(nranks, t, tacc), T) / nranks;
    if (B > fit && fit >= 1) B = fit;
  }
  st = packet_geometry(fn, fullmesh_kernel(nranks, t, tacc), nranks, cvec, T, 1, B, &B);
  if (st != MRR_OK) return st;
  FullmeshArgs a = {};
  for (int r = 0; r < nranks; ++r) {
    a.in[r] = inputs[r];
    a.out[r] = outputs[r];
  }
  a.sem = (uint64_t*)scratch;
  a.inbox = (uint8_t*)scratch + fullmesh_sem_bytes(nranks);
  a.flags = flags;
  a.dev_err = dev_err;
  a.count = count;
  a.chunk = chunk;
  a.vec_per_block = (cvec + (uint64_t)B - 1) / (uint64_t)B;
  a.nblocks = (uint32_t)B;
  a.max_spins = max_spins;
  return hip_status(launch_fullmesh(a, nranks, t, tacc, T, (hipStream_t)stream), fn);
}

mrr_status mrr_allreduce_packet(const void* const* inputs, void* const* outputs, void* scratch,
                                size_t scratch_bytes, uint32_t* flags, size_t count,
                                mrr_dtype dtype, mrr_dtype accum, int nranks,
                                uint32_t max_spins, uint32_t* dev_err, void* stream) {
  return mrr_allreduce_packet_ex(inputs, outputs, scratch, scratch_bytes, flags, count, dtype,
                                 accum, nranks, max_spins, dev_err, 0, 0, stream);
}

mrr_status mrr_allreduce(const void* const* inputs, void* const* outputs, size_t count,
                         mrr_dtype dtype, mrr_dtype accum, int nranks, void* scratch,
                         size_t scratch_bytes, uint32_t* flags, size_t packet_max_bytes,
                         uint32_t max_spins, uint32_t* dev_err, void* stream) {
  static const char* fn = "mrr_allreduce";
  if (nranks < 1 || nranks > MRR_MAX_RANKS) return refuse(MRR_EUNSUPPORTED, fn, "nranks outside [1, 32]");
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  const size_t e = tsize(t);
  const bool packets = valid_nranks(nranks) && scratch && flags && e && count > 0 &&
                       count <= packet_max_bytes / e && packet_supported(nranks, t, tacc) &&
                       scratch_bytes >= mrr_packet_scratch_bytes(count, dtype, nranks);
  if (packets)
    return mrr_allreduce_packet(inputs, outputs, scratch, scratch_bytes, flags, count, dtype,
                                accum, nranks, max_spins, dev_err, stream);
  return rsag_call(fn, inputs, outputs, count, dtype, accum, MRR_AUTO, nranks, -1, stream, true);
}

mrr_status mrr_packet_reduce(const uint64_t* const* in_pkts, uint64_t* out_pkts, size_t npkts,
                             mrr_dtype dtype, mrr_dtype accum, int nranks, uint32_t flag_in,
                             uint32_t flag_out, uint32_t max_spins, uint32_t* dev_err,
                             void* stream) {
  static const char* fn = "mrr_packet_reduce";
  if (!valid_nranks(nranks)) return refuse(MRR_EUNSUPPORTED, fn, "nranks not in {2,4,8,16,32}");
  if (!in_pkts || !out_pkts) return refuse(MRR_EINVAL, fn, "null pointer argument");
  const int t = (int)dtype;
  const int tacc = accum == MRR_AUTO ? t : (int)accum;
  if (!tsize(t) || !packet_supported(nranks, t, tacc))
    return refuse(MRR_EUNSUPPORTED, fn, "type combination");
  if (npkts == 0) return MRR_OK;
  if (npkts > SIZE_MAX / 64) return refuse(MRR_EINVAL, fn, "npkts too large");
  if (!aligned(out_pkts, 8)) return refuse(MRR_EALIGN, fn, "out_pkts");
  const Range o{(uintptr_t)out_pkts, (uintptr_t)out_pkts + npkts * 8};
  PacketReduceArgs a = {};
  for (int r = 0; r < nranks; ++r) {
    if (!in_pkts[r]) return refuse(MRR_EINVAL, fn, "null packet buffer");
    if (!aligned(in_pkts[r], 8)) return refuse(MRR_EALIGN, fn, "in_pkts");
    const Range i{(uintptr_t)in_pkts[r], (uintptr_t)in_pkts[r] + npkts * 8};
    if (overlaps(o, i)) return refuse(MRR_EOVERLAP, fn, "out_pkts overlaps an input");
    a.in[r] = in_pkts[r];
  }
  a.out = out_pkts;
  a.dev_err = dev_err;
  a.npkts = npkts;
  a.flag_in = flag_in;
  a.flag_out = flag_out;
  a.max_spins = max_spins;
  return hip_status(launch_packet_reduce(a, nranks, t, tacc, (hipStream_t)stream), fn);
}

mrr_status mrr_pack(const void* src, uint64_t* pkts, size_t nbytes, uint32_t flag, void* stream) {
  static const char* fn = "mrr_pack";
  if (nbytes == 0) return MRR_OK;
  if (!src || !pkts) return refuse(MRR_EINVAL, fn, "null pointer");
  if (nbytes > SIZE_MAX / 4) return refuse(MRR_EINVAL, fn, "nbytes too large");
  if (!aligned(src, 4) || !aligned(pkts, 8)) return refuse(MRR_EALIGN, fn, "src 4 / pkts 8 bytes");
  const Range s{(uintptr_t)src, (uintptr_t)src + nbytes};
  const Range p{(uintptr_t)pkts, (uintptr_t)pkts + (nbytes + 3) / 4 * 8};
  if (overlaps(s, p)) return refuse(MRR_EOVERLAP, fn, "src overlaps pkts");
  return hip_status(launch_pack(src, pkts, nbytes, flag, (hipStream_t)stream), fn);
}

mrr_status mrr_unpack(const uint64_t* pkts, void* dst, size_t nbytes, void* stream) {
  static const char* fn = "mrr_unpack";
  if (nbytes == 0) return MRR_OK;
  if (!dst || !pkts) return refuse(MRR_EINVAL, fn, "null pointer");
  if (nbytes > SIZE_MAX / 4) return refuse(MRR_EINVAL, fn, "nbytes too large");
  if (!aligned(dst, 4) || !aligned(pkts, 8)) return refuse(MRR_EALIGN, fn, "dst 4 / pkts 8 bytes");
  const Range d{(uintptr_t)dst, (uintptr_t)dst + nbytes};
  const Range p{(uintptr_t)pkts, (uintptr_t)pkts + (nbytes + 3) / 4 * 8};
  if (overlaps(d, p)) return refuse(MRR_EOVERLAP, fn, "dst overlaps pkts");
  return hip_status(launch_unpack(pkts, dst, nbytes, (hipStream_t)stream), fn);
}

static mrr_status codec(int dir, const void* in, size_t ein, void* out, size_t eout, size_t n,
                        void* stream, const char* fn) {
  if (n == 0) return MRR_OK;
  if (!in || !out) return refuse(MRR_EINVAL, fn, "null pointer");
  if (n > (SIZE_MAX / 8)) return refuse(MRR_EINVAL, fn, "n too large");
  if (!aligned(in, ein) || !aligned(out, eout)) return refuse(MRR_EALIGN, fn, "element alignment");
  const Range i{(uintptr_t)in, (uintptr_t)in + n * ein};
  const Range o{(uintptr_t)out, (uintptr_t)out + n * eout};
  if (overlaps(i, o)) return refuse(MRR_EOVERLAP, fn, "in overlaps out");
  const bool vec = aligned(in, 16) && aligned(out, 16);
  return hip_status(launch_codec(dir, in, out, n, vec, (hipStream_t)stream), fn);
}

mrr_status mrr_fp8b15_to_f16(const uint8_t* in, uint16_t* out, size_t n, void* stream) {
  return codec(0, in, 1, out, 2, n, stream, "mrr_fp8b15_to_f16");
}
mrr_status mrr_fp8b15_to_f32(const uint8_t* in, float* out, size_t n, void* stream) {
  return codec(1, in, 1, out, 4, n, stream, "mrr_fp8b15_to_f32");
}
mrr_status mrr_f16_to_fp8b15(const uint16_t* in, uint8_t* out, size_t n, void* stream) {
  return codec(2, in, 2, out, 1, n, stream, "mrr_f16_to_fp8b15");
}
mrr_status mrr_f32_to_fp8b15(const float* in, uint8_t* out, size_t n, void* stream) {
  return codec(3, in, 4, out, 1, n, stream, "mrr_f32_to_fp8b15");
}

mrr_status mrr_stream_copy(const void* src, void* dst, size_t nbytes, void* stream) {
  const char* fn = "mrr_stream_copy";
  if (nbytes == 0) return MRR_OK;
  if (!src || !dst) return refuse(MRR_EINVAL, fn, "null pointer");
  if (nbytes > ((size_t)1 << 40)) return refuse(MRR_EINVAL, fn, "nbytes over 1 TiB");
  if (!aligned(src, 16) || !aligned(dst, 16)) return refuse(MRR_EALIGN, fn, "16-byte alignment");
  const Range i{(uintptr_t)src, (uintptr_t)src + nbytes};
  const Range o{(uintptr_t)dst, (uintptr_t)dst + nbytes};
  if (overlaps(i, o)) return refuse(MRR_EOVERLAP, fn, "src overlaps dst");
  return hip_status(launch_stream_copy(src, dst, nbytes, (hipStream_t)stream), fn);
}

}  // extern "C"
