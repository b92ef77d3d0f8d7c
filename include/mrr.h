/*
 * mrr.h -- libmrr: N-rank allreduce reduction for AMD MI355X (gfx950).
 *
 * One GPU holds the N "rank" buffers in its own HBM; each call performs every
 * rank's share of the reduction (or one chosen rank's share) in HIP kernels.
 *
 * Operations, and the passages that define them:
 *   - RS/AG zero-copy allreduce: "Support 2 ranks in AllreduceRsAgZeroCopy"
 *     (MSCCL++ PR #948), sections "why" and "what changed": rank r reduces
 *     chunk r of every rank's input and writes the result straight into every
 *     rank's output, with no scratch; it is compiled once per rank count,
 *     with the rank loops unrolled, for 2, 4, 8, 16 and 32 ranks; any other
 *     rank count is refused.
 *   - LL-packet allpair allreduce: MSCCL++ commit history (/src), entry fixing
 *     the allreduce_allpair_packet algorithm: packets go to a scratch area so
 *     the input is never overwritten, one workgroup sends, reduces and writes
 *     back, block/thread counts are validated, and the flag update works when
 *     a workgroup has fewer threads than flags.  Entry on the default flag
 *     buffer: one flag buffer shared by all algorithms so that switching
 *     between them by message size cannot hang.
 *   - FP8 E4M3B15 and accumulation precision: MSCCL++ commit history, entries
 *     adding the fp8_e4m3b15 datatype (4 exponent bits, 3 mantissa bits,
 *     bias 15, largest finite value 0.9375, converted through fp16) and the
 *     accumDtype parameter (AUTO resolves to the input type), and the entry
 *     adding ROCm support for the type with FP16/FP32 accumulation.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers on the calling thread's current
 *     HIP device.  Pointer arrays (inputs[], outputs[], in_pkts[]) are HOST
 *     arrays of nranks device pointers; they are copied into the kernel
 *     arguments, so the host arrays may be reused as soon as the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call is stream-ordered and asynchronous: it validates its
 *     arguments on the host, launches, and returns without synchronising.
 *     No call allocates or frees memory, so calls may be captured in a HIP
 *     graph (the allocation-free entry point after its first call on a
 *     device, which sets up its workspace).
 *   - The caller owns every buffer.  Apart from the workspace of the
 *     allocation-free packet entry point (mrr_allreduce_packet_noalloc,
 *     below), the library keeps no device state; it caches only per-device
 *     properties (CU count, LDS size, occupancy).
 *   - Validation happens before any launch: on an error nothing is launched
 *     and the specific status is returned.  MRR_LOG=1 in the environment
 *     prints one stderr line per refused call (see mrr_reload_env).
 *   - count == 0 (or n == 0) returns MRR_OK without launching.
 *   - Element types travel as raw bits: f16 / bf16 as 16-bit IEEE binary16 /
 *     bfloat16, FP8 E4M3B15 as one byte (sign, 4-bit exponent with bias 15,
 *     3-bit mantissa; exponent 15 encodes inf (mantissa 0) and NaN).
 *   - Rounding is IEEE round-to-nearest-even everywhere.  f16 / bf16 overflow
 *     gives +-inf; FP8 E4M3B15 saturates to +-0.9375 and OCP FP8 E4M3FN to
 *     +-448 (also from +-inf); NaN gives NaN (FP8: 0x7F with the input's
 *     sign).  Denormals are kept.
 *   - OCP FP8 E4M3FN (MRR_FP8_E4M3FN) is accepted wherever FP8 E4M3B15 is as
 *     an input / accumulator / output type of the allreduce entry points
 *     (the pages' benchmarks reduce fp8_e4m3fn data; PR #948, "why").
 */
#ifndef MRR_H
#define MRR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mrr_status {
  MRR_OK = 0,
  MRR_EINVAL = 1,       /* bad argument: null pointer, rank or geometry out of range */
  MRR_EUNSUPPORTED = 2, /* rank count or type combination not provided */
  MRR_EALIGN = 3,       /* a pointer not aligned as the entry point requires */
  MRR_EOVERLAP = 4,     /* an output overlaps another buffer other than its own input */
  MRR_ESCRATCH = 5,     /* packet scratch smaller than mrr_packet_scratch_bytes() */
  MRR_ETIMEDOUT = 6,    /* (device error word only) a packet poll exceeded max_spins */
  MRR_EHIP = 7          /* the HIP runtime refused the launch */
} mrr_status;

typedef enum mrr_dtype {
  MRR_AUTO = 0, /* accumulation: the input type; output: the input type */
  MRR_F32 = 1,
  MRR_F16 = 2,
  MRR_BF16 = 3,
  MRR_FP8_E4M3B15 = 4,
  MRR_FP8_E4M3FN = 5 /* OCP FP8 E4M3FN: bias 7, largest finite 448, 0x7F/0xFF NaN, no inf */
} mrr_dtype;

/* Packet / RS-AG crossover for mrr_allreduce, measured on one MI355X: 0.
 * There RS/AG is faster at every size (8 ranks of f16, per call under HIP
 * graph replay: 1.9 us against 5.7-8.8 us for allpair packets at 16-64 KiB
 * per rank, 3.6 us against 47.3 us at 1 MiB), because within one GPU it
 * needs no cross-rank synchronisation while packets double the bytes moved.
 * The pages' selectors, spanning GPUs, switch to RS/AG above 512 KiB
 * (Python default) or 2 MiB (NCCL shim). */
#define MRR_PACKET_MAX_BYTES_ONE_GPU 0

/* Largest rank count any entry point accepts. */
#define MRR_MAX_RANKS 32
/* Flag slots per rank in a packet flag buffer. */
#define MRR_PKT_FLAG_SLOTS 1024

/* --------------------------------------------------------------------------
 * RS/AG zero-copy allreduce ("Support 2 ranks in AllreduceRsAgZeroCopy",
 * sections "why" and "what changed").
 *
 * For every k < nranks and i < count:
 *   outputs[k][i] = round_out( x_0[i] + x_1[i] + ... + x_{nranks-1}[i] )
 * summed in rank order 0..nranks-1 starting from x_0 (so -0 sums stay -0).
 * The index space is split into nranks chunks of
 *   C = roundup(ceil(count / nranks), 256 / sizeof(input element))
 * elements (the last chunks may be short or empty); chunk r is rank r's
 * reduce-scatter share, and its reduced values are written to all nranks
 * outputs (the all-gather).  The result does not depend on the partition;
 * the 256-byte rounding keeps every chunk on the cache-line grid.
 *
 * mrr_allreduce_rsag: input type == output type == dtype (F32, F16, BF16 or
 *   FP8_E4M3B15), FP32 accumulation, every chunk.
 * mrr_allreduce_rsag_ex:
 *   in     F32 | F16 | BF16 | FP8_E4M3B15
 *   accum  AUTO (= in) | F32 | F16 (F16 and FP8 inputs) | BF16 (BF16 inputs) |
 *          FP8_E4M3B15 (FP8 inputs).  With a non-F32 accumulator every
 *          partial sum is rounded to that type.
 *   out    AUTO (= in); FP8 inputs may also produce F16 or F32.
 *   rank   -1: all chunks (every rank's share); 0..nranks-1: chunk `rank`
 *          only, i.e. one GPU's share at its real shape (reads count/nranks
 *          elements of every input, writes them to every output).
 *
 * Buffers: inputs[r] holds count input elements, outputs[k] room for count
 * output elements.  outputs[k] may be exactly inputs[k] (in place; only when
 * the input and output types have the same size); any other overlap between
 * an output and any buffer gives MRR_EOVERLAP.  Inputs may overlap each
 * other.  Pointers must be aligned to their element size (MRR_EALIGN);
 * 16-byte alignment of every pointer selects the vector kernels, otherwise a
 * slower element-wise kernel runs.
 * Errors: MRR_EUNSUPPORTED for nranks not in {2,4,8,16,32} or a type
 * combination not listed; MRR_EINVAL for null arrays/pointers or a rank
 * outside [-1, nranks); MRR_EHIP when the launch fails.
 * ------------------------------------------------------------------------ */
mrr_status mrr_allreduce_rsag(const void* const* inputs, void* const* outputs, size_t count,
                              mrr_dtype dtype, int nranks, void* stream);

mrr_status mrr_allreduce_rsag_ex(const void* const* inputs, void* const* outputs, size_t count,
                                 mrr_dtype in, mrr_dtype accum, mrr_dtype out, int nranks,
                                 int rank, void* stream);

/* --------------------------------------------------------------------------
 * RS/AG allreduce of FP8 inputs with two outputs from one pass ("MSCCL++
 * commit history for /src", FP8 accumulation entry: FP8 data reduced with
 * higher-precision accumulation; the FP8 workloads emit an f16 result and an
 * FP8 re-encode of the same sums).
 *
 * Same sum, partition and rank semantics as mrr_allreduce_rsag_ex with
 * in = FP8_E4M3B15 or FP8_E4M3FN; every reduced value is written twice:
 *   outputs[k][i]  = round_f16(sum)           (count f16 elements)
 *   outputs2[k][i] = round_in(sum)            (count codes of the input type,
 *                                              RNE, saturating as in the
 *                                              conversions above)
 * both rounded once from the accumulator (so outputs2 is not a rounding of
 * outputs).  Equivalent to two mrr_allreduce_rsag_ex calls (out = F16, then
 * out = in) but the inputs are read once: N*count*(1 + 2 + 1) bytes moved
 * instead of N*count*(1 + 2) + N*count*(1 + 1).
 *   accum  AUTO (= in) | F32 | F16
 * Buffers: every inputs[r], outputs[k] and outputs2[k] 16-byte aligned
 * (MRR_EALIGN otherwise); outputs2[k] may be exactly inputs[k]; any other
 * overlap of an output gives MRR_EOVERLAP.
 * Errors: MRR_EUNSUPPORTED for nranks not in {2,4,8,16,32} or another type;
 * MRR_EINVAL for null arrays/pointers or rank outside [-1, nranks);
 * MRR_EHIP when the launch fails.
 * ------------------------------------------------------------------------ */
mrr_status mrr_allreduce_rsag_dual(const void* const* inputs, void* const* outputs,
                                   void* const* outputs2, size_t count, mrr_dtype in,
                                   mrr_dtype accum, int nranks, int rank, void* stream);

/* --------------------------------------------------------------------------
 * LL-packet allpair allreduce (commit history: allreduce_allpair_packet fix;
 * default flag buffer entry).
 *
 * A packet is 8 bytes: payload word k of a rank's buffer (bytes [4k, 4k+4),
 * little-endian, bytes past the end read as zero) in the low 32 bits and a
 * 32-bit flag in the high 32 bits.  npkt = ceil(count * elem_size / 4).
 *
 * Each call takes F = (flag slot value) + 1, skipping 0 on 32-bit wrap.
 * Workgroup (rank d, block b) packs slice b of inputs[d] and stores the
 * packets into scratch[p][d][*] for every peer p != d (64-bit agent-scope
 * stores); it then polls scratch[d][s][*] of slice b for every s != d until
 * every packet carries F (wavefront-level vote, 64-bit agent-scope loads),
 * sums in rank order 0..nranks-1 -- taking its own contribution straight
 * from inputs[d] -- and writes slice b of outputs[d]; finally it sets every
 * flag slot j of rank d with j % B == b to F.  The inputs are never written.
 *
 * scratch:  device, 8-byte aligned, layout [dst][src][npkt] of uint64 packets,
 *           at least mrr_packet_scratch_bytes() bytes (else MRR_ESCRATCH);
 *           the self slots [d][d] are unused.  Zero it once before first use.
 * flags:    device, nranks * MRR_PKT_FLAG_SLOTS uint32, zero-filled once
 *           before first use (and whenever it is recycled).  Every call leaves
 *           every slot equal to the F it used, so count, geometry and the
 *           algorithm may change between calls without a hang, and graph
 *           replays advance F on the device.  All ranks' slots must hold the
 *           same value.  May be shared with later calls of any packet entry.
 *           Flag wrap: after 2^32 - 1 calls on one flag buffer F returns to
 *           1.  Scratch packets that an earlier, larger call wrote and no
 *           later call rewrote keep their old flags, which the wrapped
 *           sequence reaches again, and a poll could then take such a stale
 *           packet for a new one.  Re-zero the flags and the scratch together
 *           before 2^32 - 1 calls (about 2.4 hours of back-to-back 2 us
 *           calls).
 * inputs / outputs: device, 4-byte aligned (MRR_EALIGN), outputs[k] may be
 *           inputs[k] exactly; other overlaps give MRR_EOVERLAP.
 * dtype:    F32 | F16 | BF16 | FP8_E4M3B15 (output type == input type).
 * accum:    AUTO (= dtype) | F32 | F16 (F16 and FP8 data).
 * max_spins: bound on poll iterations per wavefront; on expiry the kernel
 *           writes MRR_ETIMEDOUT into *dev_err (if dev_err is not NULL; first
 *           error wins) and finishes; outputs are then undefined.  0 = no
 *           bound.  Read *dev_err after synchronising the stream.
 * blocks_per_rank / threads (_ex only): B and the workgroup size; 0 = auto.
 *           B must be in [1, MRR_PKT_FLAG_SLOTS]; threads a multiple of 64 in
 *           [64, 512]; nranks * B workgroups must fit on the GPU at once
 *           (every workgroup waits for its peers), else MRR_EINVAL.
 * Calls that overlap in time on the same scratch or flags race; calls on one
 * stream never overlap.
 * Co-residency is checked against an idle GPU.  Work running at the same time
 * on other streams (an RS/AG call, whose workgroups also hold LDS, or any
 * other kernel) only delays the packet workgroups that do not fit until it
 * drains.  But two packet calls running at the same time on different
 * streams can each hold workgroups that wait for peers the other keeps off
 * the GPU: order such calls on one stream, or give them a max_spins bound,
 * or set MRR_COOPERATIVE=1 (see mrr_reload_env) to have such launches
 * refused instead.
 * ------------------------------------------------------------------------ */
/* Scratch and flag sizes for the calls above; 0 for an unknown type, nranks
 * outside [1, 32], or a count the entry points refuse as too large. */
size_t mrr_packet_scratch_bytes(size_t count, mrr_dtype dtype, int nranks);
size_t mrr_packet_flag_bytes(int nranks);

mrr_status mrr_allreduce_packet(const void* const* inputs, void* const* outputs, void* scratch,
                                size_t scratch_bytes, uint32_t* flags, size_t count,
                                mrr_dtype dtype, mrr_dtype accum, int nranks,
                                uint32_t max_spins, uint32_t* dev_err, void* stream);

mrr_status mrr_allreduce_packet_ex(const void* const* inputs, void* const* outputs, void* scratch,
                                   size_t scratch_bytes, uint32_t* flags, size_t count,
                                   mrr_dtype dtype, mrr_dtype accum, int nranks,
                                   uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                   int threads, void* stream);

/* --------------------------------------------------------------------------
 * LL-packet allpair allreduce that allocates nothing, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same operation, results and flag protocol as mrr_allreduce_packet, but the
 * scratch and the flag slots live in a workspace the library owns: one
 * statically sized device array per GPU, MRR_NOALLOC_SCRATCH_BYTES of packet
 * scratch plus the flag slots of 32 ranks (about 32.1 MiB in all), held on
 * every GPU the library runs on until the process ends.  The call allocates
 * and frees nothing.
 *   - A call needs nranks^2 * ceil(count * elem_size / 4) * 8 bytes of packet
 *     scratch (mrr_packet_scratch_bytes); above MRR_NOALLOC_SCRATCH_BYTES it
 *     returns MRR_ESCRATCH and launches nothing.  For example 8 ranks take up
 *     to 256 KiB per rank of f16, 32 ranks up to 16 KiB.
 *   - The first call on each device clears the workspace with a kernel on
 *     `stream`, ahead of its own kernel; it must not be made under stream
 *     capture (MRR_EINVAL, nothing set up).  Later calls may be captured.
 *   - Every call on one GPU shares that GPU's workspace, which keeps the last
 *     call's packets and flags; calls of any rank count, size and type
 *     continue one flag sequence.  Calls that overlap in time on one GPU
 *     (different streams without ordering, or concurrent graphs) race and may
 *     hang until max_spins: order them on one stream.
 *   - The flag sequence wraps after 2^32 - 1 calls; past that a stale packet
 *     could be taken for a new one (see the flag notes above), so a process
 *     making that many calls should use mrr_allreduce_packet with its own
 *     buffers, which it can re-zero.
 * inputs / outputs / dtype / accum / nranks / max_spins / dev_err as for
 * mrr_allreduce_packet; geometry is chosen automatically.
 * ------------------------------------------------------------------------ */
#define MRR_NOALLOC_SCRATCH_BYTES (32u << 20)

mrr_status mrr_allreduce_packet_noalloc(const void* const* inputs, void* const* outputs,
                                        size_t count, mrr_dtype dtype, mrr_dtype accum,
                                        int nranks, uint32_t max_spins, uint32_t* dev_err,
                                        void* stream);

/* --------------------------------------------------------------------------
 * Two-phase packet allreduce: reduce-scatter then all-gather, both in LL
 * packets (the "packet" allreduce the commit log lists beside allpair, in
 * the entry adding accumDtype; its structure is not on the pages, so this is
 * the RS/AG partition carried by packets).  The index space is split as for
 * RS/AG: chunk c = elements [c*C, (c+1)*C), C = roundup(ceil(count/N),
 * 16/elem_size), i.e. cw = C*elem_size/4 payload words per chunk.
 *   1. rank d sends chunk c of its input to rank c: rs[c][d][k] (c != d);
 *   2. rank c waits for rs[c][s] (s != c), sums chunk c in rank order with
 *      its own chunk read from its input, writes it to outputs[c] and sends
 *      it to every peer: ag[p][c][k] (p != c);
 *   3. rank p waits for ag[p][s] (s != p) and writes chunk s of outputs[p].
 * Every packet carries the call's flag F (same flag contract, flag buffer
 * and time-out behaviour as mrr_allreduce_packet; one flag buffer may serve
 * both packet entry points).  Per rank it moves about 10*S bytes against
 * (3 + 4(N-1))*S for allpair.
 * scratch: 8-byte aligned, mrr_packet_rsag_scratch_bytes() bytes: the rs
 *   region then the ag region, each [dst][src][cw] uint64 packets.  Zero it
 *   once before first use.
 * Other arguments and errors as mrr_allreduce_packet_ex.
 * ------------------------------------------------------------------------ */
/* 0 for an unknown type, nranks outside [1, 32], or a count refused as too large. */
size_t mrr_packet_rsag_scratch_bytes(size_t count, mrr_dtype dtype, int nranks);

mrr_status mrr_allreduce_packet_rsag(const void* const* inputs, void* const* outputs,
                                     void* scratch, size_t scratch_bytes, uint32_t* flags,
                                     size_t count, mrr_dtype dtype, mrr_dtype accum, int nranks,
                                     uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                     int threads, void* stream);

/* --------------------------------------------------------------------------
 * Full-mesh allreduce (commit history: the entries adding accumDtype and
 * ROCm FP8 E4M3B15 support name a "fullmesh" allreduce beside the allpair
 * packet one; its steps are not on the pages, so this is the plain reading of
 * the name: every rank talks to every peer directly, by writes only, in plain
 * data rather than LL packets, each delivery signalled by a flag written
 * after it).  Chunks as the two-phase packet allreduce: C = roundup(ceil(count
 * / N), 16 / elem_size) elements, chunk c = elements [c*C, min((c+1)*C,
 * count)).  Workgroup (rank d, block b) takes slice b of every chunk:
 *   1. it writes slice b of chunk c of inputs[d] into inbox [c][d] of the
 *      scratch, for every peer c != d;
 *   2. it sets semaphore [c][d][b] = (uint64)F << 32 for every peer c != d
 *      (agent-scope release after the data);
 *   3. it waits until semaphore [d][s][b] carries F for every peer s
 *      (agent-scope acquire; bounded by max_spins), sums slice b of chunk d
 *      in rank order 0..nranks-1 -- its own part from inputs[d], the others
 *      from inbox [d][s] -- and writes it to chunk d of every outputs[k];
 *   4. it sets the flag slots j of rank d with j % B == b to F.
 * Per call it moves about (4N - 2) * S bytes (S = count * elem_size), against
 * 2N * S for RS/AG.
 * scratch: device, 16-byte aligned, mrr_fullmesh_scratch_bytes() bytes: the
 *   semaphores, N * N * MRR_PKT_FLAG_SLOTS uint64 [dst][src][slot], then the
 *   inboxes, N * N * C * elem_size bytes [dst][src][chunk].  Zero it once
 *   before first use (a semaphore must never hold a flag the sequence has
 *   not reached).  It may be shared with the packet entry points and the same
 *   flag buffer.
 * inputs / outputs: 16-byte aligned (MRR_EALIGN); outputs[k] may be
 *   inputs[k] exactly.  flags, dtype, accum, max_spins, dev_err,
 *   blocks_per_rank, threads and errors as mrr_allreduce_packet_ex (the
 *   auto geometry covers one 16-byte vector per lane per chunk).
 * ------------------------------------------------------------------------ */
size_t mrr_fullmesh_scratch_bytes(size_t count, mrr_dtype dtype, int nranks);

mrr_status mrr_allreduce_fullmesh(const void* const* inputs, void* const* outputs, void* scratch,
                                  size_t scratch_bytes, uint32_t* flags, size_t count,
                                  mrr_dtype dtype, mrr_dtype accum, int nranks,
                                  uint32_t max_spins, uint32_t* dev_err, int blocks_per_rank,
                                  int threads, void* stream);

/* --------------------------------------------------------------------------
 * One-call allreduce with algorithm selection ("Support 2 ranks in
 * AllreduceRsAgZeroCopy", section "why": selectors pick RS/AG zero-copy above
 * a message size and packets below it; section "what changed": rank counts
 * the RS/AG kernel does not cover could fall back to another algorithm).
 *
 * out type == dtype; accum as for the packet path (AUTO = dtype).
 *   - nranks in {2,4,8,16,32}, scratch and flags non-NULL, scratch_bytes >=
 *     mrr_packet_scratch_bytes(), count * elem_size <= packet_max_bytes and
 *     the (dtype, accum) pair has a packet kernel: the LL-packet allpair
 *     (same contract as mrr_allreduce_packet).
 *   - otherwise RS/AG over all chunks; a rank count in [1, 32] without a
 *     compiled kernel (1, 3, 5, 6, 7, 9, ...) runs the runtime-N RS/AG kernel,
 *     with the same results (sum in rank order 0..N-1).
 * MRR_PACKET_MAX_BYTES_ONE_GPU is the crossover measured on one MI355X (see
 * its definition); callers sharing work over several GPUs pick their own.
 * Errors as for the chosen path; nranks outside [1, 32] -> MRR_EUNSUPPORTED.
 * ------------------------------------------------------------------------ */
mrr_status mrr_allreduce(const void* const* inputs, void* const* outputs, size_t count,
                         mrr_dtype dtype, mrr_dtype accum, int nranks, void* scratch,
                         size_t scratch_bytes, uint32_t* flags, size_t packet_max_bytes,
                         uint32_t max_spins, uint32_t* dev_err, void* stream);

/* Receive step alone: for every k < npkts, wait until in_pkts[s][k] carries
 * flag_in for every s, sum the payload elements (4 / elem_size per word) in
 * rank order with accumulator accum, round to dtype and store
 * out_pkts[k] = (flag_out << 32) | word with a 64-bit agent-scope store.
 * in_pkts: host array of nranks device pointers (8-byte aligned); out_pkts
 * must not overlap them.  max_spins / dev_err as above.  No co-residency is
 * needed (the producers are outside the call), so any npkts works. */
mrr_status mrr_packet_reduce(const uint64_t* const* in_pkts, uint64_t* out_pkts, size_t npkts,
                             mrr_dtype dtype, mrr_dtype accum, int nranks, uint32_t flag_in,
                             uint32_t flag_out, uint32_t max_spins, uint32_t* dev_err,
                             void* stream);

/* pkts[k] = (flag << 32) | word_k(src) for k < ceil(nbytes / 4) (64-bit
 * agent-scope stores).  src: 4-byte aligned device buffer of nbytes bytes;
 * pkts: 8-byte aligned. */
mrr_status mrr_pack(const void* src, uint64_t* pkts, size_t nbytes, uint32_t flag, void* stream);
/* Writes the nbytes payload bytes of pkts into dst (4-byte aligned). */
mrr_status mrr_unpack(const uint64_t* pkts, void* dst, size_t nbytes, void* stream);

/* --------------------------------------------------------------------------
 * FP8 E4M3B15 codec (commit history: fp8_e4m3b15 datatype entry).
 * Decode is exact; encode rounds once, to nearest-even, saturating at
 * +-0.9375.  n elements; pointers aligned to their element size (MRR_EALIGN),
 * 16-byte alignment selects the vector kernels.  In and out must not overlap
 * (MRR_EOVERLAP).
 * ------------------------------------------------------------------------ */
mrr_status mrr_fp8b15_to_f16(const uint8_t* in, uint16_t* out, size_t n, void* stream);
mrr_status mrr_fp8b15_to_f32(const uint8_t* in, float* out, size_t n, void* stream);
mrr_status mrr_f16_to_fp8b15(const uint16_t* in, uint8_t* out, size_t n, void* stream);
mrr_status mrr_f32_to_fp8b15(const float* in, uint8_t* out, size_t n, void* stream);

/* --------------------------------------------------------------------------
 * Copy-kernel calibration (measurement aid, not part of the reduction).
 * Copies nbytes from src to dst with the launch scheme of the RS/AG kernels
 * (one single-wave workgroup per tile, residency capped through an unused
 * LDS reservation, non-temporal 16-byte loads and stores): the same 1:1 mix
 * of streaming reads and writes as a reduction, without its arithmetic, so
 * its bandwidth is the practical ceiling a reduction is read against.
 * src and dst: device pointers, 16-byte aligned (MRR_EALIGN), ranges
 * disjoint (MRR_EOVERLAP); nbytes == 0 launches nothing; nbytes over 1 TiB
 * -> MRR_EINVAL.  Stream-ordered and asynchronous; allocates nothing.
 * ------------------------------------------------------------------------ */
mrr_status mrr_stream_copy(const void* src, void* dst, size_t nbytes, void* stream);

/* --------------------------------------------------------------------------
 * HBM placement of the simulated rank buffers (one GPU holds all N).
 *
 * When the N same-size rank buffers of one side (inputs, or outputs) are
 * carved from one device allocation, consecutive buffers should be
 * mrr_rank_buffer_pitch(bytes, nranks) bytes apart: bytes rounded up to
 * 4 KiB plus a stagger of 4 KiB (nranks < 16) or 3 KiB (nranks >= 16); from
 * 4 ranks up, when the rounded size is an odd multiple of 128 MiB, 5 KiB and
 * 8 KiB instead (8 x 128 MiB bf16: 0.74 -> 0.80 of the HBM peak).
 * Buffers spaced by a large power of two put the 2N equal-offset streams of
 * a reduction on the same DRAM channels; the stagger spreads them.  Measured
 * on MI355X with the RS/AG kernel, 8 x 64 MiB f16: 186.8 us with one
 * allocation per buffer, 180-181 us at this pitch, 205 us at an exact 64 MiB
 * pitch.  At 16 and 32 ranks (64 and 256 MiB each, mean of three runs) a
 * 3 KiB stagger gives 5.62 / 5.47 TB/s (N=16) and 5.28 / 5.10 TB/s (N=32),
 * against 5.31 / 5.55 and 5.17 / 5.13 at 2 KiB and 4.97-5.38 at 4 KiB.
 * Advisory only: every entry point accepts any placement.  Returns 0 for
 * bytes == 0 or nranks < 1.
 * ------------------------------------------------------------------------ */
size_t mrr_rank_buffer_pitch(size_t bytes_per_rank, int nranks);

/* --------------------------------------------------------------------------
 * Environment overrides (diagnostics and tuning; none changes a result).
 *   MRR_LOG=1          one stderr line per refused call
 *   MRR_MAX_GRID=<g>   at most g workgroups per RS/AG, codec or copy launch
 *                      (each then walks several tiles)
 *   MRR_LDS_CAP=0      persistent grids without the LDS reservation that caps
 *                      residency (frees the LDS for concurrent kernels)
 *   MRR_RSAG_WPC, MRR_RSAG_ANY_M, MRR_RSAG_SMALL=0, MRR_CODEC_U, MRR_CODEC_WPC
 *                      replace entries of the measured launch tables
 *   MRR_COOPERATIVE=1  launch the kernels whose workgroups wait for each other
 *                      (allpair, two-phase packets, full mesh) with
 *                      hipLaunchCooperativeKernel: a grid that cannot be
 *                      resident at once (for instance behind work on other
 *                      streams) is then refused at launch (MRR_EHIP) instead
 *                      of waiting; costs about 15 us per eager call on MI355X
 * They are read once, when the library is loaded.  mrr_reload_env() reads
 * them again (for tests and tuning sweeps that change them in-process); calls
 * running on other threads meanwhile see either the old or the new values.
 * ------------------------------------------------------------------------ */
void mrr_reload_env(void);

/* Static description of a status code (never NULL). */
const char* mrr_status_string(mrr_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mrr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MRR_H */
