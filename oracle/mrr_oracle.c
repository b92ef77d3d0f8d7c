/*
 * mrr_oracle.c -- plain CPU oracle for the N-rank allreduce reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library libmrr) never calls it, includes nothing from it, and shares no
 * code, header, table or constant with it.
 *
 * What it computes (the pages it follows):
 *   - "Support 2 ranks in AllreduceRsAgZeroCopy" (MSCCL++ PR #948), section
 *     "what changed": rank r reduces chunk r of every rank's input and writes
 *     the result into every rank's output (reduce-scatter then all-gather,
 *     no scratch).  Because the reduction is elementwise, the value of every
 *     output element is a plain sum over ranks; the chunk partition only
 *     decides who computes it.  The oracle writes that plain definition out:
 *     out[k][i] = narrow_out( x_0[i] (+) x_1[i] (+) ... (+) x_{N-1}[i] ),
 *     summed sequentially in rank order 0..N-1, starting from x_0.
 *   - MSCCL++ commit history, entry adding the fp8_e4m3b15 datatype and the
 *     accumDtype parameter: accumulation runs in a chosen precision (FP32,
 *     FP16, or the input type itself, which is what AUTO resolves to).
 *     With accumulation type A every partial sum is rounded to A.
 *   - Same entry: FP8 E4M3B15 has 4 exponent bits, 3 mantissa bits, bias 15,
 *     and its largest finite value is 0.9375.  Exponent field 15 therefore
 *     holds no finite value; it is read as IEEE-style inf (m=0) / NaN (m!=0).
 *   - "Support 2 ranks in AllreduceRsAgZeroCopy", section "why": the pages
 *     also reduce OCP fp8_e4m3fn data (4 exponent bits, bias 7, 3 mantissa
 *     bits, no infinity, S.1111.111 = NaN, largest finite 448); its rounding
 *     is taken to saturate like E4M3B15's.
 *   - MSCCL++ commit history, entry fixing allreduce_allpair_packet: each rank
 *     sends its data as low-latency packets to every peer, the receiver waits
 *     for the packet flag, reduces and writes back; the input buffer is never
 *     overwritten.  A packet is 8 bytes: 4 payload bytes (low word) and a
 *     32-bit flag (high word).
 *
 * How it rounds (obviously-correct, table driven, no bit tricks):
 *   every target format's non-negative finite values are listed in a sorted
 *   table whose index equals the format's code; a value is rounded by finding
 *   its two neighbours and comparing 2*x with their sum (an exact comparison
 *   in double for every input used here), ties going to the even code.
 *   For f16 and bf16 one extra entry holds the first power of two above the
 *   largest finite value, standing for infinity, so IEEE overflow-to-inf
 *   falls out of the same search.  FP8 E4M3B15 saturates instead.
 *
 * Compile: gcc -O2 -std=c11 -fPIC -shared (no fast-math, no FMA contraction).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- type ids, private to the oracle (the Python wrapper maps names) ---- */
enum { ORC_F32 = 1, ORC_F16 = 2, ORC_BF16 = 3, ORC_FP8 = 4, ORC_FP8FN = 5 };

static int orc_size(int t) {
  switch (t) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8: return 1;
    case ORC_FP8FN: return 1;
    default: return 0;
  }
}

/* ---------------------------------------------------------------------- */
/* Decoding: code -> exact value (double), from each format's definition.  */
/* ---------------------------------------------------------------------- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_value(uint16_t c) {
  int s = c >> 15, e = (c >> 10) & 0x1F, m = c & 0x3FF;
  double v;
  if (e == 0x1F) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);              /* m/1024 * 2^-14 */
  else v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -v : v;
}

/* bfloat16: the upper half of IEEE binary32 -- 1 sign, 8 exponent (bias 127),
 * 7 fraction bits. */
static double bf16_value(uint16_t c) {
  int s = c >> 15, e = (c >> 7) & 0xFF, m = c & 0x7F;
  double v;
  if (e == 0xFF) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -133);             /* m/128 * 2^-126 */
  else v = ldexp(1.0 + (double)m / 128.0, e - 127);
  return s ? -v : v;
}

/* FP8 E4M3B15: 1 sign, 4 exponent (bias 15), 3 fraction bits; e=0 is
 * subnormal (m/8 * 2^-14); e=15 is inf (m=0) or NaN (m!=0), the reading that
 * makes 0.9375 the largest finite value. */
static double fp8_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 0xF) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m / 8.0, -14);
  else v = ldexp(1.0 + (double)m / 8.0, e - 15);
  return s ? -v : v;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; e=0 is
 * subnormal (m/8 * 2^-6); no infinity; e=15 with m=7 is NaN, so the largest
 * finite value is 2^8 * 1.75 = 448. */
static double fp8fn_value(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
  double v;
  if (e == 0xF && m == 7) v = NAN;
  else if (e == 0) v = ldexp((double)m / 8.0, -6);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* IEEE binary32 from its bits, by the same field definition. */
static double f32_value(uint32_t c) {
  int s = c >> 31, e = (c >> 23) & 0xFF;
  uint32_t m = c & 0x7FFFFF;
  double v;
  if (e == 0xFF) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -149);
  else v = ldexp(1.0 + (double)m / 8388608.0, e - 127);
  return s ? -v : v;
}

/* ---------------------------------------------------------------------- */
/* Tables of non-negative finite values, index == code.                    */
/* ---------------------------------------------------------------------- */
#define F16_NFIN 0x7C00   /* codes 0x0000..0x7BFF are the finite >= 0 values */
#define BF16_NFIN 0x7F80  /* codes 0x0000..0x7F7F */
#define FP8_NFIN 0x78     /* codes 0x00..0x77 */
#define FP8FN_NFIN 0x7F   /* codes 0x00..0x7E */

static double f16_tab[F16_NFIN + 1];   /* + sentinel 2^16 standing for inf  */
static double bf16_tab[BF16_NFIN + 1]; /* + sentinel 2^128 standing for inf */
static double fp8_tab[FP8_NFIN];
static double fp8fn_tab[FP8FN_NFIN];
static int tabs_ready = 0;

static void build_tables(void) {
  if (tabs_ready) return;
  for (int c = 0; c < F16_NFIN; ++c) f16_tab[c] = f16_value((uint16_t)c);
  f16_tab[F16_NFIN] = ldexp(1.0, 16);
  for (int c = 0; c < BF16_NFIN; ++c) bf16_tab[c] = bf16_value((uint16_t)c);
  bf16_tab[BF16_NFIN] = ldexp(1.0, 128);
  for (int c = 0; c < FP8_NFIN; ++c) fp8_tab[c] = fp8_value((uint8_t)c);
  for (int c = 0; c < FP8FN_NFIN; ++c) fp8fn_tab[c] = fp8fn_value((uint8_t)c);
  tabs_ready = 1;
}

/* Index of the table entry nearest to a (a >= 0, tab[0] <= a <= tab[n-1]);
 * ties go to the even index.  2*a and tab[lo]+tab[hi] are exact in double for
 * every table here (neighbouring entries differ in exponent by at most one). */
static int nearest_even(const double* tab, int n, double a) {
  int lo = 0, hi = n - 1;
  while (hi - lo > 1) { /* invariant: tab[lo] <= a <= tab[hi] */
    int mid = lo + (hi - lo) / 2;
    if (tab[mid] <= a) lo = mid; else hi = mid;
  }
  if (tab[lo] == a) return lo;
  if (tab[hi] == a) return hi;
  double twice = 2.0 * a, mids = tab[lo] + tab[hi];
  if (twice < mids) return lo;
  if (twice > mids) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

/* Round-to-nearest-even into binary16; overflow gives +-inf (IEEE). */
static uint16_t narrow_f16(double x) {
  if (isnan(x)) return (uint16_t)((signbit(x) ? 0x8000 : 0) | 0x7E00);
  uint16_t s = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a >= f16_tab[F16_NFIN]) return s | 0x7C00;
  return s | (uint16_t)nearest_even(f16_tab, F16_NFIN + 1, a);
}

/* Round-to-nearest-even into bfloat16; overflow gives +-inf. */
static uint16_t narrow_bf16(double x) {
  if (isnan(x)) return (uint16_t)((signbit(x) ? 0x8000 : 0) | 0x7FC0);
  uint16_t s = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a >= bf16_tab[BF16_NFIN]) return s | 0x7F80;
  return s | (uint16_t)nearest_even(bf16_tab, BF16_NFIN + 1, a);
}

/* Round-to-nearest-even into FP8 E4M3B15, saturating at +-0.9375 (also for
 * +-inf); NaN gives the code 0x7F with the input's sign. */
static uint8_t narrow_fp8(double x) {
  if (isnan(x)) return (uint8_t)((signbit(x) ? 0x80 : 0) | 0x7F);
  uint8_t s = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= fp8_tab[FP8_NFIN - 1]) return s | (uint8_t)(FP8_NFIN - 1);
  return s | (uint8_t)nearest_even(fp8_tab, FP8_NFIN, a);
}

/* Round-to-nearest-even into OCP FP8 E4M3FN, saturating at +-448 (also for
 * +-inf); NaN gives 0x7F with the input's sign. */
static uint8_t narrow_fp8fn(double x) {
  if (isnan(x)) return (uint8_t)((signbit(x) ? 0x80 : 0) | 0x7F);
  uint8_t s = signbit(x) ? 0x80 : 0;
  double a = fabs(x);
  if (a >= fp8fn_tab[FP8FN_NFIN - 1]) return s | (uint8_t)(FP8FN_NFIN - 1);
  return s | (uint8_t)nearest_even(fp8fn_tab, FP8FN_NFIN, a);
}

/* Round-to-nearest-even into binary32: the C cast does exactly this on IEEE
 * hosts (FLT_EVAL_METHOD 0); used only for already-representable values
 * and for the f32 accumulator, whose adds are IEEE binary32 adds. */
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ---------------------------------------------------------------------- */
/* Element access on raw buffers.                                          */
/* ---------------------------------------------------------------------- */
static double load_value(const void* p, size_t i, int t) {
  const uint8_t* b = (const uint8_t*)p + i * (size_t)orc_size(t);
  switch (t) {
    case ORC_F32: { uint32_t u; memcpy(&u, b, 4); return f32_value(u); }
    case ORC_F16: { uint16_t u; memcpy(&u, b, 2); return f16_value(u); }
    case ORC_BF16: { uint16_t u; memcpy(&u, b, 2); return bf16_value(u); }
    case ORC_FP8: return fp8_value(b[0]);
    case ORC_FP8FN: return fp8fn_value(b[0]);
  }
  return NAN;
}

/* Writes value v (already a member of type t, or to be rounded into it). */
static void store_value(void* p, size_t i, int t, double v) {
  uint8_t* b = (uint8_t*)p + i * (size_t)orc_size(t);
  switch (t) {
    case ORC_F32: {
      uint32_t u;
      if (isnan(v)) u = (signbit(v) ? 0x80000000u : 0) | 0x7FC00000u;
      else u = f32_bits((float)v);
      memcpy(b, &u, 4);
      break;
    }
    case ORC_F16: { uint16_t u = narrow_f16(v); memcpy(b, &u, 2); break; }
    case ORC_BF16: { uint16_t u = narrow_bf16(v); memcpy(b, &u, 2); break; }
    case ORC_FP8: b[0] = narrow_fp8(v); break;
    case ORC_FP8FN: b[0] = narrow_fp8fn(v); break;
  }
}

/* Round v into type t and return the rounded value (for native accumulation). */
static double round_to(int t, double v) {
  switch (t) {
    case ORC_F16: return f16_value(narrow_f16(v));
    case ORC_BF16: return bf16_value(narrow_bf16(v));
    case ORC_FP8: return fp8_value(narrow_fp8(v));
    case ORC_FP8FN: return fp8fn_value(narrow_fp8fn(v));
    case ORC_F32: return isnan(v) ? v : (double)(float)v;
  }
  return NAN;
}

/* ---------------------------------------------------------------------- */
/* Public oracle entry points.                                             */
/* ---------------------------------------------------------------------- */

/* Sum of element i over ranks in order 0..N-1 with accumulation type acc,
 * returned as an exact double holding a member of acc. */
static double rank_sum(const void* const* in, size_t i, int tin, int acc, int nranks) {
  if (acc == ORC_F32) {
    /* IEEE binary32 accumulator, first term x_0 (so -0 + -0 stays -0). */
    float a = (float)load_value(in[0], i, tin);
    for (int r = 1; r < nranks; ++r) {
      float x = (float)load_value(in[r], i, tin);
      a = a + x;
    }
    return (double)a;
  }
  /* Native-precision accumulation: every partial sum rounded to acc.  The
   * first term is x_0 rounded into acc (exact whenever tin is narrower).  For
   * f16 and fp8 operands the double sum is exact, so round_to() gives the
   * correctly rounded sum; for bf16 the double sum can round, and rounding a
   * 53-bit result to 8 bits again is innocuous (53 >= 2*8+2). */
  double a = round_to(acc, load_value(in[0], i, tin));
  for (int r = 1; r < nranks; ++r) a = round_to(acc, a + load_value(in[r], i, tin));
  return a;
}

/* Allreduce (RS/AG layout, every chunk): writes every outputs[k], k < nout.
 * Returns 0, or -1 on a bad type id. */
int orc_allreduce(const void* const* inputs, void* const* outputs, size_t count,
                  int tin, int tacc, int tout, int nranks, int nout) {
  build_tables();
  if (!orc_size(tin) || !orc_size(tacc) || !orc_size(tout) || nranks < 1) return -1;
  for (size_t i = 0; i < count; ++i) {
    double s = rank_sum(inputs, i, tin, tacc, nranks);
    for (int k = 0; k < nout; ++k) store_value(outputs[k], i, tout, s);
  }
  return 0;
}

/* Elementwise codec: converts n elements of type tin into type tout, by
 * decoding to the exact value and rounding once (RNE; FP8 saturates). */
int orc_convert(const void* in, void* out, size_t n, int tin, int tout) {
  build_tables();
  if (!orc_size(tin) || !orc_size(tout)) return -1;
  for (size_t i = 0; i < n; ++i) store_value(out, i, tout, load_value(in, i, tin));
  return 0;
}

/* Rounds n doubles into type t (bits written to out).  Used by the pins. */
int orc_narrow_f64(const double* in, void* out, size_t n, int t) {
  build_tables();
  if (!orc_size(t)) return -1;
  for (size_t i = 0; i < n; ++i) store_value(out, i, t, in[i]);
  return 0;
}

/* Decodes n codes of type t into doubles.  Used by the pins. */
int orc_widen_f64(const void* in, double* out, size_t n, int t) {
  build_tables();
  if (!orc_size(t)) return -1;
  for (size_t i = 0; i < n; ++i) out[i] = load_value(in, i, t);
  return 0;
}

/* ---- low-latency packets ---------------------------------------------- */

/* Payload word k of a byte buffer: bytes [4k, 4k+4), little-endian, the bytes
 * past nbytes read as zero. */
static uint32_t word_at(const uint8_t* src, size_t nbytes, size_t k) {
  uint32_t w = 0;
  for (int b = 0; b < 4; ++b) {
    size_t at = 4 * k + (size_t)b;
    uint32_t byte = at < nbytes ? src[at] : 0;
    w |= byte << (8 * b);
  }
  return w;
}

static uint64_t make_packet(uint32_t word, uint32_t flag) {
  return ((uint64_t)flag << 32) | (uint64_t)word;
}

/* pkts[k] = flag:word_k for k < ceil(nbytes/4). */
void orc_pack(const uint8_t* src, size_t nbytes, uint32_t flag, uint64_t* pkts) {
  size_t n = (nbytes + 3) / 4;
  for (size_t k = 0; k < n; ++k) pkts[k] = make_packet(word_at(src, nbytes, k), flag);
}

/* Inverse of orc_pack: writes exactly nbytes payload bytes. */
void orc_unpack(const uint64_t* pkts, size_t nbytes, uint8_t* dst) {
  for (size_t at = 0; at < nbytes; ++at) {
    uint32_t w = (uint32_t)(pkts[at / 4] & 0xFFFFFFFFu);
    dst[at] = (uint8_t)(w >> (8 * (at % 4)));
  }
}

/* The flag a packet allreduce call stamps when every flag slot holds `prev`:
 * one more, skipping 0 on 32-bit wrap (0 marks an empty slot). */
uint32_t orc_next_flag(uint32_t prev) {
  uint32_t f = prev + 1u;
  return f == 0 ? 1u : f;
}

/* Expected state after one allpair packet allreduce with flag F:
 *   scratch[(d*N + s)*npkt + k] = pack(word_k(in[s]), F) for every d != s
 *   (self slots d == s are left as they were), and outputs as orc_allreduce
 *   with out type == in type.  scratch must hold N*N*npkt packets. */
int orc_allreduce_packet(const void* const* inputs, void* const* outputs,
                         uint64_t* scratch, size_t count, int t, int tacc,
                         int nranks, uint32_t flag) {
  build_tables();
  int e = orc_size(t);
  if (!e || !orc_size(tacc)) return -1;
  size_t nbytes = count * (size_t)e, npkt = (nbytes + 3) / 4;
  for (int s = 0; s < nranks; ++s)
    for (int d = 0; d < nranks; ++d) {
      if (d == s) continue;
      uint64_t* dst = scratch + ((size_t)d * nranks + s) * npkt;
      orc_pack((const uint8_t*)inputs[s], nbytes, flag, dst);
    }
  return orc_allreduce(inputs, outputs, count, t, tacc, t, nranks, nranks);
}

/* Two-phase packet allreduce (the "packet" variant: reduce-scatter then
 * all-gather, both in packets) with flag F.  The index space is split into N
 * chunks of C = roundup(ceil(count/N), 16/e) elements, i.e. cw = C*e/4
 * payload words; chunk c's words are k = 0 .. words(c)-1 where words(c) is
 * what remains of ceil(count*e/4) after c*cw (none for an empty chunk).
 * Expected state after the call, scratch = two regions of N*N*cw packets:
 *   phase 1: rs[(c*N + d)*cw + k] = pack(word c*cw + k of in[d], F), c != d
 *   phase 2: ag[(p*N + c)*cw + k] = pack(word c*cw + k of the sum, F), p != c
 * (other slots untouched), and every output equals orc_allreduce's. */
int orc_allreduce_packet_rsag(const void* const* inputs, void* const* outputs,
                              uint64_t* scratch, size_t count, int t, int tacc, int nranks,
                              uint32_t flag) {
  build_tables();
  int e = orc_size(t);
  if (!e || !orc_size(tacc) || nranks < 1) return -1;
  size_t nbytes = count * (size_t)e, nwords = (nbytes + 3) / 4;
  size_t per = (count + (size_t)nranks - 1) / (size_t)nranks;
  size_t vw = 16 / (size_t)e;
  size_t chunk = (per + vw - 1) / vw * vw;
  size_t cw = chunk * (size_t)e / 4;
  int rc = orc_allreduce(inputs, outputs, count, t, tacc, t, nranks, nranks);
  if (rc) return rc;
  uint64_t* rs = scratch;
  uint64_t* ag = scratch + (size_t)nranks * nranks * cw;
  for (int c = 0; c < nranks; ++c) {
    for (size_t k = 0; k < cw; ++k) {
      size_t w = (size_t)c * cw + k;
      if (w >= nwords) break;
      for (int d = 0; d < nranks; ++d) {
        if (d == c) continue;
        rs[((size_t)c * nranks + d) * cw + k] =
            make_packet(word_at((const uint8_t*)inputs[d], nbytes, w), flag);
        ag[((size_t)d * nranks + c) * cw + k] =
            make_packet(word_at((const uint8_t*)outputs[0], nbytes, w), flag);
      }
    }
  }
  return 0;
}

/* Receive step alone: every input packet must carry flag_in (else the call
 * would wait forever; returns -2 without writing).  Each payload word holds
 * 4/e elements, summed over ranks in order with accumulation tacc, rounded to
 * t and repacked with flag_out. */
int orc_packet_reduce(const uint64_t* const* in_pkts, uint64_t* out_pkts, size_t npkts,
                      int t, int tacc, int nranks, uint32_t flag_in, uint32_t flag_out) {
  build_tables();
  int e = orc_size(t);
  if (!e || !orc_size(tacc) || nranks < 1 || nranks > 64) return -1;
  for (int r = 0; r < nranks; ++r)
    for (size_t k = 0; k < npkts; ++k)
      if ((uint32_t)(in_pkts[r][k] >> 32) != flag_in) return -2;
  int per = 4 / e;
  const void* lanes[64];
  uint8_t words[64][4];
  for (int r = 0; r < nranks; ++r) lanes[r] = words[r];
  for (size_t k = 0; k < npkts; ++k) {
    for (int r = 0; r < nranks; ++r) {
      uint32_t w = (uint32_t)(in_pkts[r][k] & 0xFFFFFFFFu);
      for (int b = 0; b < 4; ++b) words[r][b] = (uint8_t)(w >> (8 * b));
    }
    uint8_t res[4];
    for (int j = 0; j < per; ++j) {
      const void* elems[64];
      for (int r = 0; r < nranks; ++r) elems[r] = (const uint8_t*)lanes[r] + j * e;
      double s = rank_sum(elems, 0, t, tacc, nranks);
      store_value(res + j * e, 0, t, s);
    }
    uint32_t w = (uint32_t)res[0] | ((uint32_t)res[1] << 8) | ((uint32_t)res[2] << 16) |
                 ((uint32_t)res[3] << 24);
    out_pkts[k] = make_packet(w, flag_out);
  }
  return 0;
}

/* Full-mesh allreduce (the commit history names a "fullmesh" allreduce beside
 * the allpair packet one, in the entries adding accumDtype and ROCm FP8
 * support; its steps are not on the pages, so this follows the plain reading
 * of the name: every rank exchanges data directly with every peer, by writes
 * only, in plain data rather than LL packets, with a flag written after the
 * data to signal it):
 *   1. rank d writes chunk c of its input into inbox [c][d] of the scratch,
 *      for every peer c != d;
 *   2. it then sets, for every peer c != d and block b < nblocks, semaphore
 *      [c][d][b] to the call's flag F (the flag in the high 32 bits, as in a
 *      packet, the low 32 bits zero);
 *   3. rank c, once the semaphores from every peer carry F, sums chunk c in
 *      rank order (its own chunk from its input, the others from its inbox)
 *      and writes the result into chunk c of every rank's output.
 * Chunks as the two-phase packet variant: C = roundup(ceil(count/N), 16/e)
 * elements, chunk c = elements [c*C, min((c+1)*C, count)).
 * Expected state after one call with flag F, in a scratch image laid out as
 *   semaphores: N*N*1024 uint64, [dst][src][slot]
 *   inboxes:    N*N*C*e bytes, [dst][src][byte of chunk]
 * the semaphore slots b < nblocks of every pair dst != src hold F << 32, the
 * inbox bytes of every element of chunk dst below count hold that element of
 * input src (dst != src), every other byte of the image keeps its previous
 * value, and every output equals orc_allreduce's. */
int orc_allreduce_fullmesh(const void* const* inputs, void* const* outputs, uint8_t* scratch,
                           size_t count, int t, int tacc, int nranks, int nblocks,
                           uint32_t flag) {
  build_tables();
  int e = orc_size(t);
  if (!e || !orc_size(tacc) || nranks < 1 || nblocks < 1 || nblocks > 1024) return -1;
  size_t per = (count + (size_t)nranks - 1) / (size_t)nranks;
  size_t vw = 16 / (size_t)e;
  size_t chunk = (per + vw - 1) / vw * vw;
  size_t n = (size_t)nranks;
  uint64_t* sem = (uint64_t*)scratch;
  uint8_t* inbox = scratch + n * n * 1024 * sizeof(uint64_t);
  for (size_t dst = 0; dst < n; ++dst)
    for (size_t src = 0; src < n; ++src) {
      if (dst == src) continue;
      for (int b = 0; b < nblocks; ++b) sem[(dst * n + src) * 1024 + (size_t)b] = (uint64_t)flag << 32;
      uint8_t* slot = inbox + (dst * n + src) * chunk * (size_t)e;
      const uint8_t* in = (const uint8_t*)inputs[src];
      for (size_t j = 0; j < chunk; ++j) {
        size_t i = dst * chunk + j;
        if (i >= count) break;
        memcpy(slot + j * (size_t)e, in + i * (size_t)e, (size_t)e);
      }
    }
  return orc_allreduce(inputs, outputs, count, t, tacc, t, nranks, nranks);
}
