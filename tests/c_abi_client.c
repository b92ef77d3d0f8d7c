/* A plain C client of libmrr: uses only include/mrr.h, the HIP runtime's C
 * API and raw device pointers (no Python, no torch).  Exercises the RS/AG
 * entry point at a compiled rank count, the size-based dispatcher at a rank
 * count without a compiled kernel, two LL-packet calls on one flag buffer and
 * a refused call, and checks every output against sums computed here.  Data
 * are small integers, so every sum is exact in any order and must match
 * exactly.  Prints "c client ok" and exits 0 on success.
 *
 * With --timing it instead measures small calls from C, without Python in
 * the way: per call, the host time to issue K calls back to back, and the
 * GPU time of the same K eager calls between two HIP events on the stream.
 * One JSON line per call shape. */
#define _POSIX_C_SOURCE 199309L
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "mrr.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    if ((x) != hipSuccess) {                                                   \
      fprintf(stderr, "%s:%d HIP call failed\n", __FILE__, __LINE__);         \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

static int check_status(mrr_status st, mrr_status want, const char* what) {
  if (st != want) {
    fprintf(stderr, "%s: %s (wanted %s)\n", what, mrr_status_string(st), mrr_status_string(want));
    return 1;
  }
  return 0;
}

/* Reduces n f32 buffers of `count` elements (rank r holds (r + 1) * (i % 7))
 * with `call` and checks every output equals n(n+1)/2 * (i % 7). */
static int run_f32(int n, size_t count, int use_dispatch) {
  void* in[32];
  void* out[32];
  float* host = (float*)malloc(count * sizeof(float));
  int bad = 0;
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipMalloc(&in[r], count * sizeof(float)));
    HIP_OK(hipMalloc(&out[r], count * sizeof(float)));
    for (size_t i = 0; i < count; ++i) host[i] = (float)((r + 1) * (int)(i % 7));
    HIP_OK(hipMemcpy(in[r], host, count * sizeof(float), hipMemcpyHostToDevice));
  }
  mrr_status st = use_dispatch
      ? mrr_allreduce((const void* const*)in, out, count, MRR_F32, MRR_F32, n, NULL, 0, NULL, 0,
                      0, NULL, NULL)
      : mrr_allreduce_rsag((const void* const*)in, out, count, MRR_F32, n, NULL);
  bad |= check_status(st, MRR_OK, use_dispatch ? "mrr_allreduce" : "mrr_allreduce_rsag");
  HIP_OK(hipDeviceSynchronize());
  const float scale = (float)(n * (n + 1) / 2);
  for (int k = 0; k < n && !bad; ++k) {
    HIP_OK(hipMemcpy(host, out[k], count * sizeof(float), hipMemcpyDeviceToHost));
    for (size_t i = 0; i < count; ++i) {
      if (host[i] != scale * (float)(i % 7)) {
        fprintf(stderr, "n=%d out[%d][%zu] = %g, want %g\n", n, k, i, host[i],
                scale * (float)(i % 7));
        bad = 1;
        break;
      }
    }
  }
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipFree(in[r]));
    HIP_OK(hipFree(out[r]));
  }
  free(host);
  return bad;
}

static int run_packets(void) {
  const int n = 4;
  const size_t count = 1000;
  void* in[4];
  void* out[4];
  float host[1000];
  int bad = 0;
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipMalloc(&in[r], count * sizeof(float)));
    HIP_OK(hipMalloc(&out[r], count * sizeof(float)));
    for (size_t i = 0; i < count; ++i) host[i] = (float)(r * 10 + (int)(i % 5));
    HIP_OK(hipMemcpy(in[r], host, sizeof(host), hipMemcpyHostToDevice));
  }
  const size_t sbytes = mrr_packet_scratch_bytes(count, MRR_F32, n);
  const size_t fbytes = mrr_packet_flag_bytes(n);
  void *scratch, *flags, *err;
  HIP_OK(hipMalloc(&scratch, sbytes));
  HIP_OK(hipMalloc(&flags, fbytes));
  HIP_OK(hipMalloc(&err, sizeof(uint32_t)));
  HIP_OK(hipMemset(scratch, 0, sbytes));
  HIP_OK(hipMemset(flags, 0, fbytes));
  HIP_OK(hipMemset(err, 0, sizeof(uint32_t)));
  for (int call = 0; call < 2; ++call)
    bad |= check_status(mrr_allreduce_packet((const void* const*)in, out, scratch, sbytes,
                                             (uint32_t*)flags, count, MRR_F32, MRR_F32, n,
                                             1000000u, (uint32_t*)err, NULL),
                        MRR_OK, "mrr_allreduce_packet");
  HIP_OK(hipDeviceSynchronize());
  uint32_t dev_err = 1;
  HIP_OK(hipMemcpy(&dev_err, err, sizeof(dev_err), hipMemcpyDeviceToHost));
  if (dev_err != 0) {
    fprintf(stderr, "packet device error %u\n", dev_err);
    bad = 1;
  }
  uint32_t* fl = (uint32_t*)malloc(fbytes);
  HIP_OK(hipMemcpy(fl, flags, fbytes, hipMemcpyDeviceToHost));
  for (size_t j = 0; j < fbytes / 4 && !bad; ++j)
    if (fl[j] != 2u) {
      fprintf(stderr, "flag slot %zu = %u, want 2\n", j, fl[j]);
      bad = 1;
    }
  free(fl);
  for (int k = 0; k < n && !bad; ++k) {
    HIP_OK(hipMemcpy(host, out[k], sizeof(host), hipMemcpyDeviceToHost));
    for (size_t i = 0; i < count; ++i)
      if (host[i] != (float)(60 + 4 * (int)(i % 5))) {
        fprintf(stderr, "packet out[%d][%zu] = %g\n", k, i, host[i]);
        bad = 1;
        break;
      }
  }
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipFree(in[r]));
    HIP_OK(hipFree(out[r]));
  }
  HIP_OK(hipFree(scratch));
  HIP_OK(hipFree(flags));
  HIP_OK(hipFree(err));
  return bad;
}

/* ---- --timing ------------------------------------------------------------ */
typedef struct {
  int kind; /* 0 RS/AG, 1 allpair packets, 2 allpair packets (no-alloc), 3 full mesh */
  int n;
  size_t count;
  mrr_dtype t;
  void* in[32];
  void* out[32];
  void* scratch;
  size_t sbytes;
  uint32_t* flags;
  uint32_t* err;
} Shape;

static double now_us(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec * 1e6 + (double)ts.tv_nsec * 1e-3;
}

static mrr_status issue(Shape* s) {
  const void* const* in = (const void* const*)s->in;
  switch (s->kind) {
    case 0: return mrr_allreduce_rsag(in, s->out, s->count, s->t, s->n, NULL);
    case 1:
      return mrr_allreduce_packet(in, s->out, s->scratch, s->sbytes, s->flags, s->count, s->t,
                                  MRR_F32, s->n, 4000000u, s->err, NULL);
    case 2:
      return mrr_allreduce_packet_noalloc(in, s->out, s->count, s->t, MRR_F32, s->n, 4000000u,
                                          s->err, NULL);
    default:
      return mrr_allreduce_fullmesh(in, s->out, s->scratch, s->sbytes, s->flags, s->count, s->t,
                                    MRR_F32, s->n, 4000000u, s->err, 0, 0, NULL);
  }
}

static int time_shape(const char* name, int kind, int n, size_t count, mrr_dtype t, int esize) {
  Shape s;
  memset(&s, 0, sizeof(s));
  s.kind = kind;
  s.n = n;
  s.count = count;
  s.t = t;
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipMalloc(&s.in[r], count * esize));
    HIP_OK(hipMalloc(&s.out[r], count * esize));
    HIP_OK(hipMemset(s.in[r], 0, count * esize));
  }
  if (kind == 1 || kind == 3) {
    s.sbytes = kind == 1 ? mrr_packet_scratch_bytes(count, t, n) : mrr_fullmesh_scratch_bytes(count, t, n);
    HIP_OK(hipMalloc(&s.scratch, s.sbytes));
    HIP_OK(hipMemset(s.scratch, 0, s.sbytes));
    HIP_OK(hipMalloc((void**)&s.flags, mrr_packet_flag_bytes(n)));
    HIP_OK(hipMemset(s.flags, 0, mrr_packet_flag_bytes(n)));
  }
  HIP_OK(hipMalloc((void**)&s.err, 4));
  HIP_OK(hipMemset(s.err, 0, 4));
  const int warm = 50, iters = 2000;
  for (int i = 0; i < warm; ++i)
    if (check_status(issue(&s), MRR_OK, name)) return 1;
  HIP_OK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  HIP_OK(hipEventCreate(&e0));
  HIP_OK(hipEventCreate(&e1));
  HIP_OK(hipEventRecord(e0, NULL));
  const double t0 = now_us();
  for (int i = 0; i < iters; ++i) issue(&s);
  const double t1 = now_us();
  HIP_OK(hipEventRecord(e1, NULL));
  HIP_OK(hipEventSynchronize(e1));
  float ms = 0.f;
  HIP_OK(hipEventElapsedTime(&ms, e0, e1));
  uint32_t err = 0;
  HIP_OK(hipMemcpy(&err, s.err, 4, hipMemcpyDeviceToHost));
  printf("{\"call\": \"%s\", \"nranks\": %d, \"bytes_per_rank\": %zu, \"calls\": %d, "
         "\"host_issue_us_per_call\": %.3f, \"eager_us_per_call\": %.3f, \"device_error\": %u}\n",
         name, n, count * esize, iters, (t1 - t0) / iters, ms * 1000.0 / iters, err);
  HIP_OK(hipEventDestroy(e0));
  HIP_OK(hipEventDestroy(e1));
  for (int r = 0; r < n; ++r) {
    HIP_OK(hipFree(s.in[r]));
    HIP_OK(hipFree(s.out[r]));
  }
  if (s.scratch) HIP_OK(hipFree(s.scratch));
  if (s.flags) HIP_OK(hipFree(s.flags));
  HIP_OK(hipFree(s.err));
  return err != 0;
}

static int timing(void) {
  int bad = 0;
  bad |= time_shape("rsag 2 x 1 MiB bf16", 0, 2, 524288, MRR_BF16, 2);
  bad |= time_shape("rsag 8 x 16 KiB f16", 0, 8, 8192, MRR_F16, 2);
  bad |= time_shape("packet allpair 8 x 16 KiB f16", 1, 8, 8192, MRR_F16, 2);
  bad |= time_shape("packet allpair no-alloc 8 x 16 KiB f16", 2, 8, 8192, MRR_F16, 2);
  bad |= time_shape("full mesh 8 x 16 KiB f16", 3, 8, 8192, MRR_F16, 2);
  return bad;
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "--timing") == 0) return timing();
  int bad = 0;
  bad |= run_f32(8, 100003, 0);  /* compiled kernel */
  bad |= run_f32(3, 50001, 1);   /* runtime-N kernel through the dispatcher */
  bad |= run_packets();
  void* fake[3] = {(void*)0x1000, (void*)0x2000, (void*)0x3000};
  bad |= check_status(mrr_allreduce_rsag((const void* const*)fake, fake, 16, MRR_F32, 3, NULL),
                      MRR_EUNSUPPORTED, "refused rank count");
  if (bad) return 1;
  printf("c client ok (libmrr %d)\n", mrr_version());
  return 0;
}
