/* A plain C client of libmrr: uses only include/mrr.h, the HIP runtime's C
 * API and raw device pointers (no Python, no torch).  Exercises the RS/AG
 * entry point at a compiled rank count, the size-based dispatcher at a rank
 * count without a compiled kernel, two LL-packet calls on one flag buffer and
 * a refused call, and checks every output against sums computed here.  Data
 * are small integers, so every sum is exact in any order and must match
 * exactly.  Prints "c client ok" and exits 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

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

int main(void) {
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
