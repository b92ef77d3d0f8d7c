"""Host sanitizer run of the C oracle (CPU only): the oracle and a small
driver are built with gcc's AddressSanitizer and UndefinedBehaviorSanitizer,
and the driver calls every oracle entry point on exactly sized heap buffers
(so any read or write past an end is reported) over edge sizes, odd rank
counts, every type and random bytes, including NaN / inf / FP8 special codes.
Any report fails the test."""
import os
import shutil
import subprocess

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "mrr_oracle.c")

DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_allreduce(const void* const*, void* const*, size_t, int, int, int, int, int);
int orc_convert(const void*, void*, size_t, int, int);
int orc_narrow_f64(const double*, void*, size_t, int);
int orc_widen_f64(const void*, double*, size_t, int);
void orc_pack(const uint8_t*, size_t, uint32_t, uint64_t*);
void orc_unpack(const uint64_t*, size_t, uint8_t*);
uint32_t orc_next_flag(uint32_t);
int orc_allreduce_packet(const void* const*, void* const*, uint64_t*, size_t, int, int, int,
                         uint32_t);
int orc_allreduce_packet_rsag(const void* const*, void* const*, uint64_t*, size_t, int, int, int,
                              uint32_t);
int orc_packet_reduce(const uint64_t* const*, uint64_t*, size_t, int, int, int, uint32_t,
                      uint32_t);

static const int SZ[6] = {0, 4, 2, 2, 1, 1};
static uint64_t state = 88172645463325252ull;
static uint8_t rnd(void) {
  state ^= state << 13; state ^= state >> 7; state ^= state << 17;
  return (uint8_t)(state >> 24);
}
static void* fill(size_t n) {  /* exactly n bytes (1 if n == 0), random */
  uint8_t* p = (uint8_t*)malloc(n ? n : 1);
  for (size_t i = 0; i < n; ++i) p[i] = rnd();
  return p;
}

int main(void) {
  const size_t counts[] = {0, 1, 3, 15, 16, 17, 255, 1023};
  const int ranks[] = {1, 2, 3, 8, 32};
  for (unsigned ci = 0; ci < sizeof counts / sizeof *counts; ++ci)
    for (unsigned ri = 0; ri < sizeof ranks / sizeof *ranks; ++ri)
      for (int t = 1; t <= 5; ++t)
        for (int acc = 1; acc <= 5; ++acc) {
          const size_t count = counts[ci];
          const int n = ranks[ri];
          void* in[32]; void* out[32];
          for (int r = 0; r < n; ++r) { in[r] = fill(count * SZ[t]); out[r] = fill(count * 4); }
          for (int tout = 1; tout <= 5; ++tout)
            if (orc_allreduce((const void* const*)in, out, count, t, acc, tout, n, n)) return 1;
          const size_t nbytes = count * SZ[t], npkt = (nbytes + 3) / 4;
          uint64_t* scratch = (uint64_t*)fill((size_t)n * n * npkt * 8);
          if (orc_allreduce_packet((const void* const*)in, out, scratch, count, t, acc, n, 7)) return 2;
          free(scratch);
          const size_t per = (count + n - 1) / n, vw = 16 / SZ[t];
          const size_t cw = (per + vw - 1) / vw * vw * SZ[t] / 4;
          scratch = (uint64_t*)fill(2 * (size_t)n * n * cw * 8);
          if (orc_allreduce_packet_rsag((const void* const*)in, out, scratch, count, t, acc, n, 9))
            return 3;
          free(scratch);
          uint64_t* pk[32];
          for (int r = 0; r < n; ++r) {
            pk[r] = (uint64_t*)fill(npkt * 8);
            orc_pack((const uint8_t*)in[r], nbytes, 41, pk[r]);
          }
          uint64_t* po = (uint64_t*)fill(npkt * 8);
          if (orc_packet_reduce((const uint64_t* const*)pk, po, npkt, t, acc, n, 41, 42)) return 4;
          uint8_t* back = (uint8_t*)fill(nbytes);
          orc_unpack(po, nbytes, back);
          free(back); free(po);
          for (int r = 0; r < n; ++r) { free(pk[r]); free(in[r]); free(out[r]); }
        }
  for (int t = 1; t <= 5; ++t)
    for (int u = 1; u <= 5; ++u)
      for (unsigned ci = 0; ci < sizeof counts / sizeof *counts; ++ci) {
        const size_t n = counts[ci];
        void* a = fill(n * SZ[t]); void* b = fill(n * SZ[u]);
        double* d = (double*)malloc(n ? n * 8 : 8);
        for (size_t i = 0; i < n; ++i) {
          uint64_t bits = 0;
          for (int k = 0; k < 8; ++k) bits = bits << 8 | rnd();
          memcpy(&d[i], &bits, 8);  /* every pattern: NaN, inf, denormals */
        }
        if (orc_convert(a, b, n, t, u) || orc_narrow_f64(d, b, n, u) || orc_widen_f64(a, d, n, t))
          return 5;
        free(a); free(b); free(d);
      }
  uint32_t f = 0xFFFFFFFEu;
  for (int i = 0; i < 4; ++i) f = orc_next_flag(f);
  puts("ok");
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not present")
def test_oracle_under_asan_and_ubsan(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "driver"
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", SRC, str(drv), "-o", str(exe),
         "-lm"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr[-4000:]
