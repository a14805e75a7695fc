// Drives the file stager's host logic (filestage.hip built with the host compiler
// against the stub HIP runtime) through its ticket, buffer, failure and shutdown
// paths, from several host threads at once, and checks every staged byte.  Built
// and run under ThreadSanitizer and AddressSanitizer by test_host_sanitize.py.
#include <fcntl.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <thread>
#include <vector>

#include "hip/hip_runtime.h"
#include "../../include/vc.h"

namespace vc {  // the error helpers the library's api.hip defines
static thread_local char g_err[512];
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = '\0'; }
}  // namespace vc
extern "C" const char* vc_last_error(void) { return vc::g_err; }

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c); \
      g_fail = 1;                                                     \
    }                                                                 \
  } while (0)

// file of `n` bytes, byte i = hash(i)
static unsigned char pat(int64_t i) { return static_cast<unsigned char>((i * 2654435761u) >> 13); }
static int make_file(int64_t n) {
  char path[] = "/tmp/vc_stager_XXXXXX";
  int fd = mkstemp(path);
  unlink(path);
  std::vector<unsigned char> b(n);
  for (int64_t i = 0; i < n; ++i) b[i] = pat(i);
  CHECK(write(fd, b.data(), n) == n);
  return fd;
}

// rows [t0, t1) of every (sequence, head) of K at k_off and V at v_off, file rows F,
// device rows D, row bytes R: compares dev with the file's bytes
static void check_rows(const std::vector<unsigned char>& dev, int64_t off, int BH, int64_t F, int64_t D, int64_t R,
                       int64_t t0, int64_t t1) {
  for (int bh = 0; bh < BH; ++bh)
    for (int64_t t = t0; t < t1; ++t)
      for (int64_t c = 0; c < R; ++c) {
        const unsigned char want = pat(off + (bh * F + t) * R + c);
        if (dev[(bh * D + t) * R + c] != want) {
          fprintf(stderr, "byte mismatch bh %d row %lld col %lld\n", bh, (long long)t, (long long)c);
          g_fail = 1;
          return;
        }
      }
}

// One consumer: `calls` staging calls of ragged row ranges on its own stream, each
// waited for (ticket, then the stream), bytes checked after every call.
static void consumer(vc_file_stager* st, int fd, int seed, int calls) {
  const int B = 2, H = 3, d = 64, eb = 2;
  const int64_t F = 1000, D = 1100, R = d * eb;
  const int64_t kbytes = static_cast<int64_t>(B) * H * F * R;
  StubStream stream;
  StubEvent done;
  std::vector<unsigned char> dk(B * H * D * R), dv(B * H * D * R);
  unsigned s = 12345u + seed;
  for (int i = 0; i < calls; ++i) {
    s = s * 1103515245u + 12345u;
    const int64_t t0 = (s >> 8) % 500, t1 = t0 + 1 + (s >> 20) % 500;
    int64_t ticket = -1;
    CHECK(vc_stage_full_kv_file(st, fd, 0, kbytes, dk.data(), dv.data(), B, H, d, eb, F, D, t0, t1, &stream, &done,
                                &ticket) == VC_OK);
    CHECK(vc_file_stager_wait(st, ticket) == VC_OK);
    CHECK(hipEventSynchronize(&done) == hipSuccess);
    stream.drain();
    check_rows(dk, 0, B * H, F, D, R, t0, t1);
    check_rows(dv, kbytes, B * H, F, D, R, t0, t1);
  }
}

int main() {
  const int64_t file_bytes = 2 * 2 * 3 * 1000 * 128;  // K and V of [2, 3, 1000, 64] bf16
  const int fd = make_file(file_bytes);

  // 1. four consumers on their own streams share one stager (3 threads, 4 buffers of
  //    8 KiB: every buffer is reused many times while its last copy may be pending)
  {
    vc_file_stager* st = nullptr;
    CHECK(vc_file_stager_create(3, 8192, 4, 0.0, &st) == VC_OK);
    std::vector<std::thread> ts;
    for (int c = 0; c < 4; ++c) ts.emplace_back(consumer, st, fd, c, 12);
    for (auto& t : ts) t.join();
    CHECK(vc_file_stager_destroy(st) == VC_OK);
  }
  // 2. a read past the end of the file fails the call with VC_ERR_IO (its other chunks
  //    skipped); the next call on the same stager succeeds
  {
    vc_file_stager* st = nullptr;
    CHECK(vc_file_stager_create(2, 4096, 2, 0.0, &st) == VC_OK);
    StubStream stream;
    StubEvent done;
    std::vector<unsigned char> dk(6 * 1100 * 128), dv(dk.size());
    int64_t t1 = -1, t2 = -1;
    CHECK(vc_stage_full_kv_file(st, fd, 0, file_bytes - 1000, dk.data(), dv.data(), 2, 3, 64, 2, 1000, 1100, 0, 900,
                                &stream, &done, &t1) == VC_OK);
    CHECK(vc_stage_full_kv_file(st, fd, 0, file_bytes / 2, dk.data(), dv.data(), 2, 3, 64, 2, 1000, 1100, 100, 200,
                                &stream, &done, &t2) == VC_OK);
    CHECK(vc_file_stager_wait(st, t1) == VC_ERR_IO);
    CHECK(strstr(vc_last_error(), "end of the file") != nullptr);
    CHECK(vc_file_stager_wait(st, t2) == VC_OK);
    CHECK(vc_file_stager_wait(st, t2) == VC_ERR_INVALID_ARG);  // a ticket is collected once
    CHECK(hipEventSynchronize(&done) == hipSuccess);
    stream.drain();
    check_rows(dk, 0, 6, 1000, 1100, 128, 100, 200);
    CHECK(vc_file_stager_destroy(st) == VC_OK);
  }
  // 3. rate cap: 600 KiB at 20 MB/s takes at least ~30 ms; an empty row range only
  //    records the event
  {
    vc_file_stager* st = nullptr;
    CHECK(vc_file_stager_create(4, 16384, 8, 20e6, &st) == VC_OK);
    StubStream stream;
    StubEvent done;
    std::vector<unsigned char> dk(6 * 1000 * 128), dv(dk.size());
    const auto t0 = std::chrono::steady_clock::now();
    int64_t t = -1, te = -1;
    CHECK(vc_stage_full_kv_file(st, fd, 0, file_bytes / 2, dk.data(), dv.data(), 2, 3, 64, 2, 1000, 1000, 0, 400,
                                &stream, &done, &t) == VC_OK);
    CHECK(vc_file_stager_wait(st, t) == VC_OK);
    const double ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    CHECK(ms >= 25.0);
    CHECK(vc_stage_full_kv_file(st, fd, 0, 0, dk.data(), dv.data(), 2, 3, 64, 2, 1000, 1000, 7, 7, &stream, &done,
                                &te) == VC_OK);
    CHECK(vc_file_stager_wait(st, te) == VC_OK);
    stream.drain();
    check_rows(dk, 0, 6, 1000, 1000, 128, 0, 400);
    CHECK(vc_file_stager_destroy(st) == VC_OK);
  }
  // 4. destroy with calls still queued and never waited for: the workers finish every
  //    queued chunk (copies issued) before the buffers are freed
  {
    vc_file_stager* st = nullptr;
    CHECK(vc_file_stager_create(2, 4096, 3, 0.0, &st) == VC_OK);
    StubStream stream;
    std::vector<unsigned char> dk(6 * 1000 * 128), dv(dk.size());
    for (int i = 0; i < 5; ++i) {
      int64_t t = -1;
      CHECK(vc_stage_full_kv_file(st, fd, 0, file_bytes / 2, dk.data(), dv.data(), 2, 3, 64, 2, 1000, 1000, 0, 1000,
                                  &stream, nullptr, &t) == VC_OK);
    }
    CHECK(vc_file_stager_destroy(st) == VC_OK);
    stream.drain();
    check_rows(dk, 0, 6, 1000, 1000, 128, 0, 1000);
    check_rows(dv, file_bytes / 2, 6, 1000, 1000, 128, 0, 1000);
  }
  close(fd);
  if (g_fail) return 1;
  printf("stager host paths ok\n");
  return 0;
}
