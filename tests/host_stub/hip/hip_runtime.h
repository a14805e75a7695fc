// Stand-in for the HIP runtime's host API, for building the library's host-only
// sources (the file stager) with the host compiler under ThreadSanitizer and
// AddressSanitizer.  Test infrastructure: no GPU is involved.
//
// Each stream is a thread that runs the operations enqueued on it in order, as a DMA
// engine would: an asynchronous copy is a memcpy done later on the stream's thread,
// and an event record completes when the stream reaches it.  hipEventSynchronize
// waits for the last record of the event issued before the call.  So a host buffer
// reused before its copy has run shows up as a data race (TSan) and a buffer freed
// under a pending copy as a use after free (ASan).
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <chrono>
#include <condition_variable>
#include <deque>
#include <functional>
#include <mutex>
#include <thread>

typedef enum { hipSuccess = 0, hipErrorInvalidValue = 1, hipErrorOutOfMemory = 2 } hipError_t;
typedef enum { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2 } hipMemcpyKind;
#define hipHostMallocDefault 0u
#define hipEventDisableTiming 2u

struct StubEvent {
  std::mutex mu;
  std::condition_variable cv;
  uint64_t recorded = 0;   // records issued
  uint64_t completed = 0;  // records the stream has reached
};

struct StubStream {
  std::mutex mu;
  std::condition_variable cv;
  std::deque<std::function<void()>> ops;
  bool stop = false;
  std::thread th;
  StubStream() : th([this] { run(); }) {}
  ~StubStream() {
    {
      std::lock_guard<std::mutex> g(mu);
      stop = true;
    }
    cv.notify_all();
    th.join();
  }
  void push(std::function<void()> f) {
    {
      std::lock_guard<std::mutex> g(mu);
      ops.push_back(std::move(f));
      ++pushed;
    }
    cv.notify_all();
  }
  void run() {
    for (;;) {
      std::function<void()> f;
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || !ops.empty(); });
        if (ops.empty()) return;
        f = std::move(ops.front());
        ops.pop_front();
      }
      f();
      {
        std::lock_guard<std::mutex> g(mu);
        ++done_ops;
      }
      cv.notify_all();
    }
  }
  void drain() {  // wait until every op enqueued so far has run
    std::unique_lock<std::mutex> lk(mu);
    const uint64_t want = pushed;
    cv.wait(lk, [&] { return done_ops >= want; });
  }
  uint64_t pushed = 0, done_ops = 0;  // guarded by mu
};

typedef StubStream* hipStream_t;
typedef StubEvent* hipEvent_t;

inline const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
inline hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
inline hipError_t hipSetDevice(int) { return hipSuccess; }
inline hipError_t hipHostMalloc(void** p, size_t n, unsigned) {
  *p = malloc(n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
inline hipError_t hipHostFree(void* p) { free(p); return hipSuccess; }
inline hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { *e = new StubEvent; return hipSuccess; }
inline hipError_t hipEventDestroy(hipEvent_t e) { delete e; return hipSuccess; }
inline hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t s) {
  if (!s || !dst || !src) return hipErrorInvalidValue;
  s->push([dst, src, n] {
    std::this_thread::sleep_for(std::chrono::microseconds(50));  // the copy takes a while
    memcpy(dst, src, n);
  });
  return hipSuccess;
}
inline hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  if (!e || !s) return hipErrorInvalidValue;
  uint64_t gen;
  {
    std::lock_guard<std::mutex> g(e->mu);
    gen = ++e->recorded;
  }
  s->push([e, gen] {  // signalled under the lock: the event may be destroyed right after
    std::lock_guard<std::mutex> g(e->mu);
    if (e->completed < gen) e->completed = gen;
    e->cv.notify_all();
  });
  return hipSuccess;
}
inline hipError_t hipEventSynchronize(hipEvent_t e) {
  if (!e) return hipErrorInvalidValue;
  std::unique_lock<std::mutex> lk(e->mu);
  const uint64_t want = e->recorded;
  e->cv.wait(lk, [&] { return e->completed >= want; });
  return hipSuccess;
}
