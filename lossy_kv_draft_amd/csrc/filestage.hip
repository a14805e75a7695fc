// Full-KV staging from a file: the stand-in for a remote prefix cache.
//
// "VeriCache: Turning Lossy KV Cache into Lossless LLM Inference" (neuraltrendhub.com
// summary, "What the paper found" and "Original abstract"): the method applies to
// remote prefix caching as well as to long-context decoding; there the full KV of
// the shared prefix lives in a remote store and its swap-in is bound by the network
// instead of PCIe, and drafting over the compressed cache overlaps that transfer.
//
// Here the store is a file (any file descriptor that supports pread).  A stager
// owns a pool of host threads and a ring of pinned bounce buffers.  A staging call
// cuts the requested byte ranges into chunks and returns at once with a ticket; a
// worker takes a free buffer, waits until the buffer's previous DMA copy has
// finished, reads one chunk into it, and issues the host-to-device copy on the
// caller's copy stream.  When every chunk of a call has been issued, the call's
// `done` event is recorded on that stream.  An optional byte rate caps the reads
// (a network link of that speed).  The host thread that consumes the rows waits
// for the ticket, then makes its stream wait for `done`.

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include <unistd.h>

#include "host_common.h"

namespace vc {

struct StageJob {
  hipStream_t stream = nullptr;
  hipEvent_t done = nullptr;
  std::atomic<int64_t> remaining{0};
  bool finished = false;          // guarded by the stager's mutex
  vc_status status = VC_OK;       // first failure, guarded by the stager's mutex
  std::string message;
};

struct StageChunk {
  std::shared_ptr<StageJob> job;
  int fd;
  int64_t file_off;
  char* dst;
  size_t bytes;
};

}  // namespace vc

struct vc_file_stager {
  int device = 0;
  size_t chunk = 0;
  double rate = 0.0;  // bytes per second, 0 = unlimited
  std::vector<char*> bufs;
  std::vector<hipEvent_t> buf_ev;

  std::mutex mu;
  std::condition_variable cv_work, cv_free, cv_done;
  std::deque<vc::StageChunk> work;
  std::deque<int> free_bufs;
  std::map<int64_t, std::shared_ptr<vc::StageJob>> jobs;
  int64_t next_ticket = 1;
  bool stop = false;
  std::vector<std::thread> threads;

  std::mutex rate_mu;
  std::chrono::steady_clock::time_point next_slot{};
};

namespace vc {

static void job_fail(vc_file_stager* st, StageJob& job, vc_status s, const std::string& msg) {
  std::lock_guard<std::mutex> g(st->mu);
  if (job.status == VC_OK) {
    job.status = s;
    job.message = msg;
  }
}

// Reads exactly n bytes at off; false on an error or end of file.
static bool read_full(int fd, char* p, size_t n, int64_t off, std::string* err) {
  while (n > 0) {
    const ssize_t r = pread(fd, p, n, static_cast<off_t>(off));
    if (r < 0) {
      if (errno == EINTR) continue;
      *err = std::string("pread failed: ") + strerror(errno);
      return false;
    }
    if (r == 0) {
      *err = "pread reached the end of the file at offset " + std::to_string(off);
      return false;
    }
    p += r;
    n -= static_cast<size_t>(r);
    off += r;
  }
  return true;
}

// Rate cap: the chunk may not be complete before the link could have carried it.
static void pace(vc_file_stager* st, size_t bytes, std::chrono::steady_clock::time_point* due) {
  using namespace std::chrono;
  if (st->rate <= 0.0) return;
  const auto span = duration_cast<steady_clock::duration>(duration<double>(static_cast<double>(bytes) / st->rate));
  std::lock_guard<std::mutex> g(st->rate_mu);
  const auto start = std::max(steady_clock::now(), st->next_slot);
  st->next_slot = start + span;
  *due = st->next_slot;
}

static void worker_main(vc_file_stager* st) {
  (void)hipSetDevice(st->device);  // a failure shows up in the first copy
  for (;;) {
    StageChunk c;
    int buf = -1;
    {
      std::unique_lock<std::mutex> lk(st->mu);
      st->cv_work.wait(lk, [&] { return st->stop || !st->work.empty(); });
      if (st->work.empty()) return;  // stop requested and nothing left
      c = std::move(st->work.front());
      st->work.pop_front();
      st->cv_free.wait(lk, [&] { return !st->free_bufs.empty(); });
      buf = st->free_bufs.front();
      st->free_bufs.pop_front();
    }
    StageJob& job = *c.job;
    bool ok;
    {
      std::lock_guard<std::mutex> g(st->mu);
      ok = job.status == VC_OK;  // after a failure the job's other chunks are skipped
    }
    if (ok) {
      hipError_t e = hipEventSynchronize(st->buf_ev[buf]);  // previous copy out of this buffer
      if (e != hipSuccess) {
        job_fail(st, job, VC_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
        ok = false;
      }
    }
    if (ok) {
      std::chrono::steady_clock::time_point due{};
      pace(st, c.bytes, &due);
      std::string err;
      if (!read_full(c.fd, st->bufs[buf], c.bytes, c.file_off, &err)) {
        job_fail(st, job, VC_ERR_IO, err);
        ok = false;
      }
      if (ok && st->rate > 0.0) std::this_thread::sleep_until(due);
    }
    if (ok) {
      hipError_t e = hipMemcpyAsync(c.dst, st->bufs[buf], c.bytes, hipMemcpyHostToDevice, job.stream);
      if (e == hipSuccess) e = hipEventRecord(st->buf_ev[buf], job.stream);
      if (e != hipSuccess) job_fail(st, job, VC_ERR_HIP, std::string("host-to-device copy: ") + hipGetErrorString(e));
    }
    {
      std::lock_guard<std::mutex> g(st->mu);
      st->free_bufs.push_back(buf);
    }
    st->cv_free.notify_one();
    if (job.remaining.fetch_sub(1, std::memory_order_acq_rel) == 1) {
      // every chunk of the job has been issued on its stream (or skipped)
      hipError_t e = job.done ? hipEventRecord(job.done, job.stream) : hipSuccess;
      if (e != hipSuccess) job_fail(st, job, VC_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
      {
        std::lock_guard<std::mutex> g(st->mu);
        job.finished = true;
      }
      st->cv_done.notify_all();
    }
  }
}

static void release_stager(vc_file_stager* st) {
  {
    std::lock_guard<std::mutex> g(st->mu);
    st->stop = true;
  }
  st->cv_work.notify_all();
  for (auto& t : st->threads) t.join();
  for (size_t i = 0; i < st->bufs.size(); ++i) {
    if (st->buf_ev[i]) {
      (void)hipEventSynchronize(st->buf_ev[i]);
      (void)hipEventDestroy(st->buf_ev[i]);
    }
    if (st->bufs[i]) (void)hipHostFree(st->bufs[i]);
  }
  delete st;
}

}  // namespace vc

using namespace vc;

extern "C" vc_status vc_file_stager_create(int32_t n_threads, size_t chunk_bytes, int32_t n_buffers,
                                           double max_bytes_per_s, vc_file_stager** out) {
  clear_error();
  VC_REQUIRE(out != nullptr, "out is NULL");
  *out = nullptr;
  VC_REQUIRE(n_threads >= 1 && n_threads <= 64, "n_threads must be in [1, 64] (got %d)", n_threads);
  VC_REQUIRE(n_buffers >= n_threads && n_buffers <= 1024, "n_buffers must be in [n_threads, 1024] (got %d)",
             n_buffers);
  VC_REQUIRE(chunk_bytes >= 4096 && chunk_bytes <= (size_t(1) << 30), "chunk_bytes must be in [4 KiB, 1 GiB]");
  VC_REQUIRE(max_bytes_per_s >= 0.0, "max_bytes_per_s must be >= 0");
  auto* st = new vc_file_stager;
  st->chunk = chunk_bytes;
  st->rate = max_bytes_per_s;
  st->bufs.assign(n_buffers, nullptr);
  st->buf_ev.assign(n_buffers, nullptr);
  hipError_t e = hipGetDevice(&st->device);
  for (int i = 0; i < n_buffers && e == hipSuccess; ++i) {
    e = hipHostMalloc(reinterpret_cast<void**>(&st->bufs[i]), chunk_bytes, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&st->buf_ev[i], hipEventDisableTiming);
    if (e == hipSuccess) st->free_bufs.push_back(i);
  }
  if (e != hipSuccess) {
    set_error("stager set-up failed: %s", hipGetErrorString(e));
    release_stager(st);
    return VC_ERR_HIP;
  }
  for (int i = 0; i < n_threads; ++i) st->threads.emplace_back(worker_main, st);
  *out = st;
  return VC_OK;
}

extern "C" vc_status vc_file_stager_destroy(vc_file_stager* st) {
  clear_error();
  if (!st) return VC_OK;
  release_stager(st);  // the workers drain every queued chunk first
  return VC_OK;
}

extern "C" vc_status vc_stage_full_kv_file(vc_file_stager* st, int32_t fd, int64_t k_offset, int64_t v_offset,
                                           void* dev_k, void* dev_v, int32_t B, int32_t Hkv, int32_t d,
                                           int32_t elem_bytes, int64_t file_rows, int64_t dev_rows, int64_t tok_begin,
                                           int64_t tok_end, void* copy_stream, void* done, int64_t* ticket) {
  clear_error();
  VC_REQUIRE(st != nullptr && ticket != nullptr, "stager / ticket is NULL");
  VC_REQUIRE(fd >= 0, "bad file descriptor %d", fd);
  VC_REQUIRE(dev_k && dev_v, "NULL device pointer");
  VC_REQUIRE(k_offset >= 0 && v_offset >= 0, "file offsets must be >= 0");
  VC_REQUIRE(B > 0 && Hkv > 0 && d > 0, "bad B/Hkv/d");
  VC_REQUIRE(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4 || elem_bytes == 8, "bad elem_bytes %d",
             elem_bytes);
  VC_REQUIRE(tok_begin >= 0 && tok_begin <= tok_end && tok_end <= file_rows && tok_end <= dev_rows,
             "rows [%lld, %lld) do not fit file_rows %lld / dev_rows %lld", (long long)tok_begin, (long long)tok_end,
             (long long)file_rows, (long long)dev_rows);
  const int64_t row = static_cast<int64_t>(d) * elem_bytes;
  const int64_t width = (tok_end - tok_begin) * row;
  auto job = std::make_shared<StageJob>();
  job->stream = as_stream(copy_stream);
  job->done = reinterpret_cast<hipEvent_t>(done);
  std::vector<StageChunk> chunks;
  for (int t = 0; t < 2 && width > 0; ++t) {
    const int64_t base = t == 0 ? k_offset : v_offset;
    char* dst = static_cast<char*>(t == 0 ? dev_k : dev_v);
    for (int64_t bh = 0; bh < static_cast<int64_t>(B) * Hkv; ++bh) {
      const int64_t f0 = base + (bh * file_rows + tok_begin) * row;
      char* d0 = dst + (bh * dev_rows + tok_begin) * row;
      for (int64_t o = 0; o < width; o += static_cast<int64_t>(st->chunk))
        chunks.push_back({job, fd, f0 + o, d0 + o, static_cast<size_t>(std::min<int64_t>(st->chunk, width - o))});
    }
  }
  std::lock_guard<std::mutex> g(st->mu);
  *ticket = st->next_ticket++;
  st->jobs[*ticket] = job;
  if (chunks.empty()) {  // nothing to read: only the event
    if (job->done) {
      hipError_t e = hipEventRecord(job->done, job->stream);
      if (e != hipSuccess) {
        job->status = VC_ERR_HIP;
        job->message = std::string("hipEventRecord: ") + hipGetErrorString(e);
      }
    }
    job->finished = true;
    return VC_OK;
  }
  job->remaining.store(static_cast<int64_t>(chunks.size()), std::memory_order_relaxed);
  for (auto& c : chunks) st->work.push_back(std::move(c));
  st->cv_work.notify_all();
  return VC_OK;
}

extern "C" vc_status vc_file_stager_wait(vc_file_stager* st, int64_t ticket) {
  clear_error();
  VC_REQUIRE(st != nullptr, "stager is NULL");
  std::unique_lock<std::mutex> lk(st->mu);
  auto it = st->jobs.find(ticket);
  VC_REQUIRE(it != st->jobs.end(), "unknown or already collected ticket %lld", (long long)ticket);
  std::shared_ptr<StageJob> job = it->second;
  st->cv_done.wait(lk, [&] { return job->finished; });
  st->jobs.erase(ticket);
  if (job->status != VC_OK) {
    set_error("staging ticket %lld: %s", (long long)ticket, job->message.c_str());
    return job->status;
  }
  return VC_OK;
}
