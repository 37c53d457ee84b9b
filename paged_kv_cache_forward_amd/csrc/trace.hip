// Per-kernel timing (tracing) for libpagedattn: host code only.
//
// While tracing is on, every device call brackets each kernel it launches with
// a pair of HIP events recorded on the caller's stream; pa_trace_read waits for
// them and reports (kernel, milliseconds) in launch order.  Events come from a
// pool and are reused, so steady-state tracing creates none.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "ops.h"
#include "status.h"

namespace pa {
namespace {

constexpr size_t kMaxRecords = 4096;

struct Pending {
  const char* kernel;
  hipEvent_t start;
  hipEvent_t stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;      // idle events
std::vector<Pending> g_pending;      // recorded, not yet read
std::vector<hipEvent_t> g_open;      // start events handed out by trace_begin, by mark

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

int trace_begin(hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return -1;
  if (stream_capturing(s)) return -1;   // an event recorded in a graph fires only at replay
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (e == nullptr || hipEventRecord(e, s) != hipSuccess) return -1;
  g_open.push_back(e);
  return (int)g_open.size() - 1;
}

void trace_end(hipStream_t s, int mark, const char* kernel) {
  if (mark < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if ((size_t)mark >= g_open.size() || g_open[mark] == nullptr) return;
  hipEvent_t start = g_open[mark];
  g_open[mark] = nullptr;
  while (!g_open.empty() && g_open.back() == nullptr) g_open.pop_back();
  hipEvent_t stop = take_event();
  if (stop == nullptr || hipEventRecord(stop, s) != hipSuccess) {
    g_pool.push_back(start);
    if (stop) g_pool.push_back(stop);
    return;
  }
  if (g_pending.size() >= kMaxRecords) {   // drop the oldest record
    g_pool.push_back(g_pending.front().start);
    g_pool.push_back(g_pending.front().stop);
    g_pending.erase(g_pending.begin());
  }
  g_pending.push_back({kernel, start, stop});
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_trace_enable(int32_t on) {
  g_on.store(on != 0);
  return PA_OK;
}

extern "C" pa_status pa_trace_read(pa_trace_record* out, int32_t cap, int32_t* n) {
  if (n == nullptr || cap < 0 || (out == nullptr && cap > 0)) return fail(PA_ERR_ARG, "pa_trace_read: bad arguments");
  std::lock_guard<std::mutex> lk(g_mu);
  int32_t k = 0;
  pa_status st = PA_OK;
  for (const Pending& p : g_pending) {
    float ms = -1.0f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      st = fail(PA_ERR_HIP, "pa_trace_read: event query failed");
      ms = -1.0f;
    }
    if (k < cap) out[k++] = pa_trace_record{p.kernel, ms};
    g_pool.push_back(p.start);
    g_pool.push_back(p.stop);
  }
  g_pending.clear();
  *n = k;
  return st;
}
