// Per-kernel timing (tracing) and a shader-clock probe for libpagedattn.
//
// While tracing is on, every device call brackets each kernel it launches with
// a pair of HIP events recorded on the caller's stream; pa_trace_read waits for
// them and reports (kernel, milliseconds) in launch order.  Events come from a
// pool and are reused, so steady-state tracing creates none.
#include <hip/hip_runtime.h>

#include <algorithm>
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

// Shader-clock probe: each of kClockWaves one-wave work-groups spins on a
// dependent FMA chain and reads the shader-clock counter (s_memtime) and the
// 100 MHz real-time counter (s_memrealtime) before and after; the ratio of the
// two deltas is the shader clock it ran at.  Results go to a device array the
// library holds, so the probe allocates nothing.
constexpr int kClockWaves = 256;
__device__ unsigned long long g_clock_ticks[2 * kClockWaves];

__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* ticks, int iters) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x;
  for (int i = 0; i < iters; ++i) x = fmaf(x, 1.0000001f, 0.5f);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    ticks[2 * blockIdx.x] = x == 12345.0f ? 0ull : t1 - t0;   // x stays live; never equal in practice
    ticks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_trace_clock(void* stream, float* mhz) {
  if (mhz == nullptr) return fail(PA_ERR_ARG, "pa_trace_clock: mhz is NULL");
  hipStream_t s = (hipStream_t)stream;
  if (stream_capturing(s)) return fail(PA_ERR_ARG, "pa_trace_clock: the stream is being captured");
  void* dev = nullptr;
  hipError_t e = hipGetSymbolAddress(&dev, HIP_SYMBOL(g_clock_ticks));
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_trace_clock: hipGetSymbolAddress: %s", hipGetErrorString(e));
  unsigned long long host[2 * kClockWaves];
  hipLaunchKernelGGL(clock_probe_kernel, dim3(kClockWaves), dim3(64), 0, s, (unsigned long long*)dev, 50000);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(host, dev, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_trace_clock: %s", hipGetErrorString(e));
  std::vector<float> f;
  for (int w = 0; w < kClockWaves; ++w)
    if (host[2 * w + 1] > 0) f.push_back(100.0f * (float)host[2 * w] / (float)host[2 * w + 1]);
  if (f.empty()) return fail(PA_ERR_HIP, "pa_trace_clock: the real-time counter did not advance");
  std::sort(f.begin(), f.end());
  *mhz = f[f.size() / 2];
  return PA_OK;
}

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
