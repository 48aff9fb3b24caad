// Kernel timing with HIP events: a growing pool of event pairs, reused across
// trace sessions; records are (name, start, end) in launch order.  The pair
// is handed to hipExtLaunchKernelGGL, which stamps the kernel's own start and
// end.
#include "ttc_trace.hpp"

#include <mutex>
#include <vector>

#include "../../include/ttc_trace.h"

namespace ttc {

namespace {
struct Rec {
  const char* name;
  hipEvent_t start, end;
};
std::mutex g_mu;
bool g_on = false;
bool g_error = false;
std::vector<Rec> g_pool;  // events kept for reuse
size_t g_used = 0;        // records of the current session
}  // namespace

bool trace_on() { return g_on; }

namespace {
thread_local const char* t_pending = nullptr;
}

void trace_set_pending(const char* name) { t_pending = name; }

bool trace_take(hipEvent_t* start, hipEvent_t* stop) {
  const char* name = t_pending;
  if (!name) return false;
  t_pending = nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return false;
  if (g_used == g_pool.size()) {
    Rec r{name, nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.end) != hipSuccess) {
      g_error = true;
      return false;
    }
    g_pool.push_back(r);
  }
  Rec& r = g_pool[g_used++];
  r.name = name;
  *start = r.start;
  *stop = r.end;
  return true;
}

}  // namespace ttc

using namespace ttc;

extern "C" ttc_status ttc_trace_start(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_used = 0;
  g_error = false;
  g_on = true;
  return TTC_OK;
}

extern "C" ttc_status ttc_trace_stop(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  return g_error ? TTC_ERR_HIP : TTC_OK;
}

extern "C" ttc_status ttc_trace_count(int32_t* n) {
  if (!n) return TTC_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_mu);
  *n = (int32_t)g_used;
  return TTC_OK;
}

extern "C" ttc_status ttc_trace_get(int32_t i, const char** name, float* ms) {
  if (!name || !ms) return TTC_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || (size_t)i >= g_used) return TTC_ERR_SHAPE;
  const Rec& r = g_pool[i];
  if (hipEventSynchronize(r.end) != hipSuccess) return TTC_ERR_HIP;
  float t = 0.f;
  if (hipEventElapsedTime(&t, r.start, r.end) != hipSuccess) return TTC_ERR_HIP;
  *name = r.name;
  *ms = t;
  return TTC_OK;
}
