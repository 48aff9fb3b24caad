// Kernel timing with HIP events (see include/ttc_trace.h).
//
// While tracing is on, a launch made with TTC_LAUNCH inside a TraceScope goes
// through hipExtLaunchKernelGGL with a start and a stop event, which the
// runtime stamps when the kernel itself begins and ends on its stream (no
// separate event packets around the dispatch).  Tracing off: a plain launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace ttc {

// true while tracing is on
bool trace_on();
// the name of the launch about to be made (set by TraceScope)
void trace_set_pending(const char* name);
// If tracing is on and a name is pending: a fresh event pair for that name,
// recorded in launch order; the pending name is consumed.
bool trace_take(hipEvent_t* start, hipEvent_t* stop);

// names the next TTC_LAUNCH
struct TraceScope {
  TraceScope(const char* name, hipStream_t) { trace_set_pending(trace_on() ? name : nullptr); }
  ~TraceScope() { trace_set_pending(nullptr); }
};

}  // namespace ttc

#define TTC_LAUNCH(kern, grid, block, lds, st, ...)                                     \
  do {                                                                                 \
    hipEvent_t ttc_ev0_, ttc_ev1_;                                                     \
    if (::ttc::trace_take(&ttc_ev0_, &ttc_ev1_))                                       \
      hipExtLaunchKernelGGL(kern, grid, block, lds, st, ttc_ev0_, ttc_ev1_, 0, __VA_ARGS__); \
    else                                                                               \
      hipLaunchKernelGGL(kern, grid, block, lds, st, __VA_ARGS__);                     \
  } while (0)
