// Kernel timing with HIP events (see include/ttc_trace.h).
#pragma once

#include <hip/hip_runtime.h>

namespace ttc {

// true while tracing is on
bool trace_on();
// record the start / end of a kernel launch named `name` on stream s
void trace_begin(const char* name, hipStream_t s);
void trace_end(hipStream_t s);

// RAII bracket for one launch
struct TraceScope {
  hipStream_t s;
  bool on;
  TraceScope(const char* name, hipStream_t st) : s(st), on(trace_on()) {
    if (on) trace_begin(name, s);
  }
  ~TraceScope() {
    if (on) trace_end(s);
  }
};

}  // namespace ttc
