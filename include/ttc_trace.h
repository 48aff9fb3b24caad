/*
 * ttc_trace.h - optional kernel timing of libttc with HIP events.
 *
 * While tracing is on, every kernel the library enqueues is launched with a
 * start and a stop hipEvent that the runtime stamps when the kernel itself
 * begins and ends on its stream (hipExtLaunchKernelGGL), so the elapsed time
 * of each launch can be read back afterwards.  Tracing is off by default and
 * costs nothing then.  It is meant for benchmarks and tests: reading the
 * records synchronises on the recorded events.  Do not trace inside a HIP
 * graph capture.  Not thread-safe against concurrent library calls.
 */
#ifndef TTC_TRACE_H
#define TTC_TRACE_H

#include <stdint.h>

#include "ttc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Drop every record and start recording (events are created on demand and
 * reused).  Returns TTC_ERR_HIP if an event cannot be created. */
ttc_status ttc_trace_start(void);

/* Stop recording; the records stay readable. */
ttc_status ttc_trace_stop(void);

/* Number of kernel launches recorded since the last ttc_trace_start. */
ttc_status ttc_trace_count(int32_t* n);

/*
 * Record i (0-based, in launch order): the kernel's name (static storage, one
 * of "merge", "fwd", "bwd_dy", "dz_sum", "bwd_dx", "reduce", "core", "zero",
 * "rank_grads", "seq_fwd", "seq_bwd", "seq_reduce", "ttm_sort", "ttm_lists",
 * "ttm_level", "ttm_gather", "ttm_seg", "ttm_bwd_level", "ttm_reduce") and its
 * duration in
 * milliseconds.  Waits for the record's end event.
 */
ttc_status ttc_trace_get(int32_t i, const char** name, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* TTC_TRACE_H */
