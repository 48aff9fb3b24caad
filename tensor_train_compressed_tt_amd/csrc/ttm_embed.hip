// TTM embedding lookup (placeholder entry points until the kernels land).
#include "../../include/ttc.h"

extern "C" ttc_status ttm_embed_workspace(const ttm_embed_desc* desc, int64_t T, size_t* saved_bytes,
                                          size_t* scratch_bytes) {
  (void)desc; (void)T; (void)saved_bytes; (void)scratch_bytes;
  return TTC_ERR_UNSUPPORTED;
}
extern "C" ttc_status ttm_embed_fwd(const ttm_embed_desc*, int64_t, const int64_t*, const float* const*,
                                    const float* const*, float*, void*, size_t, void*, size_t, ttc_stream_t) {
  return TTC_ERR_UNSUPPORTED;
}
extern "C" ttc_status ttm_embed_bwd(const ttm_embed_desc*, int64_t, const int64_t*, const float*,
                                    const float* const*, const float* const*, const void*, size_t, float* const*,
                                    void*, size_t, ttc_stream_t) {
  return TTC_ERR_UNSUPPORTED;
}
