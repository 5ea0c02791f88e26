// launchers.hpp -- prototypes of the host-side launchers, one per kernel
// family (internal; the public boundary is include/gdnq.h).  Arguments are
// validated by api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include "gdnq.h"
#include "launch.hpp"

namespace gdnq {

hipError_t launch_step_fused(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, const void *q,
                             const void *k, const void *v, const float *a, const float *b, void *o,
                             hipStream_t st);
hipError_t launch_step_fp32(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                            const float *a, const float *b, void *o, hipStream_t st);
hipError_t launch_window_step(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, const void *q,
                              const void *k, const void *v, const float *a, const float *b, void *o,
                              int t_in_window, hipStream_t st);
hipError_t launch_flush(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, int n_tokens, hipStream_t st);
hipError_t launch_quantize(const gdnq_desc &d, const float *S, const gdnq_state &s, hipStream_t st);
hipError_t launch_dequantize(const gdnq_desc &d, const gdnq_state &s, float *S_out, hipStream_t st);
hipError_t launch_calibrate(const gdnq_desc &d, const float *S0, const void *k, const void *v,
                            const float *a, const float *b, int n_steps, int32_t *hp_idx,
                            float *score, hipStream_t st);
hipError_t launch_fit_static(const gdnq_desc &d, const float *S0, const void *q, const void *k, const void *v,
                             const float *a, const float *b, int n_steps, float *row_scale, float *col_scale,
                             hipStream_t st);
hipError_t launch_prefill(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                          const float *a, const float *b, void *o, int T, hipStream_t st);
hipError_t launch_prefill_kda(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                              const float *a, const float *b, void *o, int T, hipStream_t st);

}  // namespace gdnq
