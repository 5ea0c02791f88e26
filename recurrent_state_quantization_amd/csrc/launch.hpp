// launch.hpp -- host-side launchers of the gdnq kernels (internal; the
// public boundary is include/gdnq.h).  Arguments are validated by api.cpp
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "gdnq.h"

namespace gdnq {

// Limits of the kernels' LDS tables: window length, compensators per
// head, DAMP rows per head.
constexpr int MAX_W = 256;
constexpr int MAX_R = 8;
constexpr int MAX_HP = 64;

// Batch entry -> heads of one call.  Input head hi = b*H + hh (the
// workgroup) reads key head b*HK + hh/(H/HK) and state head slots[b]*H + hh
// (hi itself when slots is null); pos[b], when given, replaces the call's
// window position (decode step) or token count (flush) for entry b.
struct HeadMap {
    const int32_t *slots, *pos;
    int H, HK, n_slots;
};

struct HeadIdx {
    size_t in, state, key;
    int pos;
};

// The heads of this workgroup; false: the entry is skipped (slot outside
// [0, n_slots) or pos outside [lo, hi]).  Uniform per workgroup.
__device__ __forceinline__ bool map_head(const HeadMap &m, int pos, int lo, int hi, HeadIdx &x)
{
    const unsigned w = __builtin_amdgcn_workgroup_id_x();
    if (!m.slots && !m.pos && m.HK == m.H) {   // the plain call: no divisions
        x.in = x.state = x.key = w;
        x.pos = pos;
        return true;
    }
    const unsigned b = w / (unsigned)m.H, hh = w % (unsigned)m.H;
    x.in = w;
    x.key = (size_t)b * m.HK + hh / (unsigned)(m.H / m.HK);
    long long s = b;
    if (m.slots) {
        s = m.slots[b];
        if (s < 0 || s >= m.n_slots) return false;
    }
    x.state = (size_t)s * m.H + hh;
    x.pos = m.pos ? m.pos[b] : pos;
    return x.pos >= lo && x.pos <= hi;
}

inline HeadMap plain_map(const gdnq_desc &d)
{
    return HeadMap{nullptr, nullptr, d.H, d.hk ? d.hk : d.H, d.B};
}

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

// Call f(DK, DV) as compile-time constants for the supported head dims.
template <class F>
hipError_t with_dims(int dk, int dv, F &&f)
{
    if (dk == 128 && dv == 128) return f(std::integral_constant<int, 128>{}, std::integral_constant<int, 128>{});
    if (dk == 64 && dv == 64) return f(std::integral_constant<int, 64>{}, std::integral_constant<int, 64>{});
    if (dk == 128 && dv == 64) return f(std::integral_constant<int, 128>{}, std::integral_constant<int, 64>{});
    if (dk == 64 && dv == 128) return f(std::integral_constant<int, 64>{}, std::integral_constant<int, 128>{});
    return hipErrorInvalidValue;
}

template <class F>
hipError_t with_bool(bool x, F &&f)
{
    if (x) return f(std::true_type{});
    return f(std::false_type{});
}

// Call f(BITS) with the code width as a compile-time constant (0 means 8).
template <class F>
hipError_t with_bits(int bits, F &&f)
{
    if (bits == 0 || bits == 8) return f(std::integral_constant<int, 8>{});
    if (bits == 6) return f(std::integral_constant<int, 6>{});
    if (bits == 4) return f(std::integral_constant<int, 4>{});
    return hipErrorInvalidValue;
}

}  // namespace gdnq
