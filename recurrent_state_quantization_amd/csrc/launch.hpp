// launch.hpp -- what the gdnq kernels and their host-side launchers share
// (internal; the public boundary is include/gdnq.h): table limits, the
// batch-entry -> head mapping, and the compile-time dispatch helpers.  The
// launcher prototypes are in launchers.hpp.
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

// Division of a workgroup index w < 2^31 by a divisor d fixed for the call,
// without a divide: q = mulhi(w, m) >> (l - 1) with l = ceil(log2 d) and
// m = ceil(2^(31+l) / d) is exact for every w < 2^31 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994,
// Theorem 4.2, with N = 31 dividend bits).  d = 1 is the identity.
struct Divisor {
    unsigned d, m, l;
};

inline Divisor make_divisor(unsigned d)
{
    Divisor v{d, 0u, 0u};
    if (d > 1) {
        v.l = 32u - (unsigned)__builtin_clz(d - 1u);
        v.m = (unsigned)(((1ull << (31u + v.l)) + d - 1u) / d);
    }
    return v;
}

__device__ __forceinline__ unsigned div_by(unsigned w, const Divisor &v)
{
    return v.d <= 1u ? w : ((unsigned)(((unsigned long long)w * v.m) >> 32) >> (v.l - 1u));
}

// Batch entry -> heads of one call.  Input head hi = b*H + hh (the
// workgroup) reads key head b*HK + hh/(H/HK) and state head slots[b]*H + hh
// (hi itself when slots is null); pos[b], when given, replaces the call's
// window position (decode step) or token count (flush) for entry b.
struct HeadMap {
    const int32_t *slots, *pos;
    int H, HK, n_slots;
    Divisor byH, byG;   // H, and the value heads per key head H/HK
};

struct HeadIdx {
    size_t in, state, key;
    unsigned b, hh;
    int pos;
};

// First half: the input and key heads of this workgroup (no memory read),
// so the input loads can be issued before the slot is known.
__device__ __forceinline__ void map_inputs(const HeadMap &m, HeadIdx &x)
{
    const unsigned w = __builtin_amdgcn_workgroup_id_x();
    x.in = w;
    if (!m.slots && !m.pos && m.HK == m.H) {   // the plain call
        x.b = 0;
        x.hh = 0;
        x.key = w;
        return;
    }
    // uniform values: readfirstlane lets the slot and position reads below
    // be scalar loads, which do not wait behind the vector loads in flight
    x.b = __builtin_amdgcn_readfirstlane(div_by(w, m.byH));
    x.hh = __builtin_amdgcn_readfirstlane(w - x.b * (unsigned)m.H);
    x.key = (size_t)x.b * m.HK + div_by(x.hh, m.byG);
}

// Second half: the state head and the entry's position; false: the entry is
// skipped (slot outside [0, n_slots) or pos outside [lo, hi]).  Uniform per
// workgroup.
__device__ __forceinline__ bool map_state(const HeadMap &m, int pos, int lo, int hi, HeadIdx &x)
{
    x.state = x.in;
    x.pos = pos;
    if (!m.slots && !m.pos) return pos >= lo && pos <= hi;
    if (m.slots) {
        const long long s = m.slots[x.b];
        if (s < 0 || s >= m.n_slots) return false;
        x.state = (size_t)s * m.H + x.hh;
    }
    if (m.pos) x.pos = m.pos[x.b];
    return x.pos >= lo && x.pos <= hi;
}

__device__ __forceinline__ bool map_head(const HeadMap &m, int pos, int lo, int hi, HeadIdx &x)
{
    map_inputs(m, x);
    return map_state(m, pos, lo, hi, x);
}

inline HeadMap plain_map(const gdnq_desc &d)
{
    const int hk = d.hk ? d.hk : d.H;
    return HeadMap{nullptr, nullptr, d.H, hk, d.B, make_divisor((unsigned)d.H),
                   make_divisor((unsigned)(d.H / hk))};
}

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
