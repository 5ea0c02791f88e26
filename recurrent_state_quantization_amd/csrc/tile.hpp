// tile.hpp -- register-tile geometry and cross-lane primitives shared by the
// gdnq kernels (gfx950 / CDNA4, wave64).
//
// One workgroup owns one (batch, head) state tile of DK x DV elements
// (row i = key channel, column j = value channel).  Every thread holds an
// 8 x 8 block: 8 rows and 8 *contiguous* columns, so one row of its block is
// one 8-byte INT8 load or two 16-byte fp32 loads.
//
//   NCB = DV/8 column blocks; lane = rgl*NCB + cb  (cb = column block,
//   rgl = row group within the wave); RGW = 64/NCB row groups per wave;
//   the wave owns RGW*8 rows; NW = DK/(RGW*8) waves per tile.
//   Row k (0..7) of a thread: w*RGW*8 + (k/4)*RGW*4 + 4*rgl + (k%4).
//
// With that row map one load instruction of a wave covers RGW whole rows,
// and the layout equals the accumulator layout of the 16x16x4 fp32 MFMA
// when the MFMA's logical column n is mapped to global column
// 8*(n%16) + n/16 (used by the window flush; DV = 128 only).
//
// Reductions:
//   * along a row (over the NCB lanes of a row group): DPP quad_perm,
//     row_half_mirror, row_mirror -- all-reduce, every lane gets the result;
//   * along a column inside a wave (over the RGW row-group lanes):
//     v_permlane32_swap / v_permlane16_swap reduce-scatter (plus one DPP
//     row_ror:8 all-reduce step when NCB = 8), then across waves in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdnq {

template <int DK_, int DV_>
struct Geom {
    static constexpr int DK = DK_;
    static constexpr int DV = DV_;
    static constexpr int CPT = 8;
    static constexpr int RPT = 8;
    static constexpr int NCB = DV / CPT;
    static constexpr int RGW = 64 / NCB;
    static constexpr int ROWS_W = RGW * RPT;
    static constexpr int NW = DK / ROWS_W;
    static constexpr int NT = NW * 64;
    static_assert(NCB == 8 || NCB == 16, "DV must be 64 or 128");
    static_assert(NW >= 1 && DK % ROWS_W == 0, "DK must be 64 or 128");
};

struct Lane {
    int t, lane, w, cb, rgl;
};

template <class G>
__device__ __forceinline__ Lane lane_coords()
{
    Lane c;
    c.t = (int)__builtin_amdgcn_workitem_id_x();
    c.lane = c.t & 63;
    c.w = c.t >> 6;
    c.cb = c.lane % G::NCB;
    c.rgl = c.lane / G::NCB;
    return c;
}

// First row of the thread's block; row k is row0 + koff(k), a compile-time
// offset once k is unrolled (so loads and stores use immediate offsets).
template <class G>
__device__ __forceinline__ int row0_of(const Lane &c)
{
    return c.w * G::ROWS_W + 4 * c.rgl;
}

template <class G>
__host__ __device__ constexpr int koff(int k)
{
    return (k >> 2) * (G::RGW * 4) + (k & 3);
}

template <class G>
__device__ __forceinline__ int row_of(const Lane &c, int k)
{
    return row0_of<G>(c) + koff<G>(k);
}

// ---------------------------------------------------------------- DPP
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;
constexpr int DPP_ROR8 = 0x128;

// All-reduce over the NCB column-block lanes of a row group (lane bits
// 0..log2(NCB)-1).  The mirror steps equal xor-4 / xor-8 once the smaller
// groups already hold equal values.
template <class G>
__device__ __forceinline__ float row_sum(float x)
{
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    x += dpp<DPP_HALF_MIRROR>(x);
    if constexpr (G::NCB == 16) x += dpp<DPP_MIRROR>(x);
    return x;
}

template <class G>
__device__ __forceinline__ float row_max(float x)
{
    x = fmaxf(x, dpp<DPP_XOR1>(x));
    x = fmaxf(x, dpp<DPP_XOR2>(x));
    x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
    if constexpr (G::NCB == 16) x = fmaxf(x, dpp<DPP_MIRROR>(x));
    return x;
}

// Row reduce-scatter over the NCB column-block lanes of a row group:
// x[0..7] are this lane's partials for its 8 rows; the result is the whole
// row group's reduction of x[k] with k = cb >> 1 (NCB = 16) or k = cb
// (NCB = 8).  Each step pairs lanes that still hold the same index set
// (mirror, half-mirror, then quad swaps), keeps half the values and sends
// the other half; no dynamically indexed array is involved.
template <class G, class Op>
__device__ __forceinline__ float row_reduce_scatter(const float (&x)[8], int cb)
{
    float v4[4], v2[2];
    if constexpr (G::NCB == 16) {
        // row_mirror pairs cb with cb ^ 15: every lane still holds all 8
        // values, so keep/send is decided by bit 3 alone
        const bool b3 = (cb >> 3) & 1;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float keep = b3 ? x[j + 4] : x[j];
            const float send = b3 ? x[j] : x[j + 4];
            v4[j] = Op::f(keep, dpp<DPP_MIRROR>(send));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; j++) v4[j] = 0.0f;
    }
    // row_half_mirror pairs cb with cb ^ 7 (same bit 3): decided by bit 2
    const bool b2 = (cb >> 2) & 1;
    if constexpr (G::NCB == 16) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const float keep = b2 ? v4[j + 2] : v4[j];
            const float send = b2 ? v4[j] : v4[j + 2];
            v2[j] = Op::f(keep, dpp<DPP_HALF_MIRROR>(send));
        }
    } else {
        float w4[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float keep = b2 ? x[j + 4] : x[j];
            const float send = b2 ? x[j] : x[j + 4];
            w4[j] = Op::f(keep, dpp<DPP_HALF_MIRROR>(send));
        }
        const bool b1 = (cb >> 1) & 1;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const float keep = b1 ? w4[j + 2] : w4[j];
            const float send = b1 ? w4[j] : w4[j + 2];
            v2[j] = Op::f(keep, dpp<DPP_XOR2>(send));
        }
        const bool b0 = cb & 1;
        const float keep = b0 ? v2[1] : v2[0];
        const float send = b0 ? v2[0] : v2[1];
        return Op::f(keep, dpp<DPP_XOR1>(send));  // row k = cb
    }
    const bool b1 = (cb >> 1) & 1;
    const float keep = b1 ? v2[1] : v2[0];
    const float send = b1 ? v2[0] : v2[1];
    const float v1 = Op::f(keep, dpp<DPP_XOR2>(send));
    return Op::f(v1, dpp<DPP_XOR1>(v1));           // row k = cb >> 1, both lanes of the pair
}

// Row index (0..7 within the thread's block) row_reduce_scatter leaves in
// this lane.
template <class G>
__device__ __forceinline__ int row_scatter_k(int cb)
{
    return (G::NCB == 16) ? (cb >> 1) : cb;
}

// --------------------------------------------------------- permlane swaps
// swap32(a, b): a <- [a_lo, b_lo], b <- [a_hi, b_hi] (lo = lanes 0..31).
__device__ __forceinline__ void swap32(float &a, float &b)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(a), __float_as_int(b), false, false);
    a = __int_as_float((int)r[0]);
    b = __int_as_float((int)r[1]);
}
// swap16(a, b): odd 16-lane rows of a trade places with even rows of b.
__device__ __forceinline__ void swap16(float &a, float &b)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(a), __float_as_int(b), false, false);
    a = __int_as_float((int)r[0]);
    b = __int_as_float((int)r[1]);
}

struct OpSum {
    __device__ static float f(float a, float b) { return a + b; }
};
struct OpMax {
    __device__ static float f(float a, float b) { return fmaxf(a, b); }
};

// Column reduce-scatter inside a wave: x[0..N-1] are per-lane partials over
// this lane's rows; afterwards z[p] (p < N/4) holds the whole wave's
// reduction of x[4p + e], e = 2*bit4(lane) + bit5(lane).
template <class G, class Op, int N>
__device__ __forceinline__ void col_reduce_scatter(const float (&x)[N], float (&z)[N / 4])
{
    static_assert(N % 4 == 0, "N must be a multiple of 4");
    float y[N / 2];
#pragma unroll
    for (int p = 0; p < N / 2; p++) {
        float a = x[2 * p], b = x[2 * p + 1];
        if constexpr (G::NCB == 8) {  // lane bit 3 first: all-reduce with row_ror:8
            a = Op::f(a, dpp<DPP_ROR8>(a));
            b = Op::f(b, dpp<DPP_ROR8>(b));
        }
        swap32(a, b);
        y[p] = Op::f(a, b);
    }
#pragma unroll
    for (int p = 0; p < N / 4; p++) {
        float a = y[2 * p], b = y[2 * p + 1];
        swap16(a, b);
        z[p] = Op::f(a, b);
    }
}

// Index (within x[]) of the value z[p] holds after col_reduce_scatter.
__device__ __forceinline__ int scatter_index(const Lane &c, int p)
{
    return 4 * p + 2 * ((c.lane >> 4) & 1) + ((c.lane >> 5) & 1);
}

// Inverse distribution of col_reduce_scatter<G, Op, 8>: z[p] holds the
// value of index 4p + e (e = 2*bit4(lane) + bit5(lane)); afterwards every
// lane holds all eight, y[i] = the value of index i.  swap16 with both
// operands equal hands each lane the bit4 = 0 lane's value in the first and
// the bit4 = 1 lane's in the second; swap32 does the same for bit5.
__device__ __forceinline__ void col_allgather(const float (&z)[2], float (&y)[8])
{
#pragma unroll
    for (int p = 0; p < 2; p++) {
        float a = z[p], b = z[p];
        swap16(a, b);                 // a: index 4p + bit5, b: 4p + 2 + bit5
        float a0 = a, a1 = a, b0 = b, b1 = b;
        swap32(a0, a1);               // a0: 4p,     a1: 4p + 1
        swap32(b0, b1);               // b0: 4p + 2, b1: 4p + 3
        y[4 * p + 0] = a0;
        y[4 * p + 1] = a1;
        y[4 * p + 2] = b0;
        y[4 * p + 3] = b1;
    }
}

// All-reduce of one value over the RGW row-group lanes (column direction).
template <class G, class Op>
__device__ __forceinline__ float col_allreduce(float x)
{
    if constexpr (G::NCB == 8) x = Op::f(x, dpp<DPP_ROR8>(x));
    float a = x, b = x;
    swap32(a, b);
    x = Op::f(a, b);
    a = x;
    b = x;
    swap16(a, b);
    return Op::f(a, b);
}

// --------------------------------------------------------------- LDS sync
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Load 8 consecutive io-dtype values starting at element `off`.
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, size_t off, float (&out)[8])
{
    if constexpr (BF16) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + off);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off);
        float4 a = p[0], b = p[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, size_t off)
{
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[off]);
    else return reinterpret_cast<const float *>(base)[off];
}

template <bool BF16>
__device__ __forceinline__ void store1(void *base, size_t off, float x)
{
    if constexpr (BF16) reinterpret_cast<uint16_t *>(base)[off] = f32_to_bf16(x);
    else reinterpret_cast<float *>(base)[off] = x;
}

// The thread's 8 row values of a per-row vector: rows row0..row0+3 and
// row0+RGW*4..+3 are two aligned runs of 4, loaded as two vectors.
template <class G, bool BF16>
__device__ __forceinline__ void load_rows(const void *base, size_t head_off, int row0, float (&out)[8])
{
    if constexpr (BF16) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + head_off + row0;
        const uint2 a = *reinterpret_cast<const uint2 *>(p);
        const uint2 b = *reinterpret_cast<const uint2 *>(p + G::RGW * 4);
        out[0] = __uint_as_float(a.x << 16); out[1] = __uint_as_float(a.x & 0xFFFF0000u);
        out[2] = __uint_as_float(a.y << 16); out[3] = __uint_as_float(a.y & 0xFFFF0000u);
        out[4] = __uint_as_float(b.x << 16); out[5] = __uint_as_float(b.x & 0xFFFF0000u);
        out[6] = __uint_as_float(b.y << 16); out[7] = __uint_as_float(b.y & 0xFFFF0000u);
    } else {
        const float *p = reinterpret_cast<const float *>(base) + head_off + row0;
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + G::RGW * 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

template <class G>
__device__ __forceinline__ void load_rows_f32(const float *p, float (&out)[8])
{
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + G::RGW * 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ __forceinline__ void load_f32x8(const float *p, float (&out)[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ __forceinline__ void store_f32x8(float *p, const float (&v)[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// 8-byte loads / stores with the non-temporal hint: the per-step decode
// streams every head's codes once per call (read, then overwritten in
// place), so they should not displace other lines in the caches.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 load_nt8(const int8_t *p)
{
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(t.x, t.y);
}

__device__ __forceinline__ void store_nt8(int8_t *p, uint2 v)
{
    const u32x2 t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2 *>(p));
}

// int8 x 8 (one row of the block) -> fp32
__device__ __forceinline__ void unpack8(uint2 q, float (&out)[8])
{
    const int32_t lo = (int32_t)q.x, hi = (int32_t)q.y;
    out[0] = (float)(int8_t)(lo & 0xff);
    out[1] = (float)(int8_t)((lo >> 8) & 0xff);
    out[2] = (float)(int8_t)((lo >> 16) & 0xff);
    out[3] = (float)(lo >> 24);
    out[4] = (float)(int8_t)(hi & 0xff);
    out[5] = (float)(int8_t)((hi >> 8) & 0xff);
    out[6] = (float)(int8_t)((hi >> 16) & 0xff);
    out[7] = (float)(hi >> 24);
}

// Low bytes of four fp32 bit patterns -> one dword (byte i from value i).
__device__ __forceinline__ uint32_t pack_low_bytes(float a, float b, float c, float d)
{
    uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x04000c0cu);
    return lo | hi;
}

// Low bytes of four words -> one dword (byte i from word i).
__device__ __forceinline__ uint32_t pack_low_bytes_u(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);
    return lo | hi;
}

// ------------------------------------------------------------ packed codes
// BITS-bit two's complement codes in [-Qb, Qb], Qb = 2^(BITS-1) - 1.  One
// row of DV codes takes DV*BITS/8 bytes:
//   8: one byte per code;
//   4: code j in byte j/2, bits 4(j%2)..+3;
//   6: the 8 codes of columns 8k..8k+7 form a 48-bit record (column 8k+e in
//      bits 6e..6e+5) whose low 32 bits are bytes 4k..4k+3 and whose high
//      16 bits are bytes DV/2 + 2k, +1: any code is one signed bit-field
//      extract (the one straddling the two words, one funnel shift more).
// A lane's 8 columns 8cb..8cb+7 are one 8-byte word (8 bits), one 4-byte
// word (4 bits), or a 4-byte and a 2-byte word (6 bits): CodeWord a, b.
template <int BITS>
constexpr int code_qmax() { return (1 << (BITS - 1)) - 1; }

template <class G, int BITS>
constexpr int code_row_bytes() { return G::DV * BITS / 8; }

struct CodeWord {
    uint32_t a, b;
};

template <class G, int BITS, bool NT = false>
__device__ __forceinline__ CodeWord load_code8(const int8_t *row, int cb)
{
    CodeWord w;
    if constexpr (BITS == 8) {
        uint2 v;
        if constexpr (NT) v = load_nt8(row + cb * 8);
        else v = *reinterpret_cast<const uint2 *>(row + cb * 8);
        w.a = v.x;
        w.b = v.y;
    } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(row + cb * 4);
        if constexpr (NT) w.a = __builtin_nontemporal_load(p);
        else w.a = *p;
        w.b = 0;
        if constexpr (BITS == 6) {
            const uint16_t *q = reinterpret_cast<const uint16_t *>(row + G::DV / 2 + cb * 2);
            if constexpr (NT) w.b = __builtin_nontemporal_load(q);
            else w.b = *q;
        }
    }
    return w;
}

template <class G, int BITS, bool NT = false>
__device__ __forceinline__ void store_code8(int8_t *row, int cb, const CodeWord &w)
{
    if constexpr (BITS == 8) {
        if constexpr (NT) store_nt8(row + cb * 8, make_uint2(w.a, w.b));
        else *reinterpret_cast<uint2 *>(row + cb * 8) = make_uint2(w.a, w.b);
    } else {
        uint32_t *p = reinterpret_cast<uint32_t *>(row + cb * 4);
        if constexpr (NT) __builtin_nontemporal_store(w.a, p);
        else *p = w.a;
        if constexpr (BITS == 6) {
            uint16_t *q = reinterpret_cast<uint16_t *>(row + G::DV / 2 + cb * 2);
            if constexpr (NT) __builtin_nontemporal_store((uint16_t)w.b, q);
            else *q = (uint16_t)w.b;
        }
    }
}

// The 8 codes of a CodeWord as fp32 (exact).
template <int BITS>
__device__ __forceinline__ void unpack_code8(const CodeWord &w, float (&out)[8])
{
    if constexpr (BITS == 8) {
        unpack8(make_uint2(w.a, w.b), out);
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int e = 0; e < 8; e++) out[e] = (float)((int32_t)(w.a << (28 - 4 * e)) >> 28);
    } else {
#pragma unroll
        for (int e = 0; e < 5; e++) out[e] = (float)((int32_t)(w.a << (26 - 6 * e)) >> 26);
        const uint32_t mid = __builtin_amdgcn_alignbit(w.b, w.a, 30);   // record bits 30..61
        out[5] = (float)((int32_t)(mid << 26) >> 26);
        out[6] = (float)((int32_t)(w.b << 22) >> 26);
        out[7] = (float)((int32_t)(w.b << 16) >> 26);
    }
}

// Pack 8 rounded codes: y[e] are fma(Y, iota, RINT_MAGIC) results, whose
// low byte is the code in two's complement.
template <int BITS>
__device__ __forceinline__ CodeWord pack_code8(const float (&y)[8])
{
    CodeWord w;
    uint32_t u[8];
#pragma unroll
    for (int e = 0; e < 8; e++) u[e] = __float_as_uint(y[e]);
    if constexpr (BITS == 8) {
        w.a = pack_low_bytes_u(u[0], u[1], u[2], u[3]);
        w.b = pack_low_bytes_u(u[4], u[5], u[6], u[7]);
    } else if constexpr (BITS == 4) {
        uint32_t n[4];
#pragma unroll
        for (int i = 0; i < 4; i++) n[i] = (u[2 * i] & 0xFu) | (u[2 * i + 1] << 4);   // low byte: the pair
        w.a = pack_low_bytes_u(n[0], n[1], n[2], n[3]);
        w.b = 0;
    } else {
        uint32_t f[8];
#pragma unroll
        for (int e = 0; e < 8; e++) f[e] = u[e] & 0x3Fu;
        w.a = f[0] | (f[1] << 6) | (f[2] << 12) | (f[3] << 18) | (f[4] << 24) | (f[5] << 30);
        w.b = (f[5] >> 2) | (f[6] << 4) | (f[7] << 10);
    }
    return w;
}

// fma(y, iota, 1.5*2^23) rounds the exact value y*iota + 1.5*2^23 once, at
// unit spacing (the sum lies in [2^23, 2^24) for |y*iota| < 2^22), so it
// equals 1.5*2^23 + rint_even(y*iota) with the product taken exactly; the
// low mantissa byte is that integer mod 256 (two's complement int8).
constexpr float RINT_MAGIC = 12582912.0f;

}  // namespace gdnq
