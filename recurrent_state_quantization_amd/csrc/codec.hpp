// codec.hpp -- device-side state codec and Compensator Token extraction on
// the register tile (see tile.hpp for the layout).  Every kernel that writes
// codes calls these functions, so the stand-alone codec and the codec fused
// into the decode/flush kernels are the same code.
//
// Codec, layout 0 (LeapQuant project page, residual-smoothing paragraph:
// rows are balanced before quantization; STEPQuant page: key-row and
// value-column scales).  Per head, each step one IEEE fp32 operation with
// round to nearest even and no fused multiply-add (the library is built with
// -ffp-contract=off and correctly rounded divide and sqrt):
//   r_i = max_j |X_ij|; s_i = sqrt(r_i); rho_i = 1/s_i (0 if s_i = 0)
//   Y_ij = X_ij rho_i; m_j = max_i |Y_ij|
//   c_j = m_j/127, iota_j = 127/m_j (both 0 if m_j = 0 or 127/m_j overflows)
//   Q_ij = rint_even(Y_ij iota_j), the exact product rounded once (one fma)
// No clamp is applied: |Y_ij| <= m_j and iota_j <= (127/m_j)(1 + 2^-24), so
// |Y_ij iota_j| <= 127 (1 + 2^-24) < 127.5 and the code is in [-127, 127].
//
// Layout 1 (DAMP abstract: high-risk channels in higher precision, the rest
// INT8): listed rows -> IEEE fp16 (round to nearest even, saturating at
// +-65504); other rows -> the per-column steps above with s = 1 and m_j
// taken over those rows only; their codes are stored compacted.
//
// Compensator Tokens (LeapQuant, Compensator Tokens paragraph): r rank-1
// terms taken out by power iteration before the codec runs; see
// power_deflate.
#pragma once

#include "launch.hpp"
#include "tile.hpp"

namespace gdnq {

// Row stride of the transposed row-maxima table (padded, 16-byte rows).
template <class G>
constexpr int row_table_stride() { return G::ROWS_W + 4; }

template <class G>
struct CodecLds {
    float rho[G::DK];
    float red[2][G::NW][G::DV];
    float iota[G::DV];
    // per wave: the lanes' row maxima over their 8 columns, [column block][row]
    alignas(16) float rt[G::NW][G::NCB][row_table_stride<G>()];
    int misc;
    int flag[2][G::NW];  // per-wave flags of block_any, two sets used in turn
};

// Workgroup OR of a per-thread flag: each wave's ballot goes to its slot of
// flag set `parity`, and after the barrier every thread ORs the slots.
// Consecutive calls must alternate `parity`: the write to a set then
// follows the barrier of the call in between, which every read of that
// set precedes.
template <class G>
__device__ __forceinline__ bool block_any(CodecLds<G> &L, const Lane &c, bool x, int parity)
{
    const bool wave_any = __builtin_amdgcn_ballot_w64(x) != 0;
    if (c.lane == 0) L.flag[parity][c.w] = wave_any ? 1 : 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < G::NW; w++) any |= L.flag[parity][w];
    return any != 0;
}

// Which of a thread's 8 rows are DAMP (fp16) rows, their slot in hp_idx and,
// for the other rows, their index among the compacted INT8 rows.  hp lists
// the n_hp <= 64 DAMP rows strictly ascending (in LDS or global memory, the
// same list for every thread), so a row's slot and its compacted index both
// follow from the number of DAMP rows below it.  Lane t of each wave reads
// hp[t]; the rows go into a DK-bit mask (one word per 32 rows) by an OR
// across the wave; a thread's rows lie in its wave's words, and each takes
// a population count of the bits below it.
struct RowMap {
    int slot[8];   // -1: INT8 row
    int crow[8];   // compacted INT8 row index (valid when slot < 0)
};

__device__ __forceinline__ uint32_t wave_or(uint32_t x)
{
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, true);   // quad_perm [1,0,3,2]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, true);   // quad_perm [2,3,0,1]
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, true);  // row_half_mirror
    x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, true);  // row_mirror
    return (uint32_t)(__builtin_amdgcn_readlane((int)x, 0) | __builtin_amdgcn_readlane((int)x, 16) |
                      __builtin_amdgcn_readlane((int)x, 32) | __builtin_amdgcn_readlane((int)x, 48));
}

template <class G, class P>
__device__ __forceinline__ RowMap row_map(const Lane &c, P hp, int n_hp)
{
    constexpr int NWD = G::DK / 32;
    const int hv = c.lane < n_hp ? (int)hp[c.lane] : -1;
    uint32_t m[NWD];
#pragma unroll
    for (int w = 0; w < NWD; w++) m[w] = wave_or(hv >= 0 && (hv >> 5) == w ? 1u << (hv & 31) : 0u);
    RowMap r;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int i = row_of<G>(c, k);
        // the word of row i and the DAMP rows in the words before it
        // (wave-uniform: the wave's rows span whole words)
        const int wd = (c.w * G::ROWS_W + (k >> 2) * G::RGW * 4) >> 5;
        uint32_t word = 0u;
        int before = 0;
#pragma unroll
        for (int w = 0; w < NWD; w++) {
            word = w == wd ? m[w] : word;
            before += w < wd ? __builtin_popcount(m[w]) : 0;
        }
        const int b = i & 31;
        const int below = before + __builtin_popcount(word & ((1u << b) - 1u));
        r.slot[k] = (word >> b) & 1u ? below : -1;
        r.crow[k] = i - below;
    }
    return r;
}


// m / Qb rounded to nearest even for the code range's Qb (127, 31 or 7):
// q0 = m r, e = m - q0 Qb (exact, one fma), q1 = q0 + e r, with r = 1/Qb
// rounded.  Checked exhaustively, for every positive finite fp32 m and
// each of the three Qb, to equal the correctly rounded quotient (the
// division sequence it replaces costs about three times the instructions).
template <int BITS>
__device__ __forceinline__ float div_by_qmax(float m)
{
    constexpr float QB = (float)code_qmax<BITS>();
    constexpr float R = 1.0f / QB;
    const float q0 = m * R;
    return fmaf(fmaf(-q0, QB, m), R, q0);
}

// 1/s rounded to nearest even for the row scales the codec forms (s is the
// rounded square root of a positive finite fp32, so 2^-75 <= s < 2^65): the
// hardware reciprocal r0 (about one ulp) and one correction with the exact
// residual 1 - s r0.  Compared on gfx950 with the IEEE quotient 1.0f / s for
// every fp32 s in [2^-75, 2^65): identical for all of them.
__device__ __forceinline__ float recip_row_scale(float s)
{
    const float r0 = __builtin_amdgcn_rcpf(s);
    return fmaf(fmaf(-s, r0, 1.0f), r0, r0);
}

// Column scales from the per-wave column maxima in L.red[0]; thread t < DV
// owns column t.  Writes c to global memory and iota to LDS.  Codes of
// BITS bits span [-Qb, Qb]: c = m/Qb, iota = Qb/m.
template <class G, int BITS = 8>
__device__ __forceinline__ void column_scales(const Lane &c, CodecLds<G> &L, float *__restrict__ col_scale)
{
    constexpr float QB = (float)code_qmax<BITS>();
    if (c.t < G::DV) {
        float m = L.red[0][0][c.t];
#pragma unroll
        for (int w = 1; w < G::NW; w++) m = fmaxf(m, L.red[0][w][c.t]);
        float cj = 0.0f, io = 0.0f;
        if (m > 0.0f) {
            io = QB / m;
            if (__builtin_isinf(io)) io = 0.0f;
            else cj = div_by_qmax<BITS>(m);
        }
        col_scale[c.t] = cj;
        L.iota[c.t] = io;
    }
}

// Per-thread column maxima m[8] -> L.red[0][w][*] (wave partials).
template <class G>
__device__ __forceinline__ void column_max_to_lds(const Lane &c, CodecLds<G> &L, const float (&m)[8])
{
    float z[2];
    col_reduce_scatter<G, OpMax, 8>(m, z);
#pragma unroll
    for (int p = 0; p < 2; p++) L.red[0][c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
}

// Layout-0 codec of the register tile P (overwritten with Y).  Writes this
// head's BITS-bit codes (DK rows of code_row_bytes), row scales [DK] and
// column scales [DV]; STREAM marks the code stores non-temporal.
template <class G, bool STREAM = false, int BITS = 8>
__device__ void codec_rowcol(float (&P)[8][8], const Lane &c, CodecLds<G> &L, int8_t *__restrict__ codes,
                             float *__restrict__ row_scale, float *__restrict__ col_scale)
{
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        float m = fabsf(P[k][0]);
#pragma unroll
        for (int j = 1; j < 8; j++) m = fmaxf(m, fabsf(P[k][j]));
        r[k] = m;
    }
    const int row0 = row0_of<G>(c);
    {
        // Row maxima, transposed through LDS inside the wave (a row group
        // lives in one wave): each lane stores its 8 partials, two runs of 4
        // rows of its column block; lane L then takes the NCB/PAIR partials
        // of the wave's row L/PAIR (PAIR = 64/ROWS_W lanes per row, joined by
        // one DPP step) and forms that row's scale.
        constexpr int RS = row_table_stride<G>();
        constexpr int PAIR = 64 / G::ROWS_W;
        float *rt = &L.rt[c.w][0][0];
        *reinterpret_cast<float4 *>(rt + c.cb * RS + 4 * c.rgl) = make_float4(r[0], r[1], r[2], r[3]);
        *reinterpret_cast<float4 *>(rt + c.cb * RS + G::RGW * 4 + 4 * c.rgl) = make_float4(r[4], r[5], r[6], r[7]);
        wave_lds_sync();
        const int lr = c.lane / PAIR, part = c.lane % PAIR;
        const float *col = rt + part * (G::NCB / PAIR) * RS + lr;
        float rk = col[0];
#pragma unroll
        for (int e = 1; e < G::NCB / PAIR; e++) rk = fmaxf(rk, col[e * RS]);
        if constexpr (PAIR == 2) rk = fmaxf(rk, dpp<DPP_XOR1>(rk));
        const float s = (rk > 0.0f) ? sqrtf(rk) : 0.0f;
        const float rho = (s > 0.0f) ? recip_row_scale(s) : 0.0f;
        if (part == 0) {
            const int i = c.w * G::ROWS_W + lr;
            L.rho[i] = rho;
            row_scale[i] = s;
        }
    }
    wave_lds_sync();
    float rho[8];
    load_rows_f32<G>(L.rho + row0, rho);
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) m[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            P[k][j] = P[k][j] * rho[k];
            m[j] = fmaxf(m[j], fabsf(P[k][j]));
        }
    float io[8];
    column_max_to_lds<G>(c, L, m);
    __syncthreads();
    column_scales<G, BITS>(c, L, col_scale);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; j++) io[j] = L.iota[c.cb * 8 + j];
    constexpr int RB = code_row_bytes<G, BITS>();
    int8_t *rbase = codes + (size_t)row0 * RB;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; j++) y[j] = fmaf(P[k][j], io[j], RINT_MAGIC);
        store_code8<G, BITS, STREAM>(rbase + koff<G>(k) * RB, c.cb, pack_code8<BITS>(y));
    }
}

// Static-scale codec (the STEPQuant reading: row and column scales fitted
// offline and kept): codes of P under the fixed reciprocals of the lane's
// rows rho[k] and columns io[j] -- the integer nearest to the exact product
// (P rho) io, clamped to [-Qb, Qb] (the med3 clamp on RINT_MAGIC + q keeps
// the code in the low bits).  No reduction, no barrier; scales unchanged.
template <class G, bool STREAM, int BITS>
__device__ __forceinline__ void codec_static(const float (&P)[8][8], const Lane &c, const float (&rho)[8],
                                             const float (&io)[8], int8_t *__restrict__ codes)
{
    constexpr float QB = (float)code_qmax<BITS>();
    constexpr int RB = code_row_bytes<G, BITS>();
    int8_t *rbase = codes + (size_t)row0_of<G>(c) * RB;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            y[j] = __builtin_amdgcn_fmed3f(fmaf(P[k][j] * rho[k], io[j], RINT_MAGIC), RINT_MAGIC - QB, RINT_MAGIC + QB);
        store_code8<G, BITS, STREAM>(rbase + koff<G>(k) * RB, c.cb, pack_code8<BITS>(y));
    }
}

// fp32 -> IEEE fp16 bits, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float x)
{
    x = fminf(fmaxf(x, -65504.0f), 65504.0f);
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Layout-1 (DAMP) codec of P.  codes_c: this head's compacted INT8 rows
// [DK-n_hp][DV]; hp_rows: [n_hp][DV] fp16 bits.
template <class G>
__device__ void codec_damp(float (&P)[8][8], const Lane &c, CodecLds<G> &L, const RowMap &rm,
                           int8_t *__restrict__ codes_c, float *__restrict__ col_scale,
                           uint16_t *__restrict__ hp_rows)
{
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) m[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const bool hp = rm.slot[k] >= 0;
#pragma unroll
        for (int j = 0; j < 8; j++) m[j] = hp ? m[j] : fmaxf(m[j], fabsf(P[k][j]));
    }
    column_max_to_lds<G>(c, L, m);
    __syncthreads();
    column_scales<G>(c, L, col_scale);
    __syncthreads();
    float io[8];
#pragma unroll
    for (int j = 0; j < 8; j++) io[j] = L.iota[c.cb * 8 + j];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        if (rm.slot[k] >= 0) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                h[j] = (uint32_t)f32_to_f16_sat(P[k][2 * j]) | ((uint32_t)f32_to_f16_sat(P[k][2 * j + 1]) << 16);
            *reinterpret_cast<uint4 *>(hp_rows + (size_t)rm.slot[k] * G::DV + c.cb * 8) =
                make_uint4(h[0], h[1], h[2], h[3]);
        } else {
            float y[8];
#pragma unroll
            for (int j = 0; j < 8; j++) y[j] = fmaf(P[k][j], io[j], RINT_MAGIC);
            uint2 q;
            q.x = pack_low_bytes(y[0], y[1], y[2], y[3]);
            q.y = pack_low_bytes(y[4], y[5], y[6], y[7]);
            *reinterpret_cast<uint2 *>(codes_c + (size_t)rm.crow[k] * G::DV + c.cb * 8) = q;
        }
    }
}

// Column sums of per-thread partials y[8] over the whole tile, returned to
// every thread for its own 8 columns.  Uses L.red[buf]; the caller
// alternates buf between calls so one barrier per call suffices.
template <class G>
__device__ __forceinline__ void column_sum_all(const Lane &c, float (&red)[G::NW][G::DV], const float (&yp)[8],
                                               float (&y)[8])
{
    float z[2];
    col_reduce_scatter<G, OpSum, 8>(yp, z);
#pragma unroll
    for (int p = 0; p < 2; p++) red[c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
    __syncthreads();
    load_f32x8(&red[0][c.cb * 8], y);
#pragma unroll
    for (int w = 1; w < G::NW; w++) {
        float t[8];
        load_f32x8(&red[w][c.cb * 8], t);
#pragma unroll
        for (int j = 0; j < 8; j++) y[j] += t[j];
    }
}

// Column sums of per-thread partials yp[8] over the whole tile, finished
// only for the two columns this lane holds after the in-wave reduce-scatter:
// z[p] = column cb*8 + scatter_index(c, p), the wave partials added in wave
// order.  Uses `red`; the caller alternates buffers between calls so one
// barrier per call suffices.
template <class G>
__device__ __forceinline__ void column_sum_scattered(const Lane &c, float (&red)[G::NW][G::DV],
                                                     const float (&yp)[8], float (&z)[2])
{
    float zp[2];
    col_reduce_scatter<G, OpSum, 8>(yp, zp);
#pragma unroll
    for (int p = 0; p < 2; p++) red[c.w][c.cb * 8 + scatter_index(c, p)] = zp[p];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; p++) {
        const int col = c.cb * 8 + scatter_index(c, p);
        float s = red[0][col];
#pragma unroll
        for (int w = 1; w < G::NW; w++) s += red[w][col];
        z[p] = s;
    }
}

// Full row sums x[8] of the lane's 8 rows from its per-row partial sums
// xp[8] (over its 8 columns), transposed through LDS inside the wave like
// the codec's row maxima: the partials go to the wave's table L.rt, lane L
// adds the NCB/PAIR partials of the wave's row L/PAIR (one DPP step joins
// the pair) and stores the sum in L.rho, and every lane reads back its 8
// rows.  Uses L.rt[w] and the wave's rows of L.rho; consecutive calls in a
// wave need no other synchronization.
template <class G>
__device__ __forceinline__ void row_sums(CodecLds<G> &L, const Lane &c, const float (&xp)[8], float (&x)[8])
{
    constexpr int RS = row_table_stride<G>();
    constexpr int PAIR = 64 / G::ROWS_W;
    float *rt = &L.rt[c.w][0][0];
    *reinterpret_cast<float4 *>(rt + c.cb * RS + 4 * c.rgl) = make_float4(xp[0], xp[1], xp[2], xp[3]);
    *reinterpret_cast<float4 *>(rt + c.cb * RS + G::RGW * 4 + 4 * c.rgl) = make_float4(xp[4], xp[5], xp[6], xp[7]);
    wave_lds_sync();
    const int lr = c.lane / PAIR, part = c.lane % PAIR;
    const float *col = rt + part * (G::NCB / PAIR) * RS + lr;
    float s = col[0];
#pragma unroll
    for (int e = 1; e < G::NCB / PAIR; e++) s += col[e * RS];
    if constexpr (PAIR == 2) s += dpp<DPP_XOR1>(s);
    if (part == 0) L.rho[c.w * G::ROWS_W + lr] = s;
    wave_lds_sync();
    load_rows_f32<G>(L.rho + row0_of<G>(c), x);
}

// One power-iteration step y = P^T (P v); when |y|^2 != 0, v <- y / |y|
// (v is kept otherwise).  Returns |y|^2, the same value in every lane.
// The norm and the scaling run on the two columns a lane holds after the
// reduce-scatter; the scaled values are then gathered back to all lanes.
// Row sums of P v for the lane's 8 rows: through LDS (LDS_ROWS) or by a DPP
// all-reduce per row.  The LDS form issues fewer instructions and pays two
// wave-local LDS round trips, which the other resident workgroups hide at
// four per CU; at two or three per CU (the DAMP flush) the DPP form is
// faster.
template <class G, bool LDS_ROWS>
__device__ __forceinline__ void row_dots(const float (&P)[8][8], const Lane &c, CodecLds<G> &L, const float (&v)[8],
                                         float (&x)[8])
{
    float xp[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        float s = P[k][0] * v[0];
#pragma unroll
        for (int j = 1; j < 8; j++) s = fmaf(P[k][j], v[j], s);
        xp[k] = s;
    }
    if constexpr (LDS_ROWS) {
        row_sums<G>(L, c, xp, x);
    } else {
#pragma unroll
        for (int k = 0; k < 8; k++) x[k] = row_sum<G>(xp[k]);
    }
}

template <class G, bool LDS_ROWS>
__device__ __forceinline__ float power_step(const float (&P)[8][8], const Lane &c, CodecLds<G> &L,
                                            float (&red)[G::NW][G::DV], float (&v)[8])
{
    float x[8];
    row_dots<G, LDS_ROWS>(P, c, L, v, x);
    float yp[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float s = P[0][j] * x[0];
#pragma unroll
        for (int k = 1; k < 8; k++) s = fmaf(P[k][j], x[k], s);
        yp[j] = s;
    }
    float z[2];
    column_sum_scattered<G>(c, red, yp, z);
    // each column is held by one lane of the wave (by two lanes that differ
    // in lane bit 3 when NCB = 8: the all-reduce then counts it twice)
    float n2 = fmaf(z[1], z[1], z[0] * z[0]);
    n2 = col_allreduce<G, OpSum>(row_sum<G>(n2));
    if constexpr (G::NCB == 8) n2 *= 0.5f;
    if (n2 != 0.0f) {
        // the normalization only rescales the iterate: the hardware
        // reciprocal square root (about 1 ulp) is accurate enough
        const float inv = __builtin_amdgcn_rsqf(n2);
        z[0] *= inv;
        z[1] *= inv;
        col_allgather(z, v);
    }
    return n2;
}

// Compensator Tokens by power iteration with sequential deflation, on the
// register tile P (the rebuilt state; left holding the residual).
// For each c < r: v = all-equal unit vector; `iters` times
//   y = P^T (P v); if |y| = 0: on the first step restart from the unit
//   vector of P's largest column (lowest index on ties) when P != 0,
//   otherwise keep v; v = y/|y|.
// p = P v, w = v (fp32), P -= p w^T.  P == 0 gives p = w = 0.
// comp_k: this head's [r][DK]; comp_v: [r][DV].  LDS_ROWS: see row_dots.
template <class G, bool LDS_ROWS = true>
__device__ void power_deflate(float (&P)[8][8], const Lane &c, CodecLds<G> &L, int r, int iters,
                              float *__restrict__ comp_k, float *__restrict__ comp_v)
{
    for (int cc = 0; cc < r; cc++) {
        bool nz = false;
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) nz |= (P[k][j] != 0.0f);
        const bool any = block_any<G>(L, c, nz, cc & 1);
        float v[8], p[8];
        if (!any) {
#pragma unroll
            for (int j = 0; j < 8; j++) { v[j] = 0.0f; p[j] = 0.0f; }
        } else {
            const float v0 = (G::DV == 128) ? 0.08838834764831845f : 0.125f;
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = v0;
            // first step, with the restart rule; L.red[0] is free here (the
            // barrier of block_any follows every earlier read of it)
            float n2 = power_step<G, LDS_ROWS>(P, c, L, L.red[0], v);
            if (n2 == 0.0f) {  // uniform: every lane holds the same n2
                float cn[8], cs[8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    float s = P[0][j] * P[0][j];
#pragma unroll
                    for (int k = 1; k < 8; k++) s = fmaf(P[k][j], P[k][j], s);
                    cn[j] = s;
                }
                column_sum_all<G>(c, L.red[1], cn, cs);
                if (c.t == 0) {
                    int best = 0;
                    float bv = -1.0f;
                    for (int j = 0; j < G::DV; j++) {
                        float s = L.red[1][0][j];
                        for (int w = 1; w < G::NW; w++) s += L.red[1][w][j];
                        if (s > bv) { bv = s; best = j; }
                    }
                    L.misc = best;
                }
                __syncthreads();
                const int jb = L.misc;
#pragma unroll
                for (int j = 0; j < 8; j++) v[j] = (c.cb * 8 + j == jb) ? 1.0f : 0.0f;
                n2 = power_step<G, LDS_ROWS>(P, c, L, L.red[0], v);
            }
            if (n2 != 0.0f) {
                // remaining steps two at a time so each LDS buffer is fixed;
                // consecutive steps alternate buffers, so one barrier per
                // step orders every read of a buffer before its next write
                for (int it = 1; it < iters; it += 2) {
                    if (power_step<G, LDS_ROWS>(P, c, L, L.red[1], v) == 0.0f) break;
                    if (it + 1 >= iters) break;
                    if (power_step<G, LDS_ROWS>(P, c, L, L.red[0], v) == 0.0f) break;
                }
            }
            row_dots<G, LDS_ROWS>(P, c, L, v, p);
        }
        if (c.cb == 0) {
#pragma unroll
            for (int k = 0; k < 8; k++) comp_k[(size_t)cc * G::DK + row_of<G>(c, k)] = p[k];
        }
        if (c.w == 0 && c.rgl == 0) store_f32x8(comp_v + (size_t)cc * G::DV + c.cb * 8, v);
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) P[k][j] = fmaf(-p[k], v[j], P[k][j]);
    }
    if (r > 0) __syncthreads();  // L.red is reused by the codec
}

}  // namespace gdnq
