// codec.hip -- stand-alone state encode / decode kernels.
//
// gdn_state_quantize: fp32 state -> Compensator Tokens (power iteration) ->
// residual -> codec of the chosen layout (LeapQuant project page,
// Compensator Tokens and residual-smoothing paragraphs; DAMP abstract for
// layout 1).  It is the back half of the window flush and uses the same
// device code (codec.hpp).
//
// gdn_state_dequantize: codes -> D(Q) + DAMP fp16 rows + sum_c p_c w_c^T,
// the fixed state of a window start.
#include "codec.hpp"
#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {

struct QuantArgs {
    const float *S;
    int8_t *codes;
    float *row_scale, *col_scale, *comp_k, *comp_v, *g_cur;
    uint16_t *hp_rows;
    const int32_t *hp_idx;
    float *prequant;
    float *S_out;
    int r, n_hp, iters, kda;
};

template <class G, bool DAMP, int BITS>
__global__ __launch_bounds__(G::NT, 2) void quantize_kernel(QuantArgs A)
{
    static_assert(!DAMP || BITS == 8, "the DAMP layout keeps 8-bit codes");
    __shared__ CodecLds<G> L;
    __shared__ int hp[MAX_HP];
    const Lane c = lane_coords<G>();
    const size_t h = __builtin_amdgcn_workgroup_id_x();
    constexpr size_t E = (size_t)G::DK * G::DV;
    const int n_hp = DAMP ? A.n_hp : 0;
    if (DAMP && c.t < n_hp) hp[c.t] = A.hp_idx[h * n_hp + c.t];
    float P[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) load_f32x8(A.S + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
    __syncthreads();
    power_deflate<G, !DAMP>(P, c, L, A.r, A.iters, A.comp_k + h * A.r * G::DK, A.comp_v + h * A.r * G::DV);
    if (A.prequant) {
#pragma unroll
        for (int k = 0; k < 8; k++) store_f32x8(A.prequant + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
    }
    if constexpr (DAMP) {
        const RowMap rm = row_map<G>(c, hp, n_hp);
        codec_damp<G>(P, c, L, rm, A.codes + h * (size_t)(G::DK - n_hp) * G::DV, A.col_scale + h * G::DV,
                      A.hp_rows + h * n_hp * G::DV);
    } else {
        codec_rowcol<G, false, BITS>(P, c, L, A.codes + h * (size_t)G::DK * code_row_bytes<G, BITS>(),
                                     A.row_scale + h * G::DK, A.col_scale + h * G::DV);
    }
    if (A.g_cur && c.t < G::DK) {
        if (A.kda) A.g_cur[h * G::DK + c.t] = 1.0f;
        else if (c.t == 0) A.g_cur[h] = 1.0f;
    }
}

// Encode under fixed static scales: the rho plane follows the row scales and
// the iota plane the column scales (row_scale + nh*DK, col_scale + nh*DV).
template <class G, int BITS>
__global__ __launch_bounds__(G::NT) void quantize_static_kernel(QuantArgs A, size_t nh)
{
    const Lane c = lane_coords<G>();
    const size_t h = __builtin_amdgcn_workgroup_id_x();
    constexpr size_t E = (size_t)G::DK * G::DV;
    const int row0 = row0_of<G>(c);
    float P[8][8], rho[8], io[8];
#pragma unroll
    for (int k = 0; k < 8; k++) load_f32x8(A.S + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
    load_rows_f32<G>(A.row_scale + nh * G::DK + h * G::DK + row0, rho);
    load_f32x8(A.col_scale + nh * G::DV + h * G::DV + c.cb * 8, io);
    codec_static<G, false, BITS>(P, c, rho, io, A.codes + h * (size_t)G::DK * code_row_bytes<G, BITS>());
}

template <class G, bool DAMP, int BITS>
__global__ __launch_bounds__(G::NT) void dequantize_kernel(QuantArgs A)
{
    static_assert(!DAMP || BITS == 8, "the DAMP layout keeps 8-bit codes");
    constexpr int RB = code_row_bytes<G, BITS>();
    __shared__ int hp[MAX_HP];
    const Lane c = lane_coords<G>();
    const size_t h = __builtin_amdgcn_workgroup_id_x();
    constexpr size_t E = (size_t)G::DK * G::DV;
    const int n_hp = DAMP ? A.n_hp : 0;
    if (DAMP && c.t < n_hp) hp[c.t] = A.hp_idx[h * n_hp + c.t];
    __syncthreads();
    RowMap rm;
    if constexpr (DAMP) rm = row_map<G>(c, hp, n_hp);
    const int8_t *codes = A.codes + h * (size_t)(G::DK - n_hp) * RB;
    float cc[8];
    load_f32x8(A.col_scale + h * G::DV + c.cb * 8, cc);
    float P[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int i = row_of<G>(c, k);
        if (DAMP && rm.slot[k] >= 0) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(A.hp_rows + (h * n_hp + rm.slot[k]) * G::DV + c.cb * 8);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                P[k][2 * e] = f16_to_f32((uint16_t)(w[e] & 0xFFFFu));
                P[k][2 * e + 1] = f16_to_f32((uint16_t)(w[e] >> 16));
            }
        } else {
            const int row = DAMP ? rm.crow[k] : i;
            float X[8];
            unpack_code8<BITS>(load_code8<G, BITS>(codes + (size_t)row * RB, c.cb), X);
            const float s = DAMP ? 1.0f : A.row_scale[h * G::DK + i];
#pragma unroll
            for (int j = 0; j < 8; j++) P[k][j] = DAMP ? X[j] * cc[j] : (X[j] * cc[j]) * s;
        }
    }
    for (int cc2 = 0; cc2 < A.r; cc2++) {
        float pv[8], wv[8];
#pragma unroll
        for (int k = 0; k < 8; k++) pv[k] = A.comp_k[(h * A.r + cc2) * G::DK + row_of<G>(c, k)];
        load_f32x8(A.comp_v + (h * A.r + cc2) * G::DV + c.cb * 8, wv);
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) P[k][j] = fmaf(pv[k], wv[j], P[k][j]);
    }
#pragma unroll
    for (int k = 0; k < 8; k++) store_f32x8(A.S_out + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
}

hipError_t launch_quantize(const gdnq_desc &d, const float *S, const gdnq_state &s, hipStream_t st)
{
    QuantArgs A{S, s.codes, s.row_scale, s.col_scale, s.comp_k, s.comp_v, s.g_cur, s.hp_rows, s.hp_idx,
                (d.flags & GDNQ_DEBUG_PREQUANT) ? s.prequant_out : nullptr, nullptr,
                d.r, d.n_hp, d.power_iters, d.decay == GDNQ_DECAY_CHANNEL};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.layout == GDNQ_LAYOUT_DAMP, [&](auto damp) {
            return with_bits(d.bits, [&](auto bits) {
                constexpr bool DAMP = decltype(damp)::value;
                constexpr int BITS = decltype(bits)::value;
                if constexpr (DAMP && BITS != 8) {
                    return hipErrorInvalidValue;
                } else {
                    if (!DAMP && (d.flags & GDNQ_STATIC_SCALES))
                        hipLaunchKernelGGL((quantize_static_kernel<G, BITS>), dim3(nh), dim3(G::NT), 0, st, A,
                                           (size_t)nh);
                    else
                        hipLaunchKernelGGL((quantize_kernel<G, DAMP, BITS>), dim3(nh), dim3(G::NT), 0, st, A);
                    return hipGetLastError();
                }
            });
        });
    });
}

hipError_t launch_dequantize(const gdnq_desc &d, const gdnq_state &s, float *S_out, hipStream_t st)
{
    QuantArgs A{nullptr, s.codes, s.row_scale, s.col_scale, s.comp_k, s.comp_v, nullptr, s.hp_rows, s.hp_idx,
                nullptr, S_out, d.r, d.n_hp, d.power_iters, d.decay == GDNQ_DECAY_CHANNEL};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.layout == GDNQ_LAYOUT_DAMP, [&](auto damp) {
            return with_bits(d.bits, [&](auto bits) {
                constexpr bool DAMP = decltype(damp)::value;
                constexpr int BITS = decltype(bits)::value;
                if constexpr (DAMP && BITS != 8) {
                    return hipErrorInvalidValue;
                } else {
                    hipLaunchKernelGGL((dequantize_kernel<G, DAMP, BITS>), dim3(nh), dim3(G::NT), 0, st, A);
                    return hipGetLastError();
                }
            });
        });
    });
}

}  // namespace gdnq
