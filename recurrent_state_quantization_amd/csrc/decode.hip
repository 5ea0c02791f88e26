// decode.hip -- per-step decode kernels: the fused INT8 step (dequantize,
// gated delta update, output, requantize, store) and the fp32-state
// baseline step.  One workgroup per (batch, head) state.
//
// Recurrence: LinQuant (Functional Invariances for Low-Precision Linear
// Recurrences), appendix Table 3, Gated DeltaNet / KDA rows, transposed to
// S in R^{dk x dv}:  S' = diag(a) S;  u = b (v - S'^T k);  S_t = S' + k u^T;
// o = S_t^T q  (scalar gate: a_i = a for every row).
// Per-token load / update / write-back of the state: LeapQuant project
// page, opening paragraphs.
//
// With X_ij = s_i c_j Q_ij (dequantized state) the two mat-vecs are read
// straight off the codes:
//   (S'^T k)_j = c_j sum_i (a_i s_i k_i) Q_ij
//   o_j        = c_j sum_i (a_i s_i q_i) Q_ij + u_j (k . q)
// which is S_t^T q of the updated fp32 state before requantization (fp32
// FMAs over the thread's rows, then DPP / permlane reductions across the
// lanes and LDS across the waves).  The codec then runs on
// P_ij = fma(k_i, u_j, (Q_ij c_j)(a_i s_i)).
//
// The codes are read and written with non-temporal hints (each head's
// codes are streamed once per call); measured on MI355X this is worth ~5%
// for the INT8 kernel only when both directions carry the hint.  The
// fp32-state kernel keeps ordinary accesses: the hint slows it by ~30%.
#include "codec.hpp"
#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {

struct StepArgs {
    const void *q, *k, *v;
    const float *a, *b;
    void *o;
    int8_t *codes;
    float *row_scale, *col_scale;
    float *prequant;  // nullable
    float *S;         // fp32 state (baseline kernel)
    HeadMap map;
    size_t plane_r, plane_c;  // static scales: offsets of the rho and iota planes
};

// Column sums of R (retrieval) and O (output) partials, reduced to LDS, and
// k.q as one partial per wave of its last DK threads; the column threads
// then hold full sums.
//
// Work done once per row or column is spread so that the waves sharing a
// SIMD across resident workgroups carry about the same number of
// instructions: the first DK threads form the per-row factors and the first
// DV threads the column scales (codec), while the last DK threads reduce
// k.q and the last DV threads finish u and o.
template <class G>
struct StepLds {
    alignas(16) float rv[4][G::DK];  // per key row: a s, a s k, a s q, k (read as float4)
    float red[G::NW][2][G::DV];
    float red_kq[G::DK / 64];
    float u[G::DV];
};

template <class G>
constexpr int kq_first_thread() { return G::NT - G::DK; }
template <class G>
constexpr int col_first_thread() { return G::NT - G::DV; }

template <class G>
__device__ __forceinline__ void reduce_ro(const Lane &c, StepLds<G> &S, const float (&R)[8], const float (&O)[8])
{
    float x[16], z[4];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        x[j] = R[j];
        x[8 + j] = O[j];
    }
    col_reduce_scatter<G, OpSum, 16>(x, z);
#pragma unroll
    for (int p = 0; p < 4; p++) {
        const int idx = scatter_index(c, p);
        S.red[c.w][idx >> 3][c.cb * 8 + (idx & 7)] = z[p];
    }
}

// k.q over the key rows: thread kq_first_thread + i holds k_i q_i; each of
// those waves sums its 64 rows (DPP and permlane steps) into red_kq.
template <class G>
__device__ __forceinline__ void reduce_kq(const Lane &c, StepLds<G> &S, float ki, float qi)
{
    if (c.t >= kq_first_thread<G>()) {  // whole waves (NT - DK is a multiple of 64)
        const float kq = col_allreduce<G, OpSum>(row_sum<G>(ki * qi));
        if (c.lane == 0) S.red_kq[c.w - kq_first_thread<G>() / 64] = kq;
    }
}

template <class G>
__device__ __forceinline__ float sum_kq(const StepLds<G> &S)
{
    float kq = S.red_kq[0];
#pragma unroll
    for (int w = 1; w < G::DK / 64; w++) kq += S.red_kq[w];
    return kq;
}

template <class G, bool BF16, bool KDA, int BITS, bool STATIC>
__global__ __launch_bounds__(G::NT) void step_fused_kernel(StepArgs A)
{
    __shared__ CodecLds<G> L;
    __shared__ StepLds<G> SL;
    const Lane c = lane_coords<G>();
    constexpr size_t E = (size_t)G::DK * G::DV;
    constexpr int RB = code_row_bytes<G, BITS>();

    // The per-row factors are formed once per row (thread t < DK owns row
    // t; NT >= DK) and shared through LDS instead of by each of the row's
    // NCB lanes.  Their loads are issued first and unconditionally (rows
    // wrap for t >= DK) so that waiting for them does not wait for the
    // codes, which load meanwhile; the input-side ones go out even before
    // a pool call's slot is read.
    HeadIdx x;
    map_inputs(A.map, x);
    const size_t hi = x.in, hk = x.key;
    const int tr = c.t % G::DK;
    const int tc = c.t % G::DV;   // for t >= NT - DV: t - (NT - DV) (NT is a multiple of DV)
    const float ki = load1<BF16>(A.k, hk * G::DK + tr);
    const float qi = load1<BF16>(A.q, hk * G::DK + tr);
    const float ai = KDA ? A.a[hi * G::DK + tr] : A.a[hi];
    const float vj = load1<BF16>(A.v, hi * G::DV + tc);
    if (!map_state(A.map, 0, 0, 0, x)) return;  // uniform per workgroup, before any barrier
    const size_t h = x.state;
    int8_t *codes = A.codes + h * (size_t)G::DK * RB;
    float *rs = A.row_scale + h * G::DK;
    float *cs = A.col_scale + h * G::DV;
    const float si = rs[tr];
    const float cj = cs[tc];   // v_j and c_j serve the column threads (t >= NT - DV; columns wrap)
    float rho_t = 0.0f, io_t = 0.0f;  // static scales: one reciprocal per row / column, via LDS
    if constexpr (STATIC) {
        rho_t = A.row_scale[A.plane_r + h * G::DK + tr];
        io_t = A.col_scale[A.plane_c + h * G::DV + tc];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the codes'

    const int row0 = row0_of<G>(c);
    const int8_t *rbase = codes + (size_t)row0 * RB;
    CodeWord qraw[8];
#pragma unroll
    for (int k = 0; k < 8; k++) qraw[k] = load_code8<G, BITS, true>(rbase + koff<G>(k) * RB, c.cb);
    float cc[8];
    load_f32x8(cs + c.cb * 8, cc);
    const float bh = A.b[hi];
    if (c.t < G::DK) {
        const float asi = ai * si;
        SL.rv[0][c.t] = asi;
        SL.rv[1][c.t] = asi * ki;
        SL.rv[2][c.t] = asi * qi;
        SL.rv[3][c.t] = ki;
    }
    if constexpr (STATIC) {
        if (c.t < G::DK) L.rho[c.t] = rho_t;
        if (c.t < G::DV) L.iota[c.t] = io_t;
    }
    reduce_kq<G>(c, SL, ki, qi);  // row t % DK in thread t: the last DK threads hold every row once
    __syncthreads();
    float X[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) unpack_code8<BITS>(qraw[k], X[k]);
    {
        float ask[8], asq[8], R[8], O[8];
        load_rows_f32<G>(&SL.rv[1][row0], ask);
        load_rows_f32<G>(&SL.rv[2][row0], asq);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            R[j] = X[0][j] * ask[0];
            O[j] = X[0][j] * asq[0];
        }
#pragma unroll
        for (int k = 1; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) {
                R[j] = fmaf(X[k][j], ask[k], R[j]);
                O[j] = fmaf(X[k][j], asq[k], O[j]);
            }
        reduce_ro<G>(c, SL, R, O);
    }
    // The decayed, dequantized state (Q_ij c_j)(a_i s_i), formed while the
    // other waves finish their sums; only k and u remain for the update.
    float kk[8];
    {
        float as[8];
        load_rows_f32<G>(&SL.rv[0][row0], as);
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) X[k][j] = (X[k][j] * cc[j]) * as[k];
    }
    load_rows_f32<G>(&SL.rv[3][row0], kk);
    __syncthreads();
    if (c.t >= col_first_thread<G>()) {  // column tc = t - (NT - DV)
        float Rj = SL.red[0][0][tc], Oj = SL.red[0][1][tc];
#pragma unroll
        for (int w = 1; w < G::NW; w++) {
            Rj += SL.red[w][0][tc];
            Oj += SL.red[w][1][tc];
        }
        const float u = bh * (vj - cj * Rj);
        store1<BF16>(A.o, hi * G::DV + tc, fmaf(u, sum_kq<G>(SL), cj * Oj));
        SL.u[tc] = u;
    }
    __syncthreads();
    float u8[8];
#pragma unroll
    for (int j = 0; j < 8; j++) u8[j] = SL.u[c.cb * 8 + j];
#pragma unroll
    for (int k = 0; k < 8; k++)
#pragma unroll
        for (int j = 0; j < 8; j++) X[k][j] = fmaf(kk[k], u8[j], X[k][j]);
    if (A.prequant) {
        float *pq = A.prequant + h * E + (size_t)row0 * G::DV + c.cb * 8;
#pragma unroll
        for (int k = 0; k < 8; k++) store_f32x8(pq + koff<G>(k) * G::DV, X[k]);
    }
    if constexpr (STATIC) {
        float srho[8], sio[8];  // the reciprocals of the lane's rows and columns
        load_rows_f32<G>(&L.rho[row0], srho);
        load_f32x8(&L.iota[c.cb * 8], sio);
        codec_static<G, true, BITS>(X, c, srho, sio, codes);
    } else
        codec_rowcol<G, true, BITS>(X, c, L, codes, rs, cs);
}

template <class G, bool BF16, bool KDA>
__global__ __launch_bounds__(G::NT) void step_fp32_kernel(StepArgs A)
{
    __shared__ StepLds<G> SL;
    const Lane c = lane_coords<G>();
    HeadIdx x;
    map_head(A.map, 0, 0, 0, x);  // no pool form: every entry maps
    const size_t h = x.in, hk = x.key;
    constexpr size_t E = (size_t)G::DK * G::DV;
    float *S = A.S + h * E;

    const int row0 = row0_of<G>(c);
    float *Sb = S + (size_t)row0 * G::DV + c.cb * 8;
    float X[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) load_f32x8(Sb + koff<G>(k) * G::DV, X[k]);
    float kk[8], qq[8], av[8];
    load_rows<G, BF16>(A.k, hk * G::DK, row0, kk);
    load_rows<G, BF16>(A.q, hk * G::DK, row0, qq);
    if constexpr (KDA) {
        load_rows_f32<G>(A.a + h * G::DK + row0, av);
    } else {
        const float ag = A.a[h];
#pragma unroll
        for (int k = 0; k < 8; k++) av[k] = ag;
    }
    const float bh = A.b[h];
    float vj = 0.0f;
    if (c.t < G::DV) vj = load1<BF16>(A.v, h * G::DV + c.t);

    float ak[8], aq[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        ak[k] = av[k] * kk[k];
        aq[k] = av[k] * qq[k];
    }
    {
        const int tr = c.t % G::DK;
        reduce_kq<G>(c, SL, load1<BF16>(A.k, hk * G::DK + tr), load1<BF16>(A.q, hk * G::DK + tr));
    }
    float R[8], O[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        R[j] = X[0][j] * ak[0];
        O[j] = X[0][j] * aq[0];
    }
#pragma unroll
    for (int k = 1; k < 8; k++)
#pragma unroll
        for (int j = 0; j < 8; j++) {
            R[j] = fmaf(X[k][j], ak[k], R[j]);
            O[j] = fmaf(X[k][j], aq[k], O[j]);
        }
    reduce_ro<G>(c, SL, R, O);
    __syncthreads();
    if (c.t < G::DV) {
        float Rj = SL.red[0][0][c.t], Oj = SL.red[0][1][c.t];
#pragma unroll
        for (int w = 1; w < G::NW; w++) {
            Rj += SL.red[w][0][c.t];
            Oj += SL.red[w][1][c.t];
        }
        const float u = bh * (vj - Rj);
        store1<BF16>(A.o, h * G::DV + c.t, fmaf(u, sum_kq<G>(SL), Oj));
        SL.u[c.t] = u;
    }
    __syncthreads();
    float u8[8];
#pragma unroll
    for (int j = 0; j < 8; j++) u8[j] = SL.u[c.cb * 8 + j];
#pragma unroll
    for (int k = 0; k < 8; k++) {
#pragma unroll
        for (int j = 0; j < 8; j++) X[k][j] = fmaf(kk[k], u8[j], X[k][j] * av[k]);
        store_f32x8(Sb + koff<G>(k) * G::DV, X[k]);
    }
}

hipError_t launch_step_fused(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, const void *q,
                             const void *k, const void *v, const float *a, const float *b, void *o,
                             hipStream_t st)
{
    // state heads: n_slots * H (n_slots = B for the plain call)
    const size_t sh = (size_t)m.n_slots * (size_t)d.H;
    StepArgs A{q, k, v, a, b, o, s.codes, s.row_scale, s.col_scale,
               (d.flags & GDNQ_DEBUG_PREQUANT) ? s.prequant_out : nullptr, nullptr, m,
               sh * (size_t)d.dk, sh * (size_t)d.dv};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.io_dtype == GDNQ_IO_BF16, [&](auto bf) {
            return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
                return with_bits(d.bits, [&](auto bits) {
                    return with_bool((d.flags & GDNQ_STATIC_SCALES) != 0, [&](auto stat) {
                        hipLaunchKernelGGL((step_fused_kernel<G, decltype(bf)::value, decltype(kda)::value,
                                                              decltype(bits)::value, decltype(stat)::value>),
                                           dim3(nh), dim3(G::NT), 0, st, A);
                        return hipGetLastError();
                    });
                });
            });
        });
    });
}

hipError_t launch_step_fp32(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                            const float *a, const float *b, void *o, hipStream_t st)
{
    StepArgs A{q, k, v, a, b, o, nullptr, nullptr, nullptr, nullptr, S, plain_map(d), 0, 0};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.io_dtype == GDNQ_IO_BF16, [&](auto bf) {
            return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
                hipLaunchKernelGGL((step_fp32_kernel<G, decltype(bf)::value, decltype(kda)::value>), dim3(nh),
                                   dim3(G::NT), 0, st, A);
                return hipGetLastError();
            });
        });
    });
}

}  // namespace gdnq
