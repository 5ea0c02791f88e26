// calibrate.hip -- offline choice of the DAMP fp16 key rows.
//
// DAMP abstract: most quantization-error energy sits in a few channels and
// a channel's decay strength is stable, so high-risk channels are picked
// offline from error energy and decay-based persistence.  Reading taken:
// run n_steps of the fp32 recurrence from S0 (LinQuant Table 3 update,
// transposed); after each step quantize the state with value-column INT8
// scales over all rows and no smoothing; E_i += sum_j (S_ij - D_ij)^2;
// abar_i = mean gate of key channel i; score_i = E_i / max(1 - abar_i, 1e-6);
// keep the n_hp highest scores (lower index first on ties), ascending.
#include "codec.hpp"
#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {

struct CalArgs {
    const float *S0;
    const void *k, *v;
    const float *a, *b;
    int32_t *hp_idx;
    float *score;
    int n_steps, n_hp;
    size_t nh;
    HeadMap map;   // key heads of k (no pool form)
};

template <class G>
struct CalLds {
    float red[G::NW][G::DV];
    float u[G::DV];
    float iota[G::DV], cs[G::DV];
    float sc[G::DK];
};

template <class G, bool BF16, bool KDA>
__global__ __launch_bounds__(G::NT) void calibrate_kernel(CalArgs A)
{
    __shared__ CalLds<G> L;
    const Lane c = lane_coords<G>();
    HeadIdx x;
    map_head(A.map, 0, 0, 0, x);
    const size_t h = x.in;
    const size_t nk = A.nh / A.map.H * A.map.HK;   // key heads per step
    constexpr size_t E = (size_t)G::DK * G::DV;
    float P[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) load_f32x8(A.S0 + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
    float En[8], asum[8];
#pragma unroll
    for (int k = 0; k < 8; k++) { En[k] = 0.0f; asum[k] = 0.0f; }

    for (int t = 0; t < A.n_steps; t++) {
        const size_t hs = (size_t)t * A.nh + h;
        float kk[8], av[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const int i = row_of<G>(c, k);
            kk[k] = load1<BF16>(A.k, ((size_t)t * nk + x.key) * G::DK + i);
            av[k] = KDA ? A.a[hs * G::DK + i] : A.a[hs];
        }
        float R[8];
#pragma unroll
        for (int j = 0; j < 8; j++) R[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float ak = av[k] * kk[k];
#pragma unroll
            for (int j = 0; j < 8; j++) R[j] = fmaf(P[k][j], ak, R[j]);
        }
        float z[2];
        col_reduce_scatter<G, OpSum, 8>(R, z);
#pragma unroll
        for (int p = 0; p < 2; p++) L.red[c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
        __syncthreads();
        if (c.t < G::DV) {
            float ret = L.red[0][c.t];
#pragma unroll
            for (int w = 1; w < G::NW; w++) ret += L.red[w][c.t];
            L.u[c.t] = A.b[hs] * (load1<BF16>(A.v, hs * G::DV + c.t) - ret);
        }
        __syncthreads();
        float u8[8], m[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            u8[j] = L.u[c.cb * 8 + j];
            m[j] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                P[k][j] = fmaf(kk[k], u8[j], P[k][j] * av[k]);
                m[j] = fmaxf(m[j], fabsf(P[k][j]));
            }
            asum[k] += av[k];
        }
        col_reduce_scatter<G, OpMax, 8>(m, z);
#pragma unroll
        for (int p = 0; p < 2; p++) L.red[c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
        __syncthreads();
        if (c.t < G::DV) {
            float mm = L.red[0][c.t];
#pragma unroll
            for (int w = 1; w < G::NW; w++) mm = fmaxf(mm, L.red[w][c.t]);
            float cj = 0.0f, io = 0.0f;
            if (mm > 0.0f) {
                io = 127.0f / mm;
                if (__builtin_isinf(io)) io = 0.0f;
                else cj = mm / 127.0f;
            }
            L.cs[c.t] = cj;
            L.iota[c.t] = io;
        }
        __syncthreads();
        float io[8], cj[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            io[j] = L.iota[c.cb * 8 + j];
            cj[j] = L.cs[c.cb * 8 + j];
        }
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float q = fmaf(P[k][j], io[j], RINT_MAGIC) - RINT_MAGIC;  // rint of the exact product
                const float d = P[k][j] - q * cj[j];
                En[k] = fmaf(d, d, En[k]);
            }
        // the next step's first barrier orders these LDS reads before the
        // next writes of L.red / L.u / L.iota
    }
    {
        const float e = row_reduce_scatter<G, OpSum>(En, c.cb);
        const int k = row_scatter_k<G>(c.cb);
        // every lane of the row group holds the same gate sums, so their
        // reduce-scatter is exactly NCB times row k's sum (pairwise sums of
        // equal values are exact)
        const float as = row_reduce_scatter<G, OpSum>(asum, c.cb) * (1.0f / G::NCB);
        if (G::NCB == 8 || (c.cb & 1) == 0) {
        const int i = row0_of<G>(c) + (k >> 2) * (G::RGW * 4) + (k & 3);
        const float abar = as / (float)A.n_steps;
        const float den = fmaxf(1.0f - abar, 1e-6f);
        const float s = e / den;
        L.sc[i] = s;
        if (A.score) A.score[h * G::DK + i] = s;
        }
    }
    __syncthreads();
    if (c.t == 0) {
        // repeated arg-max with lowest index on ties; mark chosen rows
        for (int n = 0; n < A.n_hp; n++) {
            int best = -1;
            float bv = 0.0f;
            for (int i = 0; i < G::DK; i++) {
                const float v = L.sc[i];
                if (v < 0.0f) continue;  // taken
                if (best < 0 || v > bv) { best = i; bv = v; }
            }
            L.sc[best] = -1.0f;
        }
        int n = 0;
        for (int i = 0; i < G::DK; i++)
            if (L.sc[i] < 0.0f) A.hp_idx[h * A.n_hp + n++] = i;
    }
}

hipError_t launch_calibrate(const gdnq_desc &d, const float *S0, const void *k, const void *v,
                            const float *a, const float *b, int n_steps, int32_t *hp_idx,
                            float *score, hipStream_t st)
{
    const size_t nh = (size_t)d.B * (size_t)d.H;
    CalArgs A{S0, k, v, a, b, hp_idx, score, n_steps, d.n_hp, nh, plain_map(d)};
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.io_dtype == GDNQ_IO_BF16, [&](auto bf) {
            return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
                hipLaunchKernelGGL((calibrate_kernel<G, decltype(bf)::value, decltype(kda)::value>),
                                   dim3((unsigned)nh), dim3(G::NT), 0, st, A);
                return hipGetLastError();
            });
        });
    });
}

// ---------------------------------------------------------------------------
// Static scales (STEPQuant page: key-row and value-column scales fitted
// jointly and offline from the state distribution and each key row's impact
// on the output error; the page gives no formula).  Reading taken, three
// passes of n_steps of the fp32 recurrence from S0 over calibration inputs:
//   1. s_i = sqrt(max_t max_j |S_t,ij|), rho_i = 1/s_i; omega_i =
//      (mean_t q_t,i^2) / max(1 - abar_i, 1e-6) (the row's weight in
//      o = S^T q times the lifetime of an error in it under its gate);
//   2. m_j = max_t max_i |S_t,ij rho_i|; candidate ranges m_j (16-k)/16,
//      k = 0..8, with c = range/Qb and iota = Qb/range;
//   3. E_j(k) = sum_t sum_i omega_i (S_t,ij - D_t,ij(k))^2 under the static
//      codec; keep the least (smallest k on ties).
// Written to the two planes of row_scale (s, rho) and col_scale (c, iota).
// ---------------------------------------------------------------------------
struct FitArgs {
    const float *S0;
    const void *q, *k, *v;
    const float *a, *b;
    float *row_scale, *col_scale;
    int n_steps;
    size_t nh;
    HeadMap map;  // key heads of q, k (no pool form)
};

template <class G>
struct FitLds {
    float red[G::NW][G::DV];
    float u[G::DV];
    float s[G::DK], rho[G::DK], om[G::DK];
    float cc[9][G::DV], ci[9][G::DV];
    float err[9][G::NW][G::DV];
};

// One step of the fp32 recurrence on the thread's 8x8 block (as in the
// DAMP calibration): R = (a S)^T k, u = b (v - R), S <- a S + k u^T.  The
// lane's key and gate values of its rows are returned in kk, av.
template <class G, bool BF16, bool KDA>
__device__ __forceinline__ void fit_recur_step(const FitArgs &A, const Lane &c, FitLds<G> &L, size_t h,
                                               size_t key, size_t nk, int t, float (&P)[8][8], float (&av)[8])
{
    const size_t hs = (size_t)t * A.nh + h;
    float kk[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int i = row_of<G>(c, k);
        kk[k] = load1<BF16>(A.k, ((size_t)t * nk + key) * G::DK + i);
        av[k] = KDA ? A.a[hs * G::DK + i] : A.a[hs];
    }
    float R[8];
#pragma unroll
    for (int j = 0; j < 8; j++) R[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const float ak = av[k] * kk[k];
#pragma unroll
        for (int j = 0; j < 8; j++) R[j] = fmaf(P[k][j], ak, R[j]);
    }
    float z[2];
    col_reduce_scatter<G, OpSum, 8>(R, z);
#pragma unroll
    for (int p = 0; p < 2; p++) L.red[c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
    __syncthreads();
    if (c.t < G::DV) {
        float ret = L.red[0][c.t];
#pragma unroll
        for (int w = 1; w < G::NW; w++) ret += L.red[w][c.t];
        L.u[c.t] = A.b[hs] * (load1<BF16>(A.v, hs * G::DV + c.t) - ret);
    }
    __syncthreads();
    float u8[8];
#pragma unroll
    for (int j = 0; j < 8; j++) u8[j] = L.u[c.cb * 8 + j];
#pragma unroll
    for (int k = 0; k < 8; k++)
#pragma unroll
        for (int j = 0; j < 8; j++) P[k][j] = fmaf(kk[k], u8[j], P[k][j] * av[k]);
}

template <class G, bool BF16, bool KDA, int BITS>
__global__ __launch_bounds__(G::NT) void fit_static_kernel(FitArgs A)
{
    __shared__ FitLds<G> L;
    constexpr float QB = (float)code_qmax<BITS>();
    const Lane c = lane_coords<G>();
    HeadIdx x;
    map_head(A.map, 0, 0, 0, x);
    const size_t h = x.in;
    const size_t nk = A.nh / A.map.H * A.map.HK;  // key heads per step
    constexpr size_t E = (size_t)G::DK * G::DV;
    const int row0 = row0_of<G>(c);
    float P[8][8], av[8];
#define GDNQ_FIT_RESET()                                                                                    \
    _Pragma("unroll") for (int k = 0; k < 8; k++)                                                        \
        load_f32x8(A.S0 + h * E + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k])

    // pass 1: row maxima, output weights, gate means
    float rmax[8], qsum[8], asum[8];
#pragma unroll
    for (int k = 0; k < 8; k++) rmax[k] = qsum[k] = asum[k] = 0.0f;
    GDNQ_FIT_RESET();
    for (int t = 0; t < A.n_steps; t++) {
        fit_recur_step<G, BF16, KDA>(A, c, L, h, x.key, nk, t, P, av);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const float qi = load1<BF16>(A.q, ((size_t)t * nk + x.key) * G::DK + row_of<G>(c, k));
            qsum[k] = fmaf(qi, qi, qsum[k]);
            asum[k] += av[k];
#pragma unroll
            for (int j = 0; j < 8; j++) rmax[k] = fmaxf(rmax[k], fabsf(P[k][j]));
        }
    }
    {
        const float r = row_reduce_scatter<G, OpMax>(rmax, c.cb);
        // every lane of the row holds the same q and gate sums: the
        // reduce-scatter of equal values is exactly NCB times one of them
        const float qs = row_reduce_scatter<G, OpSum>(qsum, c.cb) * (1.0f / G::NCB);
        const float as = row_reduce_scatter<G, OpSum>(asum, c.cb) * (1.0f / G::NCB);
        const int k = row_scatter_k<G>(c.cb);
        if (G::NCB == 8 || (c.cb & 1) == 0) {
            const int i = row0 + (k >> 2) * (G::RGW * 4) + (k & 3);
            const float s = r > 0.0f ? sqrtf(r) : 0.0f;
            const float rho = s > 0.0f ? 1.0f / s : 0.0f;
            L.s[i] = s;
            L.rho[i] = rho;
            L.om[i] = (qs / (float)A.n_steps) / fmaxf(1.0f - as / (float)A.n_steps, 1e-6f);
            A.row_scale[h * G::DK + i] = s;
            A.row_scale[A.nh * G::DK + h * G::DK + i] = rho;
        }
    }
    __syncthreads();
    float rho8[8], s8[8], om8[8];
    load_rows_f32<G>(&L.rho[row0], rho8);
    load_rows_f32<G>(&L.s[row0], s8);
    load_rows_f32<G>(&L.om[row0], om8);

    // pass 2: column maxima of the smoothed states
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; j++) m[j] = 0.0f;
    GDNQ_FIT_RESET();
    for (int t = 0; t < A.n_steps; t++) {
        fit_recur_step<G, BF16, KDA>(A, c, L, h, x.key, nk, t, P, av);
#pragma unroll
        for (int k = 0; k < 8; k++)
#pragma unroll
            for (int j = 0; j < 8; j++) m[j] = fmaxf(m[j], fabsf(P[k][j] * rho8[k]));
    }
    {
        float z[2];
        col_reduce_scatter<G, OpMax, 8>(m, z);
#pragma unroll
        for (int p = 0; p < 2; p++) L.red[c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
    }
    __syncthreads();
    if (c.t < G::DV) {
        float mm = L.red[0][c.t];
#pragma unroll
        for (int w = 1; w < G::NW; w++) mm = fmaxf(mm, L.red[w][c.t]);
#pragma unroll
        for (int kc = 0; kc < 9; kc++) {
            const float mc = mm * ((float)(16 - kc) / 16.0f);
            float cj = 0.0f, io = 0.0f;
            if (mc > 0.0f) {
                io = QB / mc;
                if (__builtin_isinf(io)) io = 0.0f;
                else cj = mc / QB;
            }
            L.cc[kc][c.t] = cj;
            L.ci[kc][c.t] = io;
        }
    }
    __syncthreads();

    // pass 3: weighted error of every candidate
    float err[9][8];
#pragma unroll
    for (int kc = 0; kc < 9; kc++)
#pragma unroll
        for (int j = 0; j < 8; j++) err[kc][j] = 0.0f;
    GDNQ_FIT_RESET();
    for (int t = 0; t < A.n_steps; t++) {
        fit_recur_step<G, BF16, KDA>(A, c, L, h, x.key, nk, t, P, av);
#pragma unroll
        for (int kc = 0; kc < 9; kc++) {
            float cc8[8], ci8[8];
            load_f32x8(&L.cc[kc][c.cb * 8], cc8);
            load_f32x8(&L.ci[kc][c.cb * 8], ci8);
#pragma unroll
            for (int k = 0; k < 8; k++)
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const float y = __builtin_amdgcn_fmed3f(fmaf(P[k][j] * rho8[k], ci8[j], RINT_MAGIC),
                                                            RINT_MAGIC - QB, RINT_MAGIC + QB);
                    const float d = P[k][j] - ((y - RINT_MAGIC) * cc8[j]) * s8[k];
                    err[kc][j] = fmaf(om8[k] * d, d, err[kc][j]);
                }
        }
    }
#pragma unroll
    for (int kc = 0; kc < 9; kc++) {
        float z[2];
        col_reduce_scatter<G, OpSum, 8>(err[kc], z);
#pragma unroll
        for (int p = 0; p < 2; p++) L.err[kc][c.w][c.cb * 8 + scatter_index(c, p)] = z[p];
    }
    __syncthreads();
    if (c.t < G::DV) {
        int best = 0;
        float be = 0.0f;
#pragma unroll
        for (int kc = 0; kc < 9; kc++) {
            float e = L.err[kc][0][c.t];
#pragma unroll
            for (int w = 1; w < G::NW; w++) e += L.err[kc][w][c.t];
            if (kc == 0 || e < be) { best = kc; be = e; }
        }
        A.col_scale[h * G::DV + c.t] = L.cc[best][c.t];
        A.col_scale[A.nh * G::DV + h * G::DV + c.t] = L.ci[best][c.t];
    }
#undef GDNQ_FIT_RESET
}

hipError_t launch_fit_static(const gdnq_desc &d, const float *S0, const void *q, const void *k, const void *v,
                             const float *a, const float *b, int n_steps, float *row_scale, float *col_scale,
                             hipStream_t st)
{
    const size_t nh = (size_t)d.B * (size_t)d.H;
    FitArgs A{S0, q, k, v, a, b, row_scale, col_scale, n_steps, nh, plain_map(d)};
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.io_dtype == GDNQ_IO_BF16, [&](auto bf) {
            return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
                return with_bits(d.bits, [&](auto bits) {
                    hipLaunchKernelGGL((fit_static_kernel<G, decltype(bf)::value, decltype(kda)::value,
                                                          decltype(bits)::value>),
                                       dim3((unsigned)nh), dim3(G::NT), 0, st, A);
                    return hipGetLastError();
                });
            });
        });
    });
}

}  // namespace gdnq
