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

}  // namespace gdnq
