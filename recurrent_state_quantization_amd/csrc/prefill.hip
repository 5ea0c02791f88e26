// prefill.hip -- chunkwise-parallel prefill of the gated delta rule on the
// matrix cores (gdn_prefill).
//
// The recurrence is the Gated DeltaNet row of Table 3 in "LinQuant:
// Functional Invariances for Low-Precision Linear Recurrences" (appendix),
// in the dk x dv orientation: S_t = a_t S_{t-1} + k_t u_t^T with
// u_t = b_t (v_t - a_t S_{t-1}^T k_t), o_t = S_t^T q_t.  That page's
// abstract notes that chunkwise-parallel prefill turns most of it into
// dense matrix products; the chunk form used here is the published
// WY/UT-transform form of the delta rule (Yang et al., "Parallelizing
// Linear Transformers with the Delta Rule over Sequence Length", 2024, and
// its gated variant, Yang, Kautz and Hatamizadeh, "Gated Delta Networks",
// 2024), restated for this state orientation.  For a chunk of C tokens with
// g_i = sum_{t<=i} log a_t counted from the chunk start, Gam_ij = e^{g_i-g_j}
// (i >= j), beta = b and S the state at the chunk start:
//     A  = strictly lower part of diag(beta) (K K^T . Gam)
//     T  = (I + A)^{-1}
//     W  = T diag(beta e^g) K,        U = T diag(beta) V
//     U' = U - W S                    (row i is the update u_i)
//     O  = diag(e^g) Q S + (Q K^T . Gam . [i >= j]) U'
//     S <- e^{g_C} S + K^T diag(e^{g_C - g}) U'
// which is the token recurrence unrolled over the chunk (the substitution
// a_t S_{t-1} = e^{g_t} S + sum_{j<t} e^{g_t-g_j} k_j u_j^T gives the
// triangular system (I + A) U' = diag(beta) V - diag(beta e^g) K S).
//
// Precision: every product runs on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  q, k, v are bf16, so their products are exact; every fp32
// operand x (T, W, S, U', P) is split x = hi + lo, hi = bf16(x),
// lo = bf16(x - hi) (x - hi is exact in fp32), and a product takes hi*y +
// lo*y, or hi*hi' + hi*lo' + lo*hi' when both operands are split, leaving
// a relative operand error near 2^-17.  The unit lower-triangular inverse
// runs in fp32: forward substitution on the 16x16 diagonal blocks, then two
// block-merge levels on v_mfma_f32_16x16x4f32.
//
// Mapping: one workgroup per (batch, head) walks the chunks in order.  Wave
// w owns value columns 16w..16w+15 of the state, which stays in fp32 MFMA
// accumulators for the whole sequence: every state-dependent product
// (U' = U - W S, Q S, the state update) needs only the wave's own columns,
// and the accumulators feed the next product's operand directly by
// permuting the contraction index (slots 0..3 of lane group g take
// k = 4g..4g+3 of one 16-row tile, slots 4..7 those of the next tile; the
// LDS operand on the other side is read in the same order).  The chunk-local
// part (K K^T, Q K^T, the inverse, W) is shared through LDS.
#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace gdnq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // tokens per chunk

template <int D>
struct PrefillLds {
    static constexpr int SD = D + 8;   // row stride (bf16) of [CH][D] tiles (16-byte pad)
    static constexpr int SC = CH + 8;  // row stride (bf16) of [.][CH] tiles (16-byte pad)
    static constexpr int SF = CH + 4;  // row stride (fp32) of [CH][CH] fp32 tiles
    __bf16 kr[CH * SD];  // K, token-major
    __bf16 qr[CH * SD];  // Q, token-major
    __bf16 kt[D * SC];   // K^T, key-channel-major
    __bf16 vt[D * SC];   // V^T, value-channel-major
    union {
        struct {
            float a[CH * SF];  // A (strictly lower)
            float t[CH * SF];  // T = (I + A)^{-1} (lower)
        } inv;
        struct {
            __bf16 h[CH * SD];  // -W, hi part, token-major
            __bf16 l[CH * SD];  // -W, lo part
        } w;
    } u;
    __bf16 t1h[CH * SC], t1l[CH * SC];  // T diag(beta e^g), split
    __bf16 t2h[CH * SC], t2l[CH * SC];  // T diag(beta), split
    __bf16 ph[CH * SC], pl[CH * SC];    // (Q K^T . Gam . [i >= j]), split
    float g[CH], eg[CH], gam[CH], beta[CH];
};

struct PrefillArgs {
    float *S;
    const __bf16 *q, *k, *v;
    const float *a, *b;
    __bf16 *o;
    int T, H, HK;
    Divisor byH, byG;
};

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// element e of h and l <- the two bf16 parts of x
template <class V>
__device__ __forceinline__ void split(float x, V &h, V &l, int e)
{
    const __bf16 hi = (__bf16)x;
    h[e] = hi;
    l[e] = (__bf16)(x - (float)hi);
}

// Operand in the permuted slot order: 4 values at p, then 4 at p + 16.
__device__ __forceinline__ bf16x8 ld_pair(const __bf16 *p)
{
    const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 y = *reinterpret_cast<const bf16x4 *>(p + 16);
    return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Lower 16x16 tiles (I >= J) of a 64x64 chunk matrix.
__constant__ unsigned char kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ unsigned char kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int D>
__global__ __launch_bounds__(D * 4, 1) void prefill_kernel(PrefillArgs A)
{
    using Lds = PrefillLds<D>;
    constexpr int SD = Lds::SD, SC = Lds::SC, SF = Lds::SF;
    constexpr int NW = D / 16, NT = NW * 64;
    constexpr int KB = D / 32;  // 32-wide blocks along a head dim
    constexpr int DT = D / 16;  // 16-row tiles along a head dim
    static_assert(NT == CH * D / 16, "one 16-byte piece per thread per token pair");
    __shared__ Lds L;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lg = lane >> 4, ln = lane & 15;
    const unsigned bh = blockIdx.x;
    const unsigned bb = div_by(bh, A.byH), hh = bh - bb * (unsigned)A.H;
    const unsigned kh = div_by(hh, A.byG);  // key head within the batch entry
    const int T = A.T;
    const size_t tk = (size_t)A.HK * D, tv = (size_t)A.H * D;  // token strides (elements)
    const __bf16 *qg = A.q + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *kg = A.k + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *vg = A.v + (size_t)bb * T * tv + (size_t)hh * D;
    __bf16 *og = A.o + (size_t)bb * T * tv + (size_t)hh * D;
    const float *ag = A.a + (size_t)bb * T * A.H + hh;
    const float *bg = A.b + (size_t)bb * T * A.H + hh;
    float *Sg = A.S + (size_t)bh * D * D;
    const int e0 = 16 * wave;  // this wave's value columns

    // P's upper tiles are never written: clear them once.
    for (int x = tid; x < CH * SC; x += NT) {
        L.ph[x] = (__bf16)0.0f;
        L.pl[x] = (__bf16)0.0f;
    }

    // state columns e0..e0+15: S[dt][r] = S[16dt + 4lg + r][e0 + ln]
    floatx4 S[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 4; r++) S[dt][r] = Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + ln];

    // chunk loads: thread -> tokens 2p, 2p+1 (p = tid % 32), columns 8c..8c+7 (c = tid / 32)
    const int jp = 2 * (tid & 31), cp = 8 * (tid >> 5);
    u32x4 rk[2], rq[2], rv[2];
    float ra = 1.0f, rb = 0.0f;
    auto load = [&](int c0) {
#pragma unroll
        for (int s = 0; s < 2; s++) {
            const int t = c0 + jp + s;
            if (t < T) {
                rk[s] = *reinterpret_cast<const u32x4 *>(kg + (size_t)t * tk + cp);
                rq[s] = *reinterpret_cast<const u32x4 *>(qg + (size_t)t * tk + cp);
                rv[s] = *reinterpret_cast<const u32x4 *>(vg + (size_t)t * tv + cp);
            } else {
                rk[s] = rq[s] = rv[s] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (tid < CH) {
            const int t = c0 + tid;
            ra = t < T ? ag[(size_t)t * A.H] : 1.0f;  // padding: gate 1, beta 0
            rb = t < T ? bg[(size_t)t * A.H] : 0.0f;
        }
    };

    load(0);
    for (int c0 = 0; c0 < T; c0 += CH) {
        __syncthreads();  // the previous chunk is done with every LDS tile
        // ---- stage the chunk: K, Q token-major; K, V transposed (token pairs packed)
#pragma unroll
        for (int s = 0; s < 2; s++) {
            *reinterpret_cast<u32x4 *>(&L.kr[(jp + s) * SD + cp]) = rk[s];
            *reinterpret_cast<u32x4 *>(&L.qr[(jp + s) * SD + cp]) = rq[s];
        }
#pragma unroll
        for (int x = 0; x < 4; x++) {
            // dword x of a piece holds columns 2x, 2x+1; pack token pairs per column
            const unsigned k0 = rk[0][x], k1 = rk[1][x], v0 = rv[0][x], v1 = rv[1][x];
            *reinterpret_cast<unsigned *>(&L.kt[(cp + 2 * x) * SC + jp]) = (k0 & 0xffffu) | (k1 << 16);
            *reinterpret_cast<unsigned *>(&L.kt[(cp + 2 * x + 1) * SC + jp]) = (k0 >> 16) | (k1 & 0xffff0000u);
            *reinterpret_cast<unsigned *>(&L.vt[(cp + 2 * x) * SC + jp]) = (v0 & 0xffffu) | (v1 << 16);
            *reinterpret_cast<unsigned *>(&L.vt[(cp + 2 * x + 1) * SC + jp]) = (v0 >> 16) | (v1 & 0xffff0000u);
        }
        if (wave == 0) {  // cumulative log-gates over the chunk (inclusive scan)
            float x = logf(ra);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o, 64);
                if (lane >= o) x += y;
            }
            const float glast = __shfl(x, 63, 64);
            L.g[lane] = x;
            L.eg[lane] = expf(x);
            L.gam[lane] = expf(glast - x);
            L.beta[lane] = rb;
        }
        __syncthreads();
        if (c0 + CH < T) load(c0 + CH);  // next chunk in flight during this one

        // ---- A = strictly lower diag(beta)(K K^T . Gam) (fp32) and P (split);
        // tile (I, J) is computed transposed (rows j, columns i) so each lane
        // holds 4 consecutive j of one i
        for (int job = wave; job < 20; job += NW) {
            const bool isP = job >= 10;
            const int tix = isP ? job - 10 : job;
            const int I = kTileI[tix], J = kTileJ[tix];
            const __bf16 *src = isP ? L.qr : L.kr;
            floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
                acc = mma(ld8(&L.kr[(16 * J + ln) * SD + 32 * kb + 8 * lg]),
                          ld8(&src[(16 * I + ln) * SD + 32 * kb + 8 * lg]), acc);
            const int i = 16 * I + ln, j0 = 16 * J + 4 * lg;
            const float gi = L.g[i];
            if (!isP) {
                const float bi = L.beta[i];
                floatx4 out;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    out[r] = i > j0 + r ? (bi * acc[r]) * expf(gi - L.g[j0 + r]) : 0.0f;
                *reinterpret_cast<floatx4 *>(&L.u.inv.a[i * SF + j0]) = out;
            } else {
                bf16x4 h, l;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float p = i >= j0 + r ? acc[r] * expf(gi - L.g[j0 + r]) : 0.0f;
                    split(p, h, l, r);
                }
                *reinterpret_cast<bf16x4 *>(&L.ph[i * SC + j0]) = h;
                *reinterpret_cast<bf16x4 *>(&L.pl[i * SC + j0]) = l;
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1}.  Level 0: the four 16x16 diagonal blocks by
        // forward substitution, lane = (block lg, column ln)
        if (wave == 0) {
            const float *Ab = &L.u.inv.a[16 * lg * SF + 16 * lg];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float acc = r == ln ? 1.0f : 0.0f;
#pragma unroll
                for (int s = 0; s < r; s++) acc = fmaf(-Ab[r * SF + s], x[s], acc);
                x[r] = acc;
            }
            float *Tb = &L.u.inv.t[16 * lg * SF + 16 * lg];
#pragma unroll
            for (int r = 0; r < 16; r++) Tb[r * SF + ln] = x[r];
        }
        __syncthreads();
        // Level 1: T_{b+1,b} = -T_{b+1,b+1} A_{b+1,b} T_{b,b} for b = 0, 2
        if (wave < 2) {
            const int b0 = 32 * wave;
            floatx4 X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++)
                X = mma4(L.u.inv.a[(b0 + 16 + ln) * SF + b0 + 4 * s + lg], L.u.inv.t[(b0 + 4 * s + lg) * SF + b0 + ln], X);
            floatx4 Y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++) Y = mma4(L.u.inv.t[(b0 + 16 + ln) * SF + b0 + 16 + 4 * lg + s], X[s], Y);
#pragma unroll
            for (int r = 0; r < 4; r++) L.u.inv.t[(b0 + 16 + 4 * lg + r) * SF + b0 + ln] = -Y[r];
        }
        __syncthreads();
        // Level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32];
        // wave J makes block column J of it
        if (wave < 2) {
            const int J = wave;
            floatx4 X2 = {0.0f, 0.0f, 0.0f, 0.0f}, X3 = X2;
            for (int K = J; K < 2; K++) {
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    const float bt = L.u.inv.t[(16 * K + 4 * s + lg) * SF + 16 * J + ln];
                    X2 = mma4(L.u.inv.a[(32 + ln) * SF + 16 * K + 4 * s + lg], bt, X2);
                    X3 = mma4(L.u.inv.a[(48 + ln) * SF + 16 * K + 4 * s + lg], bt, X3);
                }
            }
            floatx4 Y2 = {0.0f, 0.0f, 0.0f, 0.0f}, Y3 = Y2;
#pragma unroll
            for (int s = 0; s < 4; s++) {
                Y2 = mma4(L.u.inv.t[(32 + ln) * SF + 32 + 4 * lg + s], X2[s], Y2);
                Y3 = mma4(L.u.inv.t[(48 + ln) * SF + 32 + 4 * lg + s], X2[s], Y3);
                Y3 = mma4(L.u.inv.t[(48 + ln) * SF + 48 + 4 * lg + s], X3[s], Y3);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                L.u.inv.t[(32 + 4 * lg + r) * SF + 16 * J + ln] = -Y2[r];
                L.u.inv.t[(48 + 4 * lg + r) * SF + 16 * J + ln] = -Y3[r];
            }
        }
        __syncthreads();

        // ---- T1 = T diag(beta e^g), T2 = T diag(beta), split; T's upper part is 0
        for (int x = tid; x < CH * CH / 8; x += NT) {
            const int i = x >> 3, j0 = 8 * (x & 7);
            bf16x8 h1, l1, h2, l2;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int j = j0 + e;
                const float t = j <= i ? L.u.inv.t[i * SF + j] : 0.0f;
                const float t2 = t * L.beta[j];
                const float t1 = t2 * L.eg[j];
                split(t1, h1, l1, e);
                split(t2, h2, l2, e);
            }
            *reinterpret_cast<bf16x8 *>(&L.t1h[i * SC + j0]) = h1;
            *reinterpret_cast<bf16x8 *>(&L.t1l[i * SC + j0]) = l1;
            *reinterpret_cast<bf16x8 *>(&L.t2h[i * SC + j0]) = h2;
            *reinterpret_cast<bf16x8 *>(&L.t2l[i * SC + j0]) = l2;
        }
        __syncthreads();

        // ---- W^T = K^T T1^T: wave owns key rows 16w..16w+15 (DT == NW); store -W split
        {
            floatx4 acc[4];
#pragma unroll
            for (int it = 0; it < 4; it++) acc[it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                const bf16x8 av = ld8(&L.kt[(16 * wave + ln) * SC + 32 * jb + 8 * lg]);
#pragma unroll
                for (int it = 0; it < 4; it++) {
                    acc[it] = mma(av, ld8(&L.t1h[(16 * it + ln) * SC + 32 * jb + 8 * lg]), acc[it]);
                    acc[it] = mma(av, ld8(&L.t1l[(16 * it + ln) * SC + 32 * jb + 8 * lg]), acc[it]);
                }
            }
#pragma unroll
            for (int it = 0; it < 4; it++) {
                bf16x4 h, l;
#pragma unroll
                for (int r = 0; r < 4; r++) split(-acc[it][r], h, l, r);
                const int off = (16 * it + ln) * SD + 16 * wave + 4 * lg;
                *reinterpret_cast<bf16x4 *>(&L.u.w.h[off]) = h;
                *reinterpret_cast<bf16x4 *>(&L.u.w.l[off]) = l;
            }
        }
        // ---- U = T2 V for this wave's value columns (accumulators become U')
        floatx4 U[4];
#pragma unroll
        for (int it = 0; it < 4; it++) U[it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            const bf16x8 bv = ld8(&L.vt[(e0 + ln) * SC + 32 * jb + 8 * lg]);
#pragma unroll
            for (int it = 0; it < 4; it++) {
                U[it] = mma(ld8(&L.t2h[(16 * it + ln) * SC + 32 * jb + 8 * lg]), bv, U[it]);
                U[it] = mma(ld8(&L.t2l[(16 * it + ln) * SC + 32 * jb + 8 * lg]), bv, U[it]);
            }
        }
        __syncthreads();  // -W complete

        // ---- state operand (contraction over key rows, permuted slots)
        bf16x8 Sh[KB], Sl[KB];
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                split(S[2 * kb][r], Sh[kb], Sl[kb], r);
                split(S[2 * kb + 1][r], Sh[kb], Sl[kb], 4 + r);
            }
        // ---- U' = U - W S and Q S
        floatx4 O[4];
#pragma unroll
        for (int it = 0; it < 4; it++) {
            floatx4 qs = {0.0f, 0.0f, 0.0f, 0.0f};
            const int row = (16 * it + ln) * SD + 4 * lg;
#pragma unroll
            for (int kb = 0; kb < KB; kb++) {
                const bf16x8 wh = ld_pair(&L.u.w.h[row + 32 * kb]);
                const bf16x8 wl = ld_pair(&L.u.w.l[row + 32 * kb]);
                const bf16x8 qa = ld_pair(&L.qr[row + 32 * kb]);
                U[it] = mma(wh, Sh[kb], U[it]);
                U[it] = mma(wh, Sl[kb], U[it]);
                U[it] = mma(wl, Sh[kb], U[it]);
                qs = mma(qa, Sh[kb], qs);
                qs = mma(qa, Sl[kb], qs);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) qs[r] *= L.eg[16 * it + 4 * lg + r];
            O[it] = qs;
        }
        // ---- U' as an operand (contraction over tokens), plain and scaled by e^{g_C - g_j}
        bf16x8 Vh[2], Vl[2], Gh[2], Gl[2];
#pragma unroll
        for (int jb = 0; jb < 2; jb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int ja = 32 * jb + 4 * lg + r, jc = ja + 16;
                split(U[2 * jb][r], Vh[jb], Vl[jb], r);
                split(U[2 * jb + 1][r], Vh[jb], Vl[jb], 4 + r);
                split(U[2 * jb][r] * L.gam[ja], Gh[jb], Gl[jb], r);
                split(U[2 * jb + 1][r] * L.gam[jc], Gh[jb], Gl[jb], 4 + r);
            }
        // ---- O += P U' (causal: token block jb only feeds rows i >= 32 jb)
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const int row = (16 * it + ln) * SC + 4 * lg;
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                if (32 * jb > 16 * it + 15) continue;
                const bf16x8 phv = ld_pair(&L.ph[row + 32 * jb]);
                const bf16x8 plv = ld_pair(&L.pl[row + 32 * jb]);
                O[it] = mma(phv, Vh[jb], O[it]);
                O[it] = mma(phv, Vl[jb], O[it]);
                O[it] = mma(plv, Vh[jb], O[it]);
            }
        }
        // ---- outputs of the chunk's tokens
#pragma unroll
        for (int it = 0; it < 4; it++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int t = c0 + 16 * it + 4 * lg + r;
                if (t < T) og[(size_t)t * tv + e0 + ln] = (__bf16)O[it][r];
            }
        // ---- S <- e^{g_C} S + K^T diag(e^{g_C - g}) U'
        const float egc = L.eg[CH - 1];
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            floatx4 acc = S[dt] * egc;
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                const bf16x8 ka = ld_pair(&L.kt[(16 * dt + ln) * SC + 32 * jb + 4 * lg]);
                acc = mma(ka, Gh[jb], acc);
                acc = mma(ka, Gl[jb], acc);
            }
            S[dt] = acc;
        }
    }

#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 4; r++) Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + ln] = S[dt][r];
}

}  // namespace

hipError_t launch_prefill(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                          const float *a, const float *b, void *o, int T, hipStream_t st)
{
    const int hk = d.hk ? d.hk : d.H;
    PrefillArgs A{S,
                  static_cast<const __bf16 *>(q),
                  static_cast<const __bf16 *>(k),
                  static_cast<const __bf16 *>(v),
                  a,
                  b,
                  static_cast<__bf16 *>(o),
                  T,
                  d.H,
                  hk,
                  make_divisor((unsigned)d.H),
                  make_divisor((unsigned)(d.H / hk))};
    const unsigned grid = (unsigned)d.B * (unsigned)d.H;
    if (d.dk == 128) {
        hipLaunchKernelGGL(prefill_kernel<128>, dim3(grid), dim3(512), 0, st, A);
    } else {
        hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(256), 0, st, A);
    }
    return hipGetLastError();
}

}  // namespace gdnq
