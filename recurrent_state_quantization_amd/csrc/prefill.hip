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
// (i >= j), beta = b and S the state at the chunk start (the kernel keeps
// the gates as base-2 logarithms and uses the hardware log2/exp2):
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
// runs in fp32: forward substitution on the 16x16 diagonal blocks, then
// block merges on v_mfma_f32_16x16x4f32.
//
// Two kernels: prefill_kernel (below, 64-token chunks, one group of waves,
// used for D = 64) and prefill_ws_kernel (further down, 32-token chunks, a
// chunk group and a state group of waves, used for D = 128).  In both, one
// workgroup per (batch, head) walks the chunks in order and each state wave
// owns 32 value columns of the state, which stay in fp32 MFMA accumulators
// for the whole sequence: every state-dependent product needs only the
// wave's own columns, and the accumulators feed the next product's operand
// directly by permuting the contraction index (slots 0..3 of lane group g
// take k = 4g..4g+3 of one 16-row tile, slots 4..7 those of the next tile;
// the LDS operand on the other side is read in the same order).  The
// chunk-local part (K K^T, Q K^T, the inverse) is shared through LDS.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;  // tokens per chunk

__device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma4(float a, float b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16
// lanes, then the last lane of rows 0 and 2 into rows 1 and 3, then lane 31
// into rows 2 and 3 (DPP row_shr, row_bcast:15, row_bcast:31).
__device__ __forceinline__ float scan64(float x)
{
#define GDNQ_DPP(x, ctrl, rmask) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rmask, 0xf, true))
    x += GDNQ_DPP(x, 0x111, 0xf);  // row_shr:1
    x += GDNQ_DPP(x, 0x112, 0xf);  // row_shr:2
    x += GDNQ_DPP(x, 0x114, 0xf);  // row_shr:4
    x += GDNQ_DPP(x, 0x118, 0xf);  // row_shr:8
    x += GDNQ_DPP(x, 0x142, 0xa);  // row_bcast:15 into rows 1, 3
    x += GDNQ_DPP(x, 0x143, 0xc);  // row_bcast:31 into rows 2, 3
#undef GDNQ_DPP
    return x;
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

__device__ __forceinline__ u32x4 keep(u32x4 x, bool ok) { return ok ? x : u32x4{0u, 0u, 0u, 0u}; }

// one thread's share of a chunk's inputs, held in registers while the
// previous chunk is computed
struct ChunkRegs {
    u32x4 k[4], q[4], v[4];
    float a, b;
};

// Lower 16x16 tiles (I >= J) of a 64x64 chunk matrix, job n -> (I, J) from
// nibble n of two constants (a table in memory would be a vector load, and
// its wait would also wait for the next chunk's prefetch issued before it).
__device__ __forceinline__ int tile_i(int n) { return (int)((0x3333222110ull >> (4 * n)) & 15u); }
__device__ __forceinline__ int tile_j(int n) { return (int)((0x3210210100ull >> (4 * n)) & 15u); }

}  // namespace

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
            float a[CH * SF];  // A^T (A strictly lower): a[j * SF + i] = A_ij
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


template <int D>
__global__ __launch_bounds__(D * 2, 1) void prefill_kernel(PrefillArgs A)
{
    using Lds = PrefillLds<D>;
    constexpr int SD = Lds::SD, SC = Lds::SC, SF = Lds::SF;
    constexpr int NW = D / 32, NT = NW * 64;  // waves; wave w owns value columns 32w..32w+31
    constexpr int KB = D / 32;                // 32-wide blocks along a head dim
    constexpr int DT = D / 16;                // 16-row tiles along a head dim
    static_assert(DT == 2 * NW, "two key-row tiles of W per wave");
    __shared__ Lds L;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned bh = __builtin_amdgcn_workgroup_id_x();
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
    const int e0 = 32 * wave;  // value columns e0 + 16 et + ln, et = 0, 1
    int lg = (tid & 63) >> 4, ln = tid & 15;

    // P's upper tiles are never written: clear them once.
    for (int x = tid; x < CH * SC; x += NT) {
        L.ph[x] = (__bf16)0.0f;
        L.pl[x] = (__bf16)0.0f;
    }

    // S[et][dt][r] = S[16 dt + 4 lg + r][e0 + 16 et + ln] (MFMA accumulator layout)
    floatx4 S[2][DT];
#pragma unroll
    for (int et = 0; et < 2; et++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                S[et][dt][r] = Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln];

    // identity operands of the transposes: eye[h] holds B[k][n] = (k == n + 16 h)
    bf16x8 eye[2];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) eye[h][i] = (__bf16)(8 * lg + i == ln + 16 * h ? 1.0f : 0.0f);

    // Chunk loads.  Wave w takes pieces p = 4w..4w+3 of each of K, Q, V: token
    // group p / KB (16 tokens), channel block p % KB (32 channels); lane
    // (lg, ln) takes token 16 tg + ln, channels 32 db + 8 lg .. +7, i.e. a
    // 16 x 32 tile in the A-operand layout, 64 contiguous bytes per token.
    // Lanes of wave 0 also take the gate and beta of token lane.  Every load
    // is unconditional (rows past the end are clamped) and those rows are
    // zeroed only when staged, so the compiler counts the loads and waits for
    // them at staging alone.
    auto load = [=](int c0, int which, ChunkRegs &r) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int p = 4 * wave + s, tg = p / KB, db = p % KB;
            const size_t u = (size_t)min(c0 + 16 * tg + ln, T - 1);
            const int off = 32 * db + 8 * lg;
            if (which == 0) r.k[s] = *reinterpret_cast<const u32x4 *>(kg + u * tk + off);
            if (which == 1) r.q[s] = *reinterpret_cast<const u32x4 *>(qg + u * tk + off);
            if (which == 2) r.v[s] = *reinterpret_cast<const u32x4 *>(vg + u * tv + off);
        }
        if (which == 2) {
            const size_t ua = (size_t)min(c0 + (tid & 63), T - 1);
            r.a = ag[ua * A.H];
            r.b = bg[ua * A.H];
        }
    };

    ChunkRegs nx;
    load(0, 0, nx);
    load(0, 1, nx);
    load(0, 2, nx);
    for (int c0 = 0; c0 < T; c0 += CH) {
        __syncthreads();  // the previous chunk is done with every LDS tile
        // Lane indices pass through an empty asm each chunk, so the LDS
        // addresses built from them are formed inside the loop: hoisted out
        // of it, the few dozen distinct addresses would not fit in registers.
        asm volatile("" : "+v"(lg), "+v"(ln));
        const int lane = 16 * lg + ln;

        // ---- stage the chunk: K, Q token-major; K^T, V^T through the matrix
        // cores (X E_h puts 4 consecutive tokens of one channel in each lane;
        // exact: one product by 1 per output); rows past the end are zero
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int p = 4 * wave + s, tg = p / KB, db = p % KB;
            const bool ok = c0 + 16 * tg + ln < T;
            const u32x4 kx = keep(nx.k[s], ok), qx = keep(nx.q[s], ok), vx = keep(nx.v[s], ok);
            const int row = (16 * tg + ln) * SD + 32 * db + 8 * lg;
            *reinterpret_cast<u32x4 *>(&L.kr[row]) = kx;
            *reinterpret_cast<u32x4 *>(&L.qr[row]) = qx;
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const floatx4 tkx = mma(__builtin_bit_cast(bf16x8, kx), eye[h], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                const floatx4 tvx = mma(__builtin_bit_cast(bf16x8, vx), eye[h], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                const int col = (32 * db + 16 * h + ln) * SC + 16 * tg + 4 * lg;
                *reinterpret_cast<bf16x4 *>(&L.kt[col]) =
                    bf16x4{(__bf16)tkx[0], (__bf16)tkx[1], (__bf16)tkx[2], (__bf16)tkx[3]};
                *reinterpret_cast<bf16x4 *>(&L.vt[col]) =
                    bf16x4{(__bf16)tvx[0], (__bf16)tvx[1], (__bf16)tvx[2], (__bf16)tvx[3]};
            }
        }
        if (wave == 0) {  // cumulative log2-gates over the chunk (inclusive scan)
            const bool ok = c0 + lane < T;
            const float x = scan64(__builtin_amdgcn_logf(ok ? nx.a : 1.0f));  // padding: gate 1, beta 0
            const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
            L.g[lane] = x;
            L.eg[lane] = __builtin_amdgcn_exp2f(x);
            L.gam[lane] = __builtin_amdgcn_exp2f(glast - x);
            L.beta[lane] = ok ? nx.b : 0.0f;
        }
        __syncthreads();
        // the next chunk's loads go out in three parts spread over this chunk:
        // all at once, every workgroup's burst fills the memory queues and the
        // waves stall on issue
        const bool more = c0 + CH < T;
        if (more) load(c0 + CH, 0, nx);

        // ---- A = strictly lower diag(beta)(K K^T . Gam), stored transposed
        // (fp32), and P = (Q K^T . Gam . [i >= j]) (split), one lower 16x16
        // tile (I, J) of both per job.  The K K^T tile is computed with rows i
        // and the P tile transposed (rows j), so that each lane holds 4
        // consecutive i of one j for A^T and 4 consecutive j of one i for P.
        for (int job = wave; job < 10; job += NW) {
            const int I = tile_i(job), J = tile_j(job);
            floatx4 gk = {0.0f, 0.0f, 0.0f, 0.0f}, gq = gk;
#pragma unroll
            for (int kb = 0; kb < KB; kb++) {
                const bf16x8 kj = ld8(&L.kr[(16 * J + ln) * SD + 32 * kb + 8 * lg]);
                gk = mma(ld8(&L.kr[(16 * I + ln) * SD + 32 * kb + 8 * lg]), kj, gk);
                gq = mma(kj, ld8(&L.qr[(16 * I + ln) * SD + 32 * kb + 8 * lg]), gq);
            }
            {   // A^T: lane (lg, ln) has G[16I + 4lg + r][16J + ln]
                const int i0 = 16 * I + 4 * lg, j = 16 * J + ln;
                const floatx4 gi = *reinterpret_cast<const floatx4 *>(&L.g[i0]);
                const floatx4 bi = *reinterpret_cast<const floatx4 *>(&L.beta[i0]);
                const float gj = L.g[j];
                floatx4 out;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    out[r] = i0 + r > j ? (bi[r] * gk[r]) * __builtin_amdgcn_exp2f(gi[r] - gj) : 0.0f;
                *reinterpret_cast<floatx4 *>(&L.u.inv.a[j * SF + i0]) = out;
            }
            {   // P: lane (lg, ln) has (Q K^T)[16I + ln][16J + 4lg + r]
                const int i = 16 * I + ln, j0 = 16 * J + 4 * lg;
                const float gi = L.g[i];
                const floatx4 gj = *reinterpret_cast<const floatx4 *>(&L.g[j0]);
                bf16x4 h, l;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    split(i >= j0 + r ? gq[r] * __builtin_amdgcn_exp2f(gi - gj[r]) : 0.0f, h, l, r);
                *reinterpret_cast<bf16x4 *>(&L.ph[i * SC + j0]) = h;
                *reinterpret_cast<bf16x4 *>(&L.pl[i * SC + j0]) = l;
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1}.  Level 0: the four 16x16 diagonal blocks by
        // forward substitution, lane = (block lg, column c = ln).  y = T e_c - e_c
        // solves y_r = -A_rc - sum_{s<r} A_rs y_s (A's diagonal blocks are
        // strictly lower, so y_r = 0 for r <= c); the sums are updated
        // right-looking (column s of A is row s of the stored A^T, read with
        // 16-byte loads), so the dependent chain is 16 steps long.
        if (wave == 0) {
            const float *At = &L.u.inv.a[16 * lg * SF + 16 * lg];  // At[s * SF + r] = A_rs
            // all loads first (40 x 16 bytes, broadcast within a block): left to
            // the scheduler they go out one step ahead and the 16 steps wait
            // on 16 LDS round trips
            floatx4 yv[4], col[15][4];
#pragma unroll
            for (int q = 0; q < 4; q++) yv[q] = *reinterpret_cast<const floatx4 *>(&At[ln * SF + 4 * q]);
#pragma unroll
            for (int s = 0; s < 15; s++)
#pragma unroll
                for (int q = (s + 1) / 4; q < 4; q++) col[s][q] = *reinterpret_cast<const floatx4 *>(&At[s * SF + 4 * q]);
            __builtin_amdgcn_sched_barrier(0);
            float y[16];
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int e = 0; e < 4; e++) y[4 * q + e] = -yv[q][e];
#pragma unroll
            for (int s = 0; s < 15; s++)
#pragma unroll
                for (int q = (s + 1) / 4; q < 4; q++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        if (4 * q + e > s) y[4 * q + e] = fmaf(-col[s][q][e], y[s], y[4 * q + e]);
            float *Tb = &L.u.inv.t[16 * lg * SF + 16 * lg];
#pragma unroll
            for (int r = 0; r < 16; r++) Tb[r * SF + ln] = y[r];
            Tb[ln * SF + ln] = 1.0f;
        }
        __syncthreads();
        // Level 1: T_{b+1,b} = -T_{b+1,b+1} A_{b+1,b} T_{b,b} for b = 0, 2
        if (wave < 2) {
            const int b0 = 32 * wave;
            floatx4 X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++)
                X = mma4(L.u.inv.a[(b0 + 4 * s + lg) * SF + b0 + 16 + ln], L.u.inv.t[(b0 + 4 * s + lg) * SF + b0 + ln], X);
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
                    X2 = mma4(L.u.inv.a[(16 * K + 4 * s + lg) * SF + 32 + ln], bt, X2);
                    X3 = mma4(L.u.inv.a[(16 * K + 4 * s + lg) * SF + 48 + ln], bt, X3);
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

        if (more) load(c0 + CH, 1, nx);

        // ---- T1 = T diag(beta e^g), T2 = T diag(beta), split; T's upper part is 0
#pragma unroll
        for (int sx = 0; sx < CH * CH / 8 / NT; sx++) {
            const int x = tid + sx * NT, i = x >> 3, j0 = 8 * (x & 7);
            bf16x8 h1, l1, h2, l2;
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const floatx4 tv = *reinterpret_cast<const floatx4 *>(&L.u.inv.t[i * SF + j0 + 4 * q]);
                const floatx4 bv = *reinterpret_cast<const floatx4 *>(&L.beta[j0 + 4 * q]);
                const floatx4 ev = *reinterpret_cast<const floatx4 *>(&L.eg[j0 + 4 * q]);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float t = j0 + 4 * q + e <= i ? tv[e] : 0.0f;  // T's upper part is 0
                    const float t2 = t * bv[e];
                    const float t1 = t2 * ev[e];
                    split(t1, h1, l1, 4 * q + e);
                    split(t2, h2, l2, 4 * q + e);
                }
            }
            *reinterpret_cast<bf16x8 *>(&L.t1h[i * SC + j0]) = h1;
            *reinterpret_cast<bf16x8 *>(&L.t1l[i * SC + j0]) = l1;
            *reinterpret_cast<bf16x8 *>(&L.t2h[i * SC + j0]) = h2;
            *reinterpret_cast<bf16x8 *>(&L.t2l[i * SC + j0]) = l2;
        }
        __syncthreads();

        // ---- W^T = K^T T1^T: wave w makes key-row tiles 2w, 2w+1; store -W split
        {
            floatx4 acc[2][4];
#pragma unroll
            for (int x = 0; x < 2; x++)
#pragma unroll
                for (int it = 0; it < 4; it++) acc[x][it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int jb = 0; jb < 2; jb++) {
                bf16x8 av[2];
#pragma unroll
                for (int x = 0; x < 2; x++) av[x] = ld8(&L.kt[(16 * (2 * wave + x) + ln) * SC + 32 * jb + 8 * lg]);
                bf16x8 bh[4], bl[4];
#pragma unroll
                for (int it = 0; it < 4; it++) {
                    bh[it] = ld8(&L.t1h[(16 * it + ln) * SC + 32 * jb + 8 * lg]);
                    bl[it] = ld8(&L.t1l[(16 * it + ln) * SC + 32 * jb + 8 * lg]);
                }
#pragma unroll
                for (int it = 0; it < 4; it++)
#pragma unroll
                    for (int x = 0; x < 2; x++) acc[x][it] = mma(av[x], bh[it], acc[x][it]);
#pragma unroll
                for (int it = 0; it < 4; it++)
#pragma unroll
                    for (int x = 0; x < 2; x++) acc[x][it] = mma(av[x], bl[it], acc[x][it]);
            }
#pragma unroll
            for (int x = 0; x < 2; x++)
#pragma unroll
                for (int it = 0; it < 4; it++) {
                    bf16x4 h, l;
#pragma unroll
                    for (int r = 0; r < 4; r++) split(-acc[x][it][r], h, l, r);
                    const int off = (16 * it + ln) * SD + 16 * (2 * wave + x) + 4 * lg;
                    *reinterpret_cast<bf16x4 *>(&L.u.w.h[off]) = h;
                    *reinterpret_cast<bf16x4 *>(&L.u.w.l[off]) = l;
                }
        }
        // ---- U = T2 V for this wave's value columns (accumulators become U')
        floatx4 U[2][4];
#pragma unroll
        for (int et = 0; et < 2; et++)
#pragma unroll
            for (int it = 0; it < 4; it++) U[et][it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            bf16x8 bv[2];
#pragma unroll
            for (int et = 0; et < 2; et++) bv[et] = ld8(&L.vt[(e0 + 16 * et + ln) * SC + 32 * jb + 8 * lg]);
            bf16x8 th[4], tl[4];
#pragma unroll
            for (int it = 0; it < 4; it++) {
                th[it] = ld8(&L.t2h[(16 * it + ln) * SC + 32 * jb + 8 * lg]);
                tl[it] = ld8(&L.t2l[(16 * it + ln) * SC + 32 * jb + 8 * lg]);
            }
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) U[et][it] = mma(th[it], bv[et], U[et][it]);
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) U[et][it] = mma(tl[it], bv[et], U[et][it]);
        }
        __syncthreads();  // -W complete
        if (more) load(c0 + CH, 2, nx);

        // ---- state operand (contraction over key rows, permuted slots)
        bf16x8 Sh[2][KB], Sl[2][KB];
#pragma unroll
        for (int et = 0; et < 2; et++)
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    split(S[et][2 * kb][r], Sh[et][kb], Sl[et][kb], r);
                    split(S[et][2 * kb + 1][r], Sh[et][kb], Sl[et][kb], 4 + r);
                }
        // ---- U' = U - W S and Q S (each operand read from LDS feeds both column tiles)
        floatx4 O[2][4];
#pragma unroll
        for (int et = 0; et < 2; et++)
#pragma unroll
            for (int it = 0; it < 4; it++) O[et][it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
            bf16x8 wh[4], wl[4], qa[4];
#pragma unroll
            for (int it = 0; it < 4; it++) {
                const int row = (16 * it + ln) * SD + 4 * lg + 32 * kb;
                wh[it] = ld_pair(&L.u.w.h[row]);
                wl[it] = ld_pair(&L.u.w.l[row]);
                qa[it] = ld_pair(&L.qr[row]);
            }
            // 16 independent accumulators; each product order keeps a
            // chain's consecutive products 16 instructions apart
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) {
                    U[et][it] = mma(wh[it], Sh[et][kb], U[et][it]);
                    O[et][it] = mma(qa[it], Sh[et][kb], O[et][it]);
                }
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) {
                    U[et][it] = mma(wh[it], Sl[et][kb], U[et][it]);
                    O[et][it] = mma(qa[it], Sl[et][kb], O[et][it]);
                }
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) U[et][it] = mma(wl[it], Sh[et][kb], U[et][it]);
        }
#pragma unroll
        for (int it = 0; it < 4; it++) {
            const floatx4 eg = *reinterpret_cast<const floatx4 *>(&L.eg[16 * it + 4 * lg]);
#pragma unroll
            for (int et = 0; et < 2; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) O[et][it][r] *= eg[r];
        }
        // ---- U' as an operand (contraction over tokens), plain and scaled by e^{g_C - g_j}
        bf16x8 Vh[2][2], Vl[2][2], Gh[2][2], Gl[2][2];
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            const floatx4 ga = *reinterpret_cast<const floatx4 *>(&L.gam[32 * jb + 4 * lg]);
            const floatx4 gc = *reinterpret_cast<const floatx4 *>(&L.gam[32 * jb + 16 + 4 * lg]);
#pragma unroll
            for (int et = 0; et < 2; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    split(U[et][2 * jb][r], Vh[et][jb], Vl[et][jb], r);
                    split(U[et][2 * jb + 1][r], Vh[et][jb], Vl[et][jb], 4 + r);
                    split(U[et][2 * jb][r] * ga[r], Gh[et][jb], Gl[et][jb], r);
                    split(U[et][2 * jb + 1][r] * gc[r], Gh[et][jb], Gl[et][jb], 4 + r);
                }
        }
        // ---- O += P U' (causal: token block jb only feeds rows i >= 32 jb)
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            bf16x8 phv[4], plv[4];
#pragma unroll
            for (int it = 2 * jb; it < 4; it++) {
                const int row = (16 * it + ln) * SC + 4 * lg + 32 * jb;
                phv[it] = ld_pair(&L.ph[row]);
                plv[it] = ld_pair(&L.pl[row]);
            }
#pragma unroll
            for (int it = 2 * jb; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) O[et][it] = mma(phv[it], Vh[et][jb], O[et][it]);
#pragma unroll
            for (int it = 2 * jb; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) O[et][it] = mma(phv[it], Vl[et][jb], O[et][it]);
#pragma unroll
            for (int it = 2 * jb; it < 4; it++)
#pragma unroll
                for (int et = 0; et < 2; et++) O[et][it] = mma(plv[it], Vh[et][jb], O[et][it]);
        }
        // ---- outputs of the chunk's tokens: through LDS (K's token-major tile
        // is free after the A/P tiles), then 16-byte coalesced stores
#pragma unroll
        for (int et = 0; et < 2; et++)
#pragma unroll
            for (int it = 0; it < 4; it++)
#pragma unroll
                for (int r = 0; r < 4; r++) L.kr[(16 * it + 4 * lg + r) * SD + e0 + 16 * et + ln] = (__bf16)O[et][it][r];
        // ---- S <- e^{g_C} S + K^T diag(e^{g_C - g}) U'
        const float egc = L.eg[CH - 1];
#pragma unroll
        for (int et = 0; et < 2; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++) S[et][dt] *= egc;
#pragma unroll
        for (int jb = 0; jb < 2; jb++) {
            bf16x8 ka[DT];
#pragma unroll
            for (int dt = 0; dt < DT; dt++) ka[dt] = ld_pair(&L.kt[(16 * dt + ln) * SC + 32 * jb + 4 * lg]);
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int et = 0; et < 2; et++) S[et][dt] = mma(ka[dt], Gh[et][jb], S[et][dt]);
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int et = 0; et < 2; et++) S[et][dt] = mma(ka[dt], Gl[et][jb], S[et][dt]);
        }
        __syncthreads();  // the outputs are staged
#pragma unroll
        for (int x = tid; x < CH * D / 8; x += NT) {
            const int t = x / (D / 8), c = 8 * (x % (D / 8));
            if (c0 + t < T)
                *reinterpret_cast<u32x4 *>(og + (size_t)(c0 + t) * tv + c) =
                    *reinterpret_cast<const u32x4 *>(&L.kr[t * SD + c]);
        }
    }

#pragma unroll
    for (int et = 0; et < 2; et++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln] = S[et][dt][r];
}

// ---------------------------------------------------------------------------
// Two wave groups, 32-token chunks (D = 128, prefill_ws_kernel).
//
// The chunk-local part of a chunk (staging, the A and P tiles, the inverse T
// and its scaled splits T1, T2) never reads the state, so it runs a chunk
// ahead of the state part on waves of its own.  Per chunk there are two
// phases, each closed by a barrier; in iteration c:
//   phase X  chunk group: the Gram tiles of chunk c+1 (waves 0-2), wave 0
//            taking A's three tiles and from them T's diagonal blocks
//            (forward substitution) and its one block merge, in-wave
//            through LDS; K^T of chunk c+1 from its staged K tile;
//            state group: chunk c's U' = T2 V - T1 (K S), O = diag(e^g) Q S
//            + P U' and its stores (each wave its own columns, through
//            LDS);
//   phase Y  chunk group: T1 and T2 of chunk c+1 (wave 0), while waves 1-3
//            stage chunk c+2 (K, Q, V, the gates) and load chunk c+3;
//            state group: chunk c's state update, the split state and chunk
//            c+1's K S and Q S.
// (Roles as for NS = 1; a split head rotates the chunk roles, see the
// kernel.)  The state update sits in phase Y, beside the lighter chunk work:
// K^T is the one staged tile that phase Y does not rewrite.
// The state group is WS_SW waves of D / WS_SW value columns; its state stays
// in MFMA accumulators.  Four waves of 32 columns measured faster than eight
// of 16 (each LDS operand read then feeds two accumulators).  Tiles are
// double-buffered by chunk parity: a chunk's buffer is written while the
// chunk is prepared and read until it is finished, and is restaged for
// chunk c+2 only in phase Y of iteration c.  U' = T2 V -
// T1 (K S) is the form's U - W S with W S = T1 (K S) taken in the other
// order: the chunk group then has no D-wide product, and the state group's
// K S reads its operands in the same pass as Q S.
constexpr int WC = 32;     // tokens per chunk of the two-group kernel
constexpr int WS_SW = 4;   // its state waves (D / WS_SW value columns each)

namespace {

// LDS accesses of one wave complete in issue order: once its own stores have
// completed, its other lanes read them (and the compiler keeps the order)
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// one staging wave's share of a chunk: 8 pieces of one tensor (16 tokens x
// 32 channels each, in the A-operand layout), and the gate and beta of
// token lane
struct WsRegs {
    u32x4 x[8];
    float a, b;
};

}  // namespace

template <int D>
struct __attribute__((aligned(16))) WsBuf {
    static constexpr int SD = D + 8;    // row stride (bf16) of [WC][D] tiles
    static constexpr int SC = WC + 8;   // row stride (bf16) of [.][WC] tiles
    __bf16 kr[WC * SD];                 // K, token-major
    __bf16 qr[WC * SD];                 // Q, token-major
    __bf16 kt[D * SC];                  // K^T
    __bf16 vt[D * SC];                  // V^T
    __bf16 ph[WC * SC], pl[WC * SC];    // P = (Q K^T . Gam . [i >= j]), split
    __bf16 t1h[WC * SC], t1l[WC * SC];  // T1 = T diag(beta e^g), split
    __bf16 t2h[WC * SC], t2l[WC * SC];  // T2 = T diag(beta), split
    float g[WC], eg[WC], gam[WC], beta[WC];
};

template <int D>
struct WsLds {
    static constexpr int SF = WC + 4;   // row stride (fp32) of [WC][WC] tiles
    WsBuf<D> b[2];                      // by chunk parity
    float a[WC * SF];                   // A^T of the chunk being inverted
    float t[WC * SF];                   // its T (lower)
    __bf16 out[WC * (D + 8)];           // outputs of the chunk being finished (per wave, its columns)
};

// NS workgroups share a head (NS = 1, 2, 4): each prepares every chunk in
// full (the chunk-local work is small) and finishes D / NS of the head's value
// columns, so a batch of fewer heads than CUs still fills the chip.
template <int D, int NS>
__global__ __launch_bounds__(64 * (4 + WS_SW / NS), 1) void prefill_ws_kernel(PrefillArgs A)
{
    using Buf = WsBuf<D>;
    constexpr int SD = Buf::SD, SC = Buf::SC, SF = WsLds<D>::SF;
    constexpr int NT = 64 * (4 + WS_SW / NS);        // threads (waves 0-3: chunk group)
    constexpr int ET = D / 16 / WS_SW;               // 16-column tiles per state wave
    constexpr int KB = D / 32, DT = D / 16;
    static_assert(D == 128 && ET >= 1 && ET * 16 * WS_SW == D, "state waves split the value columns");
    static_assert(NS >= 1 && WS_SW % NS == 0, "each workgroup keeps whole state waves");
    __shared__ WsLds<D> L;

    const int tid = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned gid = __builtin_amdgcn_workgroup_id_x();
    const unsigned bh = gid / NS;                    // the head
    const int part = (int)(gid % NS);                // its share of the value columns
    const unsigned bb = div_by(bh, A.byH), hh = bh - bb * (unsigned)A.H;
    const unsigned kh = div_by(hh, A.byG);
    const int T = A.T;
    const size_t tk = (size_t)A.HK * D, tv = (size_t)A.H * D;
    const __bf16 *qg = A.q + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *kg = A.k + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *vg = A.v + (size_t)bb * T * tv + (size_t)hh * D;
    __bf16 *og = A.o + (size_t)bb * T * tv + (size_t)hh * D;
    const float *ag = A.a + (size_t)bb * T * A.H + hh;
    const float *bg = A.b + (size_t)bb * T * A.H + hh;
    float *Sg = A.S + (size_t)bh * D * D;
    const bool cgroup = wave < 4;
    // chunk-group role: 0 Gram tiles of A and the inverse, 1 K, 2 Q and the
    // gates, 3 V.  With fewer than four state waves, role 0 goes to the
    // SIMD of wave 3, which then hosts no state wave.
    const int role = NS > 1 ? (wave + 1) & 3 : wave;
    const int e0 = part * (D / NS) + 16 * ET * (wave - 4);  // state waves: value columns e0 + 16 et + ln
    int lg = (tid & 63) >> 4, ln = tid & 15;
    const int nch = (T + WC - 1) / WC;

    // P's upper tile is never written: clear it once in both buffers
    for (int x = tid; x < WC * SC; x += NT) {
#pragma unroll
        for (int p = 0; p < 2; p++) {
            L.b[p].ph[x] = (__bf16)0.0f;
            L.b[p].pl[x] = (__bf16)0.0f;
        }
    }

    // S[et][dt][r] = S[16 dt + 4 lg + r][e0 + 16 et + ln] (state waves)
    floatx4 S[ET][DT];

    // identity operands of the transposes: eye[h] holds B[k][n] = (k == n + 16 h)
    bf16x8 eye[2];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < 8; i++) eye[h][i] = (__bf16)(8 * lg + i == ln + 16 * h ? 1.0f : 0.0f);

    // Staging waves 1, 2, 3 load K, Q, V: piece p = token group p / KB (16
    // tokens), channel block p % KB (32 channels); lane (lg, ln) takes token
    // 16 tg + ln, channels 32 db + 8 lg .. +7.  Wave 2 also loads the gate
    // and beta of token lane.  Rows past the end are clamped here and zeroed
    // when staged.
    const __bf16 *src = role == 1 ? kg : (role == 2 ? qg : vg);
    const size_t sstr = role == 3 ? tv : tk;
    auto load = [=](int c0) {
        WsRegs r;
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int tg = p / KB, db = p % KB;
            const size_t u = (size_t)min(c0 + 16 * tg + ln, T - 1);
            r.x[p] = *reinterpret_cast<const u32x4 *>(src + u * sstr + 32 * db + 8 * lg);
        }
        r.a = 1.0f;
        r.b = 0.0f;
        if (role == 2) {
            const size_t ua = (size_t)min(c0 + (tid & 63), T - 1);
            r.a = ag[ua * A.H];
            r.b = bg[ua * A.H];
        }
        return r;
    };

    // stage chunk c0 into B: K, Q token-major; V^T through the matrix cores
    // (exact: one product by 1 per output; K^T follows in the next phase);
    // the cumulative log2-gates (padding: gate 1, beta 0)
    auto stage = [&](Buf &B, int c0, const WsRegs &r) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int tg = p / KB, db = p % KB;
            const u32x4 x = keep(r.x[p], c0 + 16 * tg + ln < T);
            const int row = (16 * tg + ln) * SD + 32 * db + 8 * lg;
            if (role == 1) *reinterpret_cast<u32x4 *>(&B.kr[row]) = x;
            if (role == 2) *reinterpret_cast<u32x4 *>(&B.qr[row]) = x;
            if (role == 3) {
                __bf16 *dst = B.vt;
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const floatx4 tx = mma(__builtin_bit_cast(bf16x8, x), eye[h], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                    *reinterpret_cast<bf16x4 *>(&dst[(32 * db + 16 * h + ln) * SC + 16 * tg + 4 * lg]) =
                        bf16x4{(__bf16)tx[0], (__bf16)tx[1], (__bf16)tx[2], (__bf16)tx[3]};
                }
            }
        }
        if (role == 2) {
            const int lane = tid & 63;
            const bool ok = lane < WC && c0 + lane < T;
            const float x = scan64(__builtin_amdgcn_logf(ok ? r.a : 1.0f));
            const float glast =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), WC - 1));
            if (lane < WC) {
                B.g[lane] = x;
                B.eg[lane] = __builtin_amdgcn_exp2f(x);
                B.gam[lane] = __builtin_amdgcn_exp2f(glast - x);
                B.beta[lane] = ok ? r.b : 0.0f;
            }
        }
    };

    // A = strictly lower diag(beta)(K K^T . Gam), stored transposed (fp32),
    // and P = (Q K^T . Gam . [i >= j]) (split), one lower 16x16 tile (I, J)
    // each: wave 0 takes A's three tiles, wave 1 P(0,0) and P(1,0), wave 2
    // P(1,1).  Lane (lg, ln) holds 4 consecutive i of one j for A^T and 4
    // consecutive j of one i for P.
    auto gram_a = [&](Buf &B, int I, int J) {
        floatx4 gk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
            gk = mma(ld8(&B.kr[(16 * I + ln) * SD + 32 * kb + 8 * lg]), ld8(&B.kr[(16 * J + ln) * SD + 32 * kb + 8 * lg]), gk);
        const int i0 = 16 * I + 4 * lg, j = 16 * J + ln;
        const floatx4 gi = *reinterpret_cast<const floatx4 *>(&B.g[i0]);
        const floatx4 bi = *reinterpret_cast<const floatx4 *>(&B.beta[i0]);
        const float gj = B.g[j];
        floatx4 out;
#pragma unroll
        for (int r = 0; r < 4; r++) out[r] = i0 + r > j ? (bi[r] * gk[r]) * __builtin_amdgcn_exp2f(gi[r] - gj) : 0.0f;
        *reinterpret_cast<floatx4 *>(&L.a[j * SF + i0]) = out;
    };
    auto gram_p = [&](Buf &B, int I, int J) {
        floatx4 gq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
            gq = mma(ld8(&B.kr[(16 * J + ln) * SD + 32 * kb + 8 * lg]), ld8(&B.qr[(16 * I + ln) * SD + 32 * kb + 8 * lg]), gq);
        const int i = 16 * I + ln, j0 = 16 * J + 4 * lg;
        const float gi = B.g[i];
        const floatx4 gj = *reinterpret_cast<const floatx4 *>(&B.g[j0]);
        bf16x4 h, l;
#pragma unroll
        for (int r = 0; r < 4; r++) split(i >= j0 + r ? gq[r] * __builtin_amdgcn_exp2f(gi - gj[r]) : 0.0f, h, l, r);
        *reinterpret_cast<bf16x4 *>(&B.ph[i * SC + j0]) = h;
        *reinterpret_cast<bf16x4 *>(&B.pl[i * SC + j0]) = l;
    };

    // T = (I + A)^{-1} and its scaled splits, on wave 0.  invert_diag: the two
    // diagonal blocks by forward substitution (lane = block lg < 2, column ln;
    // y = T e_c - e_c solves y_r = -A_rc - sum_{s<r} A_rs y_s, updated
    // right-looking); invert_merge: T[16:32, 0:16] = -T11 A10 T00 on
    // v_mfma_f32_16x16x4f32; invert_split: T1 = T diag(beta e^g),
    // T2 = T diag(beta) split (T's upper part is 0).
    auto invert_diag = [&]() {
        if (lg < 2) {
            const float *At = &L.a[16 * lg * SF + 16 * lg];  // At[s * SF + r] = A_rs
            // the columns of steps 0-6 are loaded up front, those of steps
            // 7-14 once steps 0-2 have freed their registers
            floatx4 yv[4], col[15][4];
            auto load_cols = [&](int s0, int s1) {
#pragma unroll
                for (int s = s0; s < s1; s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++) col[s][q] = *reinterpret_cast<const floatx4 *>(&At[s * SF + 4 * q]);
            };
            float y[16];
            auto steps = [&](int s0, int s1) {
#pragma unroll
                for (int s = s0; s < s1; s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (4 * q + e > s) y[4 * q + e] = fmaf(-col[s][q][e], y[s], y[4 * q + e]);
            };
#pragma unroll
            for (int q = 0; q < 4; q++) yv[q] = *reinterpret_cast<const floatx4 *>(&At[ln * SF + 4 * q]);
            load_cols(0, 7);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4; q++)
#pragma unroll
                for (int e = 0; e < 4; e++) y[4 * q + e] = -yv[q][e];
            steps(0, 3);
            __builtin_amdgcn_sched_barrier(0);
            load_cols(7, 15);
            __builtin_amdgcn_sched_barrier(0);
            steps(3, 15);
            float *Tb = &L.t[16 * lg * SF + 16 * lg];
#pragma unroll
            for (int r = 0; r < 16; r++) Tb[r * SF + ln] = y[r];
            Tb[ln * SF + ln] = 1.0f;
        }
    };
    auto invert_merge = [&]() {
        {
            floatx4 X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++) X = mma4(L.a[(4 * s + lg) * SF + 16 + ln], L.t[(4 * s + lg) * SF + ln], X);
            floatx4 Y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++) Y = mma4(L.t[(16 + ln) * SF + 16 + 4 * lg + s], X[s], Y);
#pragma unroll
            for (int r = 0; r < 4; r++) L.t[(16 + 4 * lg + r) * SF + ln] = -Y[r];
        }
    };
    auto invert_split = [&](Buf &B) {
        const int lane = tid & 63, i = lane >> 1, j0 = 16 * (lane & 1);
        bf16x8 h1[2], l1[2], h2[2], l2[2];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const floatx4 tq = *reinterpret_cast<const floatx4 *>(&L.t[i * SF + j0 + 4 * q]);
            const floatx4 bq = *reinterpret_cast<const floatx4 *>(&B.beta[j0 + 4 * q]);
            const floatx4 eq = *reinterpret_cast<const floatx4 *>(&B.eg[j0 + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float t = j0 + 4 * q + e <= i ? tq[e] : 0.0f;
                const float t2 = t * bq[e];
                const float t1 = t2 * eq[e];
                split(t1, h1[q / 2], l1[q / 2], 4 * (q % 2) + e);
                split(t2, h2[q / 2], l2[q / 2], 4 * (q % 2) + e);
            }
        }
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
            *reinterpret_cast<bf16x8 *>(&B.t1h[i * SC + j0 + 8 * hf]) = h1[hf];
            *reinterpret_cast<bf16x8 *>(&B.t1l[i * SC + j0 + 8 * hf]) = l1[hf];
            *reinterpret_cast<bf16x8 *>(&B.t2h[i * SC + j0 + 8 * hf]) = h2[hf];
            *reinterpret_cast<bf16x8 *>(&B.t2l[i * SC + j0 + 8 * hf]) = l2[hf];
        }
    };

    // K S and Q S of the next chunk: [et][it], lane (lg, ln) holds rows
    // (tokens) 16 it + 4 lg + r of value column e0 + 16 et + ln
    floatx4 KS[ET][2], QS[ET][2];
    auto state_products = [&](Buf &B) {
        bf16x8 Sh[ET][KB], Sl[ET][KB];  // contraction over key rows, permuted slots
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    split(S[et][2 * kb][r], Sh[et][kb], Sl[et][kb], r);
                    split(S[et][2 * kb + 1][r], Sh[et][kb], Sl[et][kb], 4 + r);
                }
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) {
                KS[et][it] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                QS[et][it] = KS[et][it];
            }
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
            bf16x8 ka[2], qa[2];
#pragma unroll
            for (int it = 0; it < 2; it++) {
                const int row = (16 * it + ln) * SD + 32 * kb + 4 * lg;
                ka[it] = ld_pair(&B.kr[row]);
                qa[it] = ld_pair(&B.qr[row]);
            }
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int et = 0; et < ET; et++) {
                    KS[et][it] = mma(ka[it], Sh[et][kb], KS[et][it]);
                    QS[et][it] = mma(qa[it], Sh[et][kb], QS[et][it]);
                }
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int et = 0; et < ET; et++) {
                    KS[et][it] = mma(ka[it], Sl[et][kb], KS[et][it]);
                    QS[et][it] = mma(qa[it], Sl[et][kb], QS[et][it]);
                }
        }
    };

    // chunk finish on the state group: U' = T2 V - T1 (K S), the outputs
    // diag(e^g) Q S + P U' (stored by each wave for its columns), and the
    // operands of S <- e^{g_C} S + K^T diag(e^{g_C - g}) U' for phase Y
    bf16x8 Ghk[ET], Glk[ET];  // U' scaled by e^{g_C - g_j}, split, held from phase X to Y
    float egck = 0.0f;
    auto finish = [&](Buf &B, int c0) {
        bf16x8 Xh[ET], Xl[ET];  // -(K S) over the chunk's tokens, permuted slots
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                split(-KS[et][0][r], Xh[et], Xl[et], r);
                split(-KS[et][1][r], Xh[et], Xl[et], 4 + r);
            }
        bf16x8 t1h[2], t1l[2], t2h[2], t2l[2], vb[ET];
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int row = (16 * it + ln) * SC + 4 * lg;
            t1h[it] = ld_pair(&B.t1h[row]);
            t1l[it] = ld_pair(&B.t1l[row]);
            t2h[it] = ld_pair(&B.t2h[row]);
            t2l[it] = ld_pair(&B.t2l[row]);
        }
#pragma unroll
        for (int et = 0; et < ET; et++) vb[et] = ld_pair(&B.vt[(e0 + 16 * et + ln) * SC + 4 * lg]);
        floatx4 U[ET][2];
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) U[et][it] = mma(t2h[it], vb[et], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) U[et][it] = mma(t1h[it], Xh[et], U[et][it]);
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) U[et][it] = mma(t2l[it], vb[et], U[et][it]);
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) U[et][it] = mma(t1h[it], Xl[et], U[et][it]);
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++) U[et][it] = mma(t1l[it], Xh[et], U[et][it]);
        floatx4 O[ET][2];
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const floatx4 eg = *reinterpret_cast<const floatx4 *>(&B.eg[16 * it + 4 * lg]);
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) O[et][it][r] = QS[et][it][r] * eg[r];
        }
        // U' as operands over the chunk's tokens, plain and scaled by e^{g_C - g_j}
        bf16x8 Vh[ET], Vl[ET], Gh[ET], Gl[ET];
        {
            const floatx4 ga = *reinterpret_cast<const floatx4 *>(&B.gam[4 * lg]);
            const floatx4 gc = *reinterpret_cast<const floatx4 *>(&B.gam[16 + 4 * lg]);
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    split(U[et][0][r], Vh[et], Vl[et], r);
                    split(U[et][1][r], Vh[et], Vl[et], 4 + r);
                    split(U[et][0][r] * ga[r], Gh[et], Gl[et], r);
                    split(U[et][1][r] * gc[r], Gh[et], Gl[et], 4 + r);
                }
        }
        // O += P U' (P's upper tile is zero)
        {
            bf16x8 phv[2], plv[2];
#pragma unroll
            for (int it = 0; it < 2; it++) {
                const int row = (16 * it + ln) * SC + 4 * lg;
                phv[it] = ld_pair(&B.ph[row]);
                plv[it] = ld_pair(&B.pl[row]);
            }
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int et = 0; et < ET; et++) O[et][it] = mma(phv[it], Vh[et], O[et][it]);
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int et = 0; et < ET; et++) O[et][it] = mma(phv[it], Vl[et], O[et][it]);
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int et = 0; et < ET; et++) O[et][it] = mma(plv[it], Vh[et], O[et][it]);
        }
        // outputs: each wave writes its own columns to LDS and reads them back
        // as 16-byte rows (no other wave touches them, so no barrier)
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int it = 0; it < 2; it++)
#pragma unroll
                for (int r = 0; r < 4; r++) L.out[(16 * it + 4 * lg + r) * SD + e0 + 16 * et + ln] = (__bf16)O[et][it][r];
        wave_lds_sync();
        {
            constexpr int VPT = 2 * ET;  // 16-byte pieces per token row of the wave's columns
            const int lane = tid & 63;
#pragma unroll
            for (int x = lane; x < WC * VPT; x += 64) {
                const int t = x / VPT, col = e0 + 8 * (x % VPT);
                if (c0 + t < T)
                    *reinterpret_cast<u32x4 *>(og + (size_t)(c0 + t) * tv + col) =
                        *reinterpret_cast<const u32x4 *>(&L.out[t * SD + col]);
            }
        }
#pragma unroll
        for (int et = 0; et < ET; et++) {
            Ghk[et] = Gh[et];
            Glk[et] = Gl[et];
        }
        egck = B.eg[WC - 1];
    };
    // the state update of chunk c, in phase Y: its K^T is staged a phase late
    // (from the K tile) and no wave restages it meanwhile; 2^{g_C} was read
    // in phase X, before the gates were restaged
    auto state_update = [&](Buf &B) {
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++) S[et][dt] *= egck;
        bf16x8 ka[DT];
#pragma unroll
        for (int dt = 0; dt < DT; dt++) ka[dt] = ld_pair(&B.kt[(16 * dt + ln) * SC + 4 * lg]);
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int et = 0; et < ET; et++) S[et][dt] = mma(ka[dt], Ghk[et], S[et][dt]);
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int et = 0; et < ET; et++) S[et][dt] = mma(ka[dt], Glk[et], S[et][dt]);
    };
    // K^T of a staged chunk from its token-major K tile (role 1, phase X)
    auto stage_kt = [&](Buf &B) {
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const int tg = p / KB, db = p % KB;
            const bf16x8 x = ld8(&B.kr[(16 * tg + ln) * SD + 32 * db + 8 * lg]);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const floatx4 tx = mma(x, eye[h], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                *reinterpret_cast<bf16x4 *>(&B.kt[(32 * db + 16 * h + ln) * SC + 16 * tg + 4 * lg]) =
                    bf16x4{(__bf16)tx[0], (__bf16)tx[1], (__bf16)tx[2], (__bf16)tx[3]};
            }
        }
    };

    // Wave 0, the staging waves and the state group each run a loop of their
    // own (same trip count, the same two barriers per iteration), so no
    // role's registers are held across another role's code.  Iteration c:
    // chunk c+1 is prepared while chunk c is finished; chunk c+2 is staged
    // into chunk c's buffer once chunk c no longer reads it, from registers
    // loaded an iteration earlier.
    if (cgroup && role == 0) {
        for (int c = -2; c < nch; c++) {
            asm volatile("" : "+v"(lg), "+v"(ln));
            Buf &Bk = L.b[(c + 1) & 1];
            const bool prep = c + 1 >= 0 && c + 1 < nch;
            // ---- phase X: A, T's diagonal blocks and the merge (in-wave)
            if (prep) {
                gram_a(Bk, 0, 0);
                gram_a(Bk, 1, 1);
                gram_a(Bk, 1, 0);
                wave_lds_sync();
                invert_diag();
                wave_lds_sync();
                invert_merge();
            }
            __syncthreads();
            // ---- phase Y: T1, T2
            if (prep) invert_split(Bk);
            __syncthreads();
        }
    } else if (cgroup) {
        WsRegs nx;
        if (nch > 0) nx = load(0);
        for (int c = -2; c < nch; c++) {
            asm volatile("" : "+v"(lg), "+v"(ln));
            Buf &Bk = L.b[(c + 1) & 1];
            Buf &Bs = L.b[c & 1];
            const bool prep = c + 1 >= 0 && c + 1 < nch;
            // ---- phase X
            if (prep) {
                if (role == 1) {
                    gram_p(Bk, 0, 0);
                    gram_p(Bk, 1, 0);
                    stage_kt(Bk);
                } else if (role == 2) {
                    gram_p(Bk, 1, 1);
                }
            }
            __syncthreads();
            // ---- phase Y
            if (c + 2 < nch) {
                stage(Bs, (c + 2) * WC, nx);
                if (c + 3 < nch) nx = load((c + 3) * WC);
            }
            __syncthreads();
        }
    } else {
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    S[et][dt][r] = Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln];
        for (int c = -2; c < nch; c++) {
            asm volatile("" : "+v"(lg), "+v"(ln));
            Buf &Bk = L.b[(c + 1) & 1];
            Buf &Bs = L.b[c & 1];
            // ---- phase X
            if (c >= 0) finish(Bs, c * WC);
            __syncthreads();
            // ---- phase Y
            if (c >= 0) state_update(Bs);
            if (c + 1 >= 0 && c + 1 < nch) state_products(Bk);
            __syncthreads();
        }
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln] = S[et][dt][r];
    }
}

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
        // workgroups per head: the most of 1, 2, 4 that keeps one workgroup per CU
        int dev = 0, ncu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        const unsigned ns = grid * 4u <= (unsigned)ncu ? 4u : grid * 2u <= (unsigned)ncu ? 2u : 1u;
        if (ns == 4)
            hipLaunchKernelGGL((prefill_ws_kernel<128, 4>), dim3(grid * 4), dim3(64 * (4 + WS_SW / 4)), 0, st, A);
        else if (ns == 2)
            hipLaunchKernelGGL((prefill_ws_kernel<128, 2>), dim3(grid * 2), dim3(64 * (4 + WS_SW / 2)), 0, st, A);
        else
            hipLaunchKernelGGL((prefill_ws_kernel<128, 1>), dim3(grid), dim3(64 * (4 + WS_SW)), 0, st, A);
    } else {
        hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(128), 0, st, A);
    }
    return hipGetLastError();
}

}  // namespace gdnq
