// prefill_kda.hip -- chunkwise-parallel prefill of the delta rule with a
// per-key-channel gate (KDA) on the matrix cores (gdn_prefill with
// GDNQ_DECAY_CHANNEL).
//
// The recurrence is the KDA row of Table 3 in "LinQuant: Functional
// Invariances for Low-Precision Linear Recurrences" (appendix), in the
// dk x dv orientation: S_t = diag(a_t) S_{t-1} + k_t u_t^T with
// u_t = b_t (v_t - (diag(a_t) S_{t-1})^T k_t), o_t = S_t^T q_t.  That
// page's abstract notes that chunkwise-parallel prefill turns most of it
// into dense products; the chunk form is the WY/UT form of the delta rule
// (Yang et al., "Parallelizing Linear Transformers with the Delta Rule
// over Sequence Length", 2024) with the scalar decay of its gated variant
// replaced by a diagonal one.  For a chunk of C = 16 tokens, with
// G_tc = sum_{s<=t} log a_sc counted from the chunk start (per key channel
// c), S the state at the chunk start and beta = b:
//     A_ij = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}    (i > j)
//     P_ij = sum_c q_ic k_jc e^{G_ic - G_jc}           (i >= j)
//     T  = (I + A)^{-1},  T1 = T diag(beta)
//     W  = T1 (K . e^G),  U = T1 V,  U' = U - W S      (row i is u_i)
//     O  = (Q . e^G) S + P U'
//     S <- diag(e^{G_C}) S + (K . e^{G_C - G})^T U'
// which is the token recurrence unrolled over the chunk: with
// Gam_t = e^{G_t}, diag(a_t) S_{t-1} = diag(Gam_t) S
// + sum_{j<t} diag(Gam_t / Gam_j) k_j u_j^T, so (I + A) U' =
// diag(beta) V - diag(beta) (K . Gam) S, and S_t^T q_t gives O.  Every
// exponent used is <= 0 (the decays of A and P are taken pair by pair,
// never as a quotient of two chunk-wide factors), so no gate can overflow.
//
// Precision as in the scalar-gate kernel (prefill.hip): bf16 matrix products
// with fp32 accumulation, q, k, v exact in bf16, every fp32 operand split
// into two bf16 parts.  The decayed Gram sums A and P are fp32: as two fp32
// matrix products of the chunk's operands scaled by per-token factors
// around a reference token, or, in a chunk where some channel decays by
// more than 2^-60, pair by pair on the VALU (one e^{G_ic - G_jc} per pair
// and channel).  U and W by forward substitution in fp32.
//
// Mapping (prefill_kda_kernel, used for D = 64; D = 128 takes the two-group
// form at the end of this file): one workgroup per (batch, head) of D/16
// waves (two per SIMD: the chunk-local phases are latency-bound, and a
// second wave on each SIMD hides part of it); wave w owns value columns 16w..16w+15 of the state,
// kept in fp32 MFMA accumulators for the whole sequence (the layout and the
// permuted contraction of the scalar-gate kernel).  Products over the
// chunk's 16 tokens use v_mfma_f32_16x16x16_bf16, whose accumulator layout
// is its own B operand layout: U' feeds P U' and the state update straight
// from registers.  No accumulator chain mixes instruction shapes: the
// compiler inserts no wait between a product and one of another shape that
// reads it as its accumulator.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int KC = 16;                    // tokens per chunk
constexpr int NPAIR = KC * (KC + 1) / 2;  // pairs i >= j
constexpr int SA = KC + 4;                // fp32 stride of the A^T tile

__device__ __forceinline__ floatx4 mma32(bf16x8 a, bf16x8 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma16(bf16x4 a, bf16x4 b, floatx4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a), __builtin_bit_cast(short4v, b),
                                                     c, 0, 0, 0);
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
__device__ __forceinline__ bf16x4 ld4(const __bf16 *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ floatx4 ldf4(const float *p) { return *reinterpret_cast<const floatx4 *>(p); }

// One thread's share of a chunk's inputs, held in registers while the
// previous chunk is computed: one 8-byte piece of each of K and Q (token
// x / (D/4), channels 4 (x % (D/4)) .. +3) and of V (token x % KC, channels
// 4 (x / KC) .. +3), and for the last D threads (c = x - (threads - D)) the
// 16 gates of key channel c and, for c < KC, b of token c.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
struct KdaChunkRegs {
    u32x2 k, q, v;
    float a[KC];
    float b;
};

template <int CTRL>
__device__ __forceinline__ float dppf(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of N = 8 or 16 lanes, every lane of a group gets
// it: xor-1 and xor-2 (quad_perm), then row_half_mirror (xor-4 once the
// quads hold equal values) and, for 16, row_mirror.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
    x += dppf<0xB1>(x);
    x += dppf<0x4E>(x);
    x += dppf<0x141>(x);
    if constexpr (N == 16) x += dppf<0x140>(x);
    return x;
}

// pair index p = i (i + 1) / 2 + j (j <= i) -> i
__device__ __forceinline__ int pair_row(int p)
{
    int i = (int)((sqrtf(8.0f * (float)p + 1.0f) - 1.0f) * 0.5f);
    if (i * (i + 1) / 2 > p) i--;
    if ((i + 1) * (i + 2) / 2 <= p) i++;
    return i;
}

}  // namespace

template <int D>
struct KdaLds {
    static constexpr int SD = D + 8;   // bf16 stride of token-major [KC][D] tiles (16-byte pad)
    static constexpr int SG = D + 4;   // fp32 stride of the gate tile
    static constexpr int ST = KC + 8;  // bf16 stride of channel-major [D][KC] and of [KC][KC] tiles
    static constexpr int SK = KC + 4;  // fp32 stride of channel-major [D][KC] tiles
    __bf16 kr[KC * SD];                // K, token-major
    __bf16 ob[KC * SD];                // the chunk's outputs, token-major
    __bf16 qr[KC * SD];                // Q, token-major
    float g[KC * SG];                  // G in base 2: cumulative log2 gates from the chunk start
    __bf16 vt[D * ST];                 // V^T
    __bf16 qgh[KC * SD], qgl[KC * SD];  // Q . 2^G, split, token-major
    float kgf[D * SK];                  // (K . 2^G)^T
    __bf16 kch[D * ST], kcl[D * ST];    // (K . 2^(G_C - G))^T, split
    __bf16 wh[KC * SD], wl[KC * SD];    // -W, split, token-major
    float uf[KC * SG];                  // U = T1 V, token-major
    __bf16 ph[KC * ST], pl[KC * ST];    // P, split (upper part zero)
    float xf[KC * SG];                  // K . 2^(G - G_m), token-major (m: the chunk's reference token)
    float yf[KC * SG];                  // K . 2^(G_m - G), token-major
    float zf[KC * SG];                  // Q . 2^(G - G_m), token-major
    float gp[2][KC * SA];               // second halves of A and P^T (factored Gram sums)
    float egc[D];                       // 2^(G_C): the chunk's decay of each key row of S
    float at[KC * SA];                  // A^T: at[j * SA + i] = A_ij (i > j), zero elsewhere
    float beta[KC];
    uint8_t pij[NPAIR];                 // pair p -> i | j << 4
    int pairwise;                       // c0 + 1 when chunk c0 takes the pairwise Gram sums
};

// The decayed Gram sums of a chunk factor through its reference token m:
// 2^(G_i - G_j) = 2^(G_i - G_m) 2^(G_m - G_j), which makes A and P two dense
// products.  Every factor lies in [2^-R, 2^R] when no channel decays by more
// than 2^-R over the chunk (|G_i - G_m| <= -G_C), so with R = 60 no factor
// or product leaves fp32's normal range.  A chunk that decays
// further in some channel takes the pairwise sums, whose exponents are all
// <= 0.
constexpr float kFactorRange = 60.0f;
constexpr int kRefToken = KC / 2 - 1;

struct PrefillKdaArgs {
    float *S;
    const __bf16 *q, *k, *v;
    const float *a, *b;
    __bf16 *o;
    int T, H, HK;
    Divisor byH, byG;
};

// threads per workgroup: D/16 waves
template <int D>
constexpr int kda_threads() { return D / 16 * 64; }

template <int D>
__global__ __launch_bounds__(kda_threads<D>(), 1) void prefill_kda_kernel(PrefillKdaArgs A)
{
    using Lds = KdaLds<D>;
    constexpr int SD = Lds::SD, SG = Lds::SG, ST = Lds::ST, SK = Lds::SK;
    constexpr int ET = 1;                     // 16-column tiles of the state per wave
    constexpr int CW = 16 * ET;               // value columns (and key channels of W) per wave
    constexpr int NW = D / CW, NT = NW * 64;  // waves; wave w owns columns and channels CW w .. CW w + CW - 1
    static_assert(NT == kda_threads<D>(), "block size");
    constexpr int KB = D / 32;                // 32-wide blocks along a head dim
    constexpr int DT = D / 16;                // 16-row tiles along a head dim
    __shared__ Lds L;

    const int tid0 = (int)__builtin_amdgcn_workitem_id_x(), tid = tid0;
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
    const float *ag = A.a + (size_t)bb * T * tv + (size_t)hh * D;  // a: [B, T, H, D]
    const float *bg = A.b + (size_t)bb * T * A.H + hh;
    float *Sg = A.S + (size_t)bh * D * D;
    const int e0 = CW * wave;  // value columns e0 + 16 et + ln, et < ET
    int lg = (tid & 63) >> 4, ln = tid & 15;

    // Entries never written by the chunk loop (P's upper part, A^T's
    // diagonal and upper part) are cleared once.
    for (int x = tid; x < KC * ST; x += NT) {
        L.ph[x] = (__bf16)0.0f;
        L.pl[x] = (__bf16)0.0f;
    }
    for (int x = tid; x < KC * SA; x += NT) L.at[x] = 0.0f;
    if (tid == 0) L.pairwise = 0;
    for (int p = tid; p < NPAIR; p += NT) {
        const int i = pair_row(p);
        L.pij[p] = (uint8_t)(i | (p - i * (i + 1) / 2) << 4);
    }
    // The first chunk's staging may flag it for the pairwise sums: that
    // write must follow the clear above.
    __syncthreads();

    // Chunk loads: every load is unconditional (tokens past the end are
    // clamped to the last one) and zeroed only when staged, so the compiler
    // counts them and waits for them at staging alone.
    // K, Q, V go out first; the gates and beta later in the chunk, so that
    // their registers are not held through the Gram sums.
    // The gates go to the last D threads, whose waves wait idle while the
    // first wave solves for T.
    auto load_kqv = [=](int c0, int tid, KdaChunkRegs &r) {
        const int t = tid / (D / 4), c = 4 * (tid % (D / 4));
        const size_t u = (size_t)min(c0 + t, T - 1);
        r.k = *reinterpret_cast<const u32x2 *>(kg + u * tk + c);
        r.q = *reinterpret_cast<const u32x2 *>(qg + u * tk + c);
        const int tv_ = tid % KC, cv = 4 * (tid / KC);
        r.v = *reinterpret_cast<const u32x2 *>(vg + (size_t)min(c0 + tv_, T - 1) * tv + cv);
    };
    auto load_ab = [=](int c0, int tid, KdaChunkRegs &r) {
        const int c = tid - (NT - D);
        if (c >= 0) {
#pragma unroll
            for (int t = 0; t < KC; t++) r.a[t] = ag[(size_t)min(c0 + t, T - 1) * tv + c];
            r.b = bg[(size_t)min(c0 + (c & (KC - 1)), T - 1) * A.H];
        }
    };
    static_assert(KC * D / 4 == NT, "one 8-byte piece of K, Q and V per thread");

    // Staging of the chunk at cs from the registers: K, Q token-major and V^T
    // (tokens past the end are zero), the gates (the last D threads, one key
    // channel each: cumulative log2-gates from the chunk start, padding gate
    // 1; a channel that decays by more than 2^-60 over the chunk flags it)
    // and beta.  A chunk is staged while the previous one finishes its state
    // products: by then no phase reads these tiles.
    auto stage = [&](int cs, int tid, const KdaChunkRegs &r) {
        const int nv = min(KC, T - cs);
        {
            const int t = tid / (D / 4), c = 4 * (tid % (D / 4));
            const bool ok = t < nv;
            const u32x2 z = {0u, 0u};
            *reinterpret_cast<u32x2 *>(&L.kr[t * SD + c]) = ok ? r.k : z;
            *reinterpret_cast<u32x2 *>(&L.qr[t * SD + c]) = ok ? r.q : z;
            const int tv_ = tid % KC, cv = 4 * (tid / KC);
            const bf16x4 vv = __builtin_bit_cast(bf16x4, tv_ < nv ? r.v : z);
#pragma unroll
            for (int e = 0; e < 4; e++) L.vt[(cv + e) * ST + tv_] = vv[e];
        }
        if (const int c = tid - (NT - D); c >= 0) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < KC; t++) {
                acc += t < nv ? __builtin_amdgcn_logf(r.a[t]) : 0.0f;
                L.g[t * SG + c] = acc;
            }
            if (!(acc >= -kFactorRange)) L.pairwise = cs + 1;  // every thread that writes, writes the same
            if (c < KC) L.beta[c] = c < nv ? r.b : 0.0f;
        }
    };

    // S[et][dt][r] = S[16 dt + 4 lg + r][e0 + 16 et + ln] (MFMA accumulator layout)
    floatx4 S[ET][DT];
#pragma unroll
    for (int et = 0; et < ET; et++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                S[et][dt][r] = Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln];

    KdaChunkRegs nx;
    load_kqv(0, tid, nx);
    load_ab(0, tid, nx);
    stage(0, tid, nx);
    __syncthreads();
    for (int c0 = 0; c0 < T; c0 += KC) {
        // Lane indices pass through an empty asm each chunk, so the LDS
        // addresses built from them are formed inside the loop instead of
        // being hoisted out and held in registers across it.
        int tid = tid0;
        asm volatile("" : "+v"(lg), "+v"(ln), "+v"(tid));

        const int nv = min(KC, T - c0);  // valid tokens of this chunk
        const bool more = c0 + KC < T;
        if (more) load_kqv(c0 + KC, tid, nx);  // in flight while this chunk is computed

        // ---- element-wise operands: Q . 2^G (token-major, split), (K . 2^G)^T
        // (fp32) and (K . 2^(G_C - G))^T (split, both channel-major); every
        // exponent <= 0.  Thread c, 4 tokens of key channel c (one store per
        // channel-major tile and thread); threads c < D also keep the chunk decay
        // 2^(G_C) of key row c of S.  In a factored chunk every exponent lies
        // within [-60, 60], and the factors are products of 2^(+-G_t) with the
        // channel's 2^(+-G_m) and 2^(G_C).
        const bool factored = __builtin_amdgcn_readfirstlane(L.pairwise) != c0 + 1;
        {
            constexpr int TPT = KC * D / NT;
            static_assert(TPT == 4, "one thread takes 4 tokens of one channel");
            const int c = tid % D, t0 = TPT * (tid / D);
            const float gC = L.g[(KC - 1) * SG + c], gm = L.g[kRefToken * SG + c];
            const float egC = __builtin_amdgcn_exp2f(gC);
            const float egm = __builtin_amdgcn_exp2f(gm), emg = __builtin_amdgcn_exp2f(-gm);
            if (tid < D) L.egc[c] = egC;
            floatx4 kgv;
            bf16x4 ch, cl;
#pragma unroll
            for (int e = 0; e < TPT; e++) {
                const int t = t0 + e;
                const float gv = L.g[t * SG + c];
                const float kv = (float)L.kr[t * SD + c], qv = (float)L.qr[t * SD + c];
                const float e1 = __builtin_amdgcn_exp2f(gv);
                const float ei = factored ? __builtin_amdgcn_exp2f(-gv) : 0.0f;
                const float e2 = factored ? egC * ei : __builtin_amdgcn_exp2f(gC - gv);
                kgv[e] = kv * e1;
                split(kv * e2, ch, cl, e);
                const float qe = qv * e1;
                const __bf16 qh = (__bf16)qe;
                L.qgh[t * SD + c] = qh;
                L.qgl[t * SD + c] = (__bf16)(qe - (float)qh);
                if (factored) {
                    const float fl = e1 * emg, fr = egm * ei;
                    L.xf[t * SG + c] = kv * fl;
                    L.yf[t * SG + c] = kv * fr;
                    L.zf[t * SG + c] = qv * fl;
                }
            }
            *reinterpret_cast<floatx4 *>(&L.kgf[c * SK + t0]) = kgv;
            *reinterpret_cast<bf16x4 *>(&L.kch[c * ST + t0]) = ch;
            *reinterpret_cast<bf16x4 *>(&L.kcl[c * ST + t0]) = cl;
        }
        // ---- the decayed Gram sums, factored: waves 0 and 1 form A = X Y^T and
        // waves 2 and 3 P^T = Y Z^T (X = K . 2^(G - G_m), Y = K . 2^(G_m - G),
        // Z = Q . 2^(G - G_m)) with fp32 matrix products, each wave over half
        // of the key channels and lane group lg over D/8 of them, one per
        // instruction; the second half goes through LDS and is added to the
        // first (in that order, so the sums are reproducible).  Lane (lg, ln) then
        // holds rows 4 lg .. 4 lg + 3 of column ln: A_ij with i = 4 lg + r,
        // j = ln, which is A^T's row j, and P_ij with i = ln, j = 4 lg + r,
        // which is P's row i.
        if (factored) {
            __syncthreads();  // X, Y, Z staged
            const bool isp = wave >= 2, first = (wave & 1) == 0;  // wave-uniform
            floatx4 m = {0.0f, 0.0f, 0.0f, 0.0f};
            if (wave < 4) {
                constexpr int CPG = D / 8;  // channels per lane group and half
                const int cb = (wave & 1) * (D / 2) + CPG * lg;
                const float *xa = (isp ? L.yf : L.xf) + ln * SG + cb;
                const float *yb = (isp ? L.zf : L.yf) + ln * SG + cb;
                floatx4 m0 = {0.0f, 0.0f, 0.0f, 0.0f}, m1 = m0;
#pragma unroll
                for (int s4 = 0; s4 < CPG; s4 += 4) {
                    const floatx4 xv = ldf4(xa + s4), yv = ldf4(yb + s4);
                    m0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[0], yv[0], m0, 0, 0, 0);
                    m1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[1], yv[1], m1, 0, 0, 0);
                    m0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[2], yv[2], m0, 0, 0, 0);
                    m1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[3], yv[3], m1, 0, 0, 0);
                }
                m = m0 + m1;
                if (!first) *reinterpret_cast<floatx4 *>(&L.gp[isp][ln * SA + 4 * lg]) = m;
            }
            __syncthreads();  // second halves staged
            if (wave < 4 && first) {
                m += ldf4(&L.gp[isp][ln * SA + 4 * lg]);
                if (!isp) {
                    const floatx4 bi = ldf4(&L.beta[4 * lg]);
                    floatx4 w;
#pragma unroll
                    for (int r = 0; r < 4; r++) w[r] = 4 * lg + r > ln ? bi[r] * m[r] : 0.0f;
                    *reinterpret_cast<floatx4 *>(&L.at[ln * SA + 4 * lg]) = w;
                } else {
                    bf16x4 h, l;
#pragma unroll
                    for (int r = 0; r < 4; r++) split(ln >= 4 * lg + r ? m[r] : 0.0f, h, l, r);
                    *reinterpret_cast<bf16x4 *>(&L.ph[ln * ST + 4 * lg]) = h;
                    *reinterpret_cast<bf16x4 *>(&L.pl[ln * ST + 4 * lg]) = l;
                }
            }
        } else
        // ---- the decayed Gram sums, pairwise: D/8 lanes per pair (i, j), 8 key channels
        // each, summed across the pair's lanes by DPP (all lanes take part: a
        // slot past the last pair recomputes that pair and writes nothing);
        // the pair's first lane stores A^T (with beta) and P (split).  Every
        // pass's LDS reads go out first.
        {
            constexpr int LPP = D / 8, PPI = NT / LPP;  // lanes per pair, pairs per pass
            constexpr int NP = (NPAIR + PPI - 1) / PPI;  // passes
            const int cb = tid % LPP, slot = tid / LPP, c = 8 * cb;
            int pi[NP], pj[NP];
            bf16x8 kiv[NP], qiv[NP], kjv[NP];
            floatx4 gi0[NP], gi1[NP], gj0[NP], gj1[NP];
#pragma unroll
            for (int n = 0; n < NP; n++) {
                const int ij = L.pij[min(n * PPI + slot, NPAIR - 1)];
                pi[n] = ij & 15;
                pj[n] = ij >> 4;
            }
#pragma unroll
            for (int n = 0; n < NP; n++) {
                kiv[n] = ld8(&L.kr[pi[n] * SD + c]);
                qiv[n] = ld8(&L.qr[pi[n] * SD + c]);
                kjv[n] = ld8(&L.kr[pj[n] * SD + c]);
                gi0[n] = ldf4(&L.g[pi[n] * SG + c]);
                gi1[n] = ldf4(&L.g[pi[n] * SG + c + 4]);
                gj0[n] = ldf4(&L.g[pj[n] * SG + c]);
                gj1[n] = ldf4(&L.g[pj[n] * SG + c + 4]);
            }
#pragma unroll
            for (int n = 0; n < NP; n++) {
                const int i = pi[n], j = pj[n];
                float sa = 0.0f, sp = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float gi = e < 4 ? gi0[n][e] : gi1[n][e - 4], gj = e < 4 ? gj0[n][e] : gj1[n][e - 4];
                    const float t = (float)kjv[n][e] * __builtin_amdgcn_exp2f(gi - gj);
                    sa = fmaf((float)kiv[n][e], t, sa);
                    sp = fmaf((float)qiv[n][e], t, sp);
                }
                sa = group_sum<LPP>(sa);
                sp = group_sum<LPP>(sp);
                if (cb == 0 && n * PPI + slot < NPAIR) {
                    if (j < i) L.at[j * SA + i] = L.beta[i] * sa;
                    const __bf16 h = (__bf16)sp;
                    L.ph[i * ST + j] = h;
                    L.pl[i * ST + j] = (__bf16)(sp - (float)h);
                }
            }
        }
        __syncthreads();
        if (more) load_ab(c0 + KC, tid, nx);

        // ---- U = T1 V and W = T1 (K . 2^G), T1 = (I + A)^{-1} diag(beta), by
        // forward substitution on their columns, (I + A) Y = diag(beta) R: one
        // lane per value column (R = V) and one per key channel (R = K . 2^G),
        // updated right-looking with A's columns read as rows of A^T.  U goes
        // to LDS in fp32, -W split, both token-major.
        if (tid < 2 * D) {
            const bool isw = tid >= D;  // wave-uniform
            const int c = isw ? tid - D : tid;
            float y[KC];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const floatx4 bq = ldf4(&L.beta[4 * q]);
                if (isw) {
                    const floatx4 rq = ldf4(&L.kgf[c * SK + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; e++) y[4 * q + e] = bq[e] * rq[e];
                } else {
                    const bf16x4 rq = ld4(&L.vt[c * ST + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; e++) y[4 * q + e] = bq[e] * (float)rq[e];
                }
            }
            // the loads of each half of the steps go out together (broadcast
            // reads): issued step by step, the 15 steps would wait on 15 LDS
            // round trips, and all at once they would not fit in registers
#pragma unroll
            for (int h = 0; h < 2; h++) {
                constexpr int HS = KC / 2;  // steps per half
                floatx4 col[HS][4];
#pragma unroll
                for (int s = h * HS; s < min(KC - 1, (h + 1) * HS); s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++) col[s - h * HS][q] = ldf4(&L.at[s * SA + 4 * q]);  // A_{4q+e, s}
#pragma unroll
                for (int s = h * HS; s < min(KC - 1, (h + 1) * HS); s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (4 * q + e > s) y[4 * q + e] = fmaf(-col[s - h * HS][q][e], y[s], y[4 * q + e]);
            }
            if (isw) {
#pragma unroll
                for (int t = 0; t < KC; t++) {
                    const float w = -y[t];
                    const __bf16 h = (__bf16)w;
                    L.wh[t * SD + c] = h;
                    L.wl[t * SD + c] = (__bf16)(w - (float)h);
                }
            } else {
#pragma unroll
                for (int t = 0; t < KC; t++) L.uf[t * SG + c] = y[t];
            }
        }
        __syncthreads();  // U and -W complete
        floatx4 U[ET];  // U[et][r] = U[4 lg + r][e0 + 16 et + ln]
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int r = 0; r < 4; r++) U[et][r] = L.uf[(4 * lg + r) * SG + e0 + 16 * et + ln];

        // ---- state operand (contraction over key rows, permuted slots)
        bf16x8 Sh[ET][KB], Sl[ET][KB];
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int kb = 0; kb < KB; kb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    split(S[et][2 * kb][r], Sh[et][kb], Sl[et][kb], r);
                    split(S[et][2 * kb + 1][r], Sh[et][kb], Sl[et][kb], 4 + r);
                }
        // ---- U' = U - W S and O = (Q . 2^G) S
        floatx4 O[ET];
#pragma unroll
        for (int et = 0; et < ET; et++) O[et] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; kb++) {
            const int row = ln * SD + 4 * lg + 32 * kb;
            const bf16x8 wh = ld_pair(&L.wh[row]), wl = ld_pair(&L.wl[row]);
            const bf16x8 qh = ld_pair(&L.qgh[row]), ql = ld_pair(&L.qgl[row]);
#pragma unroll
            for (int et = 0; et < ET; et++) {
                U[et] = mma32(wh, Sh[et][kb], U[et]);
                O[et] = mma32(qh, Sh[et][kb], O[et]);
            }
#pragma unroll
            for (int et = 0; et < ET; et++) {
                U[et] = mma32(wh, Sl[et][kb], U[et]);
                O[et] = mma32(qh, Sl[et][kb], O[et]);
            }
#pragma unroll
            for (int et = 0; et < ET; et++) {
                U[et] = mma32(wl, Sh[et][kb], U[et]);
                O[et] = mma32(ql, Sh[et][kb], O[et]);
            }
        }
        // the next chunk's staging and the decay of S (whose split parts the
        // products read) fill the time these products take
        if (more) stage(c0 + KC, tid, nx);
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const floatx4 ec = ldf4(&L.egc[16 * dt + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; r++)
#pragma unroll
                for (int et = 0; et < ET; et++) S[et][dt][r] *= ec[r];
        }
        // ---- U' as the B operand over tokens (its accumulator layout), split
        bf16x4 Vh[ET], Vl[ET];
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int r = 0; r < 4; r++) split(U[et][r], Vh[et], Vl[et], r);
        // ---- O += P U' (its own accumulator, added on the VALU: a product
        // that reads as its accumulator the result of a product of another
        // shape, here 16x16x32 before 16x16x16, gets no wait from the
        // compiler and may read it before it is complete); outputs staged
        // token-major in their own tile
        {
            const bf16x4 pah = ld4(&L.ph[ln * ST + 4 * lg]), pal = ld4(&L.pl[ln * ST + 4 * lg]);
#pragma unroll
            for (int et = 0; et < ET; et++) {
                floatx4 pu = mma16(pah, Vh[et], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                pu = mma16(pah, Vl[et], pu);
                pu = mma16(pal, Vh[et], pu);
                O[et] += pu;
            }
        }
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int r = 0; r < 4; r++) L.ob[(4 * lg + r) * SD + e0 + 16 * et + ln] = (__bf16)O[et][r];
        // ---- S <- diag(2^{G_C}) S + (K . 2^(G_C - G))^T U' (S already decayed)
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            const bf16x4 kah = ld4(&L.kch[(16 * dt + ln) * ST + 4 * lg]);
            const bf16x4 kal = ld4(&L.kcl[(16 * dt + ln) * ST + 4 * lg]);
#pragma unroll
            for (int et = 0; et < ET; et++) {
                S[et][dt] = mma16(kah, Vh[et], S[et][dt]);
                S[et][dt] = mma16(kah, Vl[et], S[et][dt]);
                S[et][dt] = mma16(kal, Vh[et], S[et][dt]);
            }
        }
        __syncthreads();  // the outputs and the next chunk are staged
        for (int x = tid; x < KC * D / 8; x += NT) {
            const int t = x / (D / 8), c = 8 * (x % (D / 8));
            if (t < nv)
                *reinterpret_cast<u32x4 *>(og + (size_t)(c0 + t) * tv + c) =
                    *reinterpret_cast<const u32x4 *>(&L.ob[t * SD + c]);
        }
    }

#pragma unroll
    for (int et = 0; et < ET; et++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln] = S[et][dt][r];
}

// ---------------------------------------------------------------------------
// Two-group form for D = 128 (twelve waves, one workgroup per head; with
// fewer heads than CUs, NS = 2 or 4 workgroups per head, see the kernel):
// waves 0-3 (the chunk group) run the chunk-local phases of chunk c + 1 --
// element-wise operands, the decayed Gram sums, U and W by substitution --
// while waves 4 and up (the state group, 16 value columns each, two per
// SIMD at NS = 1) run the state phases of chunk c: U' = U - W S and
// O = (Q . 2^G) S, the outputs, the state update.  The chunk-local phases do not read S, so the
// two chains overlap on the SIMDs.  One iteration, four barriers:
//   1. chunk group: element-wise operands       state group: U', O products
//   2. chunk group: Gram products (factored)    state group: -
//   3. chunk group: Gram halves added           state group: P U', outputs
//   4. chunk group: substitution for U and W    state group: state update,
//                                               output stores, staging
// (a chunk that takes the pairwise Gram sums merges phases 2 and 3).  What
// the chunk group hands to the state group (Q . 2^G, K . 2^(G_C - G),
// 2^(G_C), P, U, -W) is double-buffered by chunk parity.  The state group
// loads and stages the raw inputs: those of chunk c + 2 go out at the start
// of the iteration; K, Q and the gates are staged in phase 4 (chunk c + 1
// reads them no more), V^T and beta at the start of the next iteration.
// The arithmetic of every phase is that of prefill_kda_kernel.
template <int D>
struct KdaWsLds {
    static constexpr int SD = D + 8, SG = D + 4, ST = KC + 8, SK = KC + 4;
    // raw chunk inputs (staging writes, the chunk group reads)
    alignas(16) __bf16 kr[KC * SD];
    alignas(16) __bf16 qr[KC * SD];
    alignas(16) float g[KC * SG];
    alignas(16) __bf16 vt[D * ST];
    alignas(16) float beta[KC];
    // chunk-group scratch
    alignas(16) float kgf[D * SK];
    alignas(16) float xf[KC * SG];
    alignas(16) float yf[KC * SG];
    alignas(16) float zf[KC * SG];
    alignas(16) float gp[2][KC * SA];
    alignas(16) float at[KC * SA];
    // chunk group -> state group, by chunk parity
    alignas(16) __bf16 qgh[2][KC * SD];
    alignas(16) __bf16 qgl[2][KC * SD];
    alignas(16) __bf16 kch[2][D * ST];
    alignas(16) __bf16 kcl[2][D * ST];
    alignas(16) __bf16 wh[2][KC * SD];
    alignas(16) __bf16 wl[2][KC * SD];
    alignas(16) float uf[2][KC * SG];
    alignas(16) __bf16 ph[2][KC * ST];
    alignas(16) __bf16 pl[2][KC * ST];
    alignas(16) float egc[2][D];
    // the state group's outputs, token-major
    alignas(16) __bf16 ob[KC * SD];
    uint8_t pij[NPAIR];
    int pairwise;
};

// One staging thread's share of a chunk: PPT 8-byte pieces of each of K, Q
// and V, and for the last D threads the gates of one key channel and, for
// channel c < KC, b of token c.
template <int PPT>
struct KdaWsRegs {
    u32x2 k[PPT], q[PPT], v[PPT];
    float a[KC];
    float b;
};

// threads per workgroup: the chunk group's 4 waves and 8 / NS state waves
template <int NS>
constexpr int kda_ws_threads() { return 64 * (4 + 8 / NS); }

// NS workgroups share a head (NS = 1, 2, 4) when a call has fewer heads than
// CUs: each prepares every chunk in full and finishes D / NS of the head's
// value columns.
template <int D, int NS>
__global__ __launch_bounds__(kda_ws_threads<NS>(), 1) void prefill_kda_ws_kernel(PrefillKdaArgs A)
{
    static_assert(D == 128, "two groups of four waves: D = 128");
    using Lds = KdaWsLds<D>;
    constexpr int SD = Lds::SD, SG = Lds::SG, ST = Lds::ST, SK = Lds::SK;
    constexpr int NT = kda_ws_threads<NS>(), GT = 256;  // threads, threads of the chunk group
    constexpr int ST_T = NT - GT;             // threads of the state group (they also stage)
    constexpr int PPT = KC * D / 4 / ST_T;    // 8-byte pieces of each of K, Q, V per staging thread
    static_assert(PPT * ST_T == KC * D / 4 && ST_T >= D, "the state group stages whole chunks");
    constexpr int ET = 1;                     // 16-column tiles of the state per state wave
    constexpr int KB = D / 32;                // 32-wide blocks along a head dim
    constexpr int DT = D / 16;                // 16-row tiles along a head dim
    __shared__ Lds L;

    const int tid0 = (int)__builtin_amdgcn_workitem_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const bool chunk_group = wave < 4;        // wave-uniform
    const unsigned gid = __builtin_amdgcn_workgroup_id_x();
    const unsigned bh = gid / NS;             // the head
    const int part = (int)(gid % NS);         // its share of the value columns
    const unsigned bb = div_by(bh, A.byH), hh = bh - bb * (unsigned)A.H;
    const unsigned kh = div_by(hh, A.byG);
    const int T = A.T;
    const int nch = (T + KC - 1) / KC;
    const size_t tk = (size_t)A.HK * D, tv = (size_t)A.H * D;
    const __bf16 *qg = A.q + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *kg = A.k + (size_t)bb * T * tk + (size_t)kh * D;
    const __bf16 *vg = A.v + (size_t)bb * T * tv + (size_t)hh * D;
    __bf16 *og = A.o + (size_t)bb * T * tv + (size_t)hh * D;
    const float *ag = A.a + (size_t)bb * T * tv + (size_t)hh * D;
    const float *bg = A.b + (size_t)bb * T * A.H + hh;
    float *Sg = A.S + (size_t)bh * D * D;
    const int e0 = part * (D / NS) + 16 * (wave - 4);  // state group: value columns e0 + 16 et + ln
    int lg = (tid0 & 63) >> 4, ln = tid0 & 15;

    for (int x = tid0; x < 2 * KC * ST; x += NT) {
        (&L.ph[0][0])[x] = (__bf16)0.0f;
        (&L.pl[0][0])[x] = (__bf16)0.0f;
    }
    for (int x = tid0; x < KC * SA; x += NT) L.at[x] = 0.0f;
    if (tid0 == 0) L.pairwise = 0;
    for (int p = tid0; p < NPAIR; p += NT) {
        const int i = pair_row(p);
        L.pij[p] = (uint8_t)(i | (p - i * (i + 1) / 2) << 4);
    }
    __syncthreads();  // the first chunk's staging may set the flag

    auto load_chunk = [=](int c0, int tid, KdaWsRegs<PPT> &r) {
#pragma unroll
        for (int p = 0; p < PPT; p++) {
            const int x = tid + p * ST_T;
            const int t = x / (D / 4), c = 4 * (x % (D / 4));
            const size_t u = (size_t)min(c0 + t, T - 1);
            r.k[p] = *reinterpret_cast<const u32x2 *>(kg + u * tk + c);
            r.q[p] = *reinterpret_cast<const u32x2 *>(qg + u * tk + c);
            const int tv_ = x % KC, cv = 4 * (x / KC);
            r.v[p] = *reinterpret_cast<const u32x2 *>(vg + (size_t)min(c0 + tv_, T - 1) * tv + cv);
        }
        const int cg = tid - (ST_T - D);
        if (cg >= 0) {
#pragma unroll
            for (int t2 = 0; t2 < KC; t2++) r.a[t2] = ag[(size_t)min(c0 + t2, T - 1) * tv + cg];
            r.b = bg[(size_t)min(c0 + (cg & (KC - 1)), T - 1) * A.H];
        }
    };
    // K, Q (token-major, zero past the end) and the gates: cumulative
    // log2-gates from the chunk start (padding gate 1), the pairwise flag
    auto stage_kqg = [&](int cs, int tid, const KdaWsRegs<PPT> &r) {
        const int nv = min(KC, T - cs);
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int p = 0; p < PPT; p++) {
            const int x = tid + p * ST_T;
            const int t = x / (D / 4), c = 4 * (x % (D / 4));
            *reinterpret_cast<u32x2 *>(&L.kr[t * SD + c]) = t < nv ? r.k[p] : z;
            *reinterpret_cast<u32x2 *>(&L.qr[t * SD + c]) = t < nv ? r.q[p] : z;
        }
        if (const int cg = tid - (ST_T - D); cg >= 0) {
            float acc = 0.0f;
#pragma unroll
            for (int t2 = 0; t2 < KC; t2++) {
                acc += t2 < nv ? __builtin_amdgcn_logf(r.a[t2]) : 0.0f;
                L.g[t2 * SG + cg] = acc;
            }
            if (!(acc >= -kFactorRange)) L.pairwise = cs + 1;
        }
    };
    // V^T (zero past the end) and beta
    auto stage_vb = [&](int cs, int tid, const KdaWsRegs<PPT> &r) {
        const int nv = min(KC, T - cs);
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int p = 0; p < PPT; p++) {
            const int x = tid + p * ST_T;
            const int tv_ = x % KC, cv = 4 * (x / KC);
            const bf16x4 vv = __builtin_bit_cast(bf16x4, tv_ < nv ? r.v[p] : z);
#pragma unroll
            for (int e = 0; e < 4; e++) L.vt[(cv + e) * ST + tv_] = vv[e];
        }
        if (const int cg = tid - (ST_T - D); cg >= 0 && cg < KC) L.beta[cg] = cg < nv ? r.b : 0.0f;
    };

    floatx4 S[ET][DT];  // state group: S[et][dt][r] = S[16 dt + 4 lg + r][e0 + 16 et + ln]
    if (!chunk_group) {
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    S[et][dt][r] = Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln];
    }
    KdaWsRegs<PPT> nx;
    if (!chunk_group) {
        load_chunk(0, tid0 - GT, nx);
        stage_kqg(0, tid0 - GT, nx);
    }
    __syncthreads();

    for (int c = -1; c < nch; c++) {
        int tid = tid0;
        asm volatile("" : "+v"(lg), "+v"(ln), "+v"(tid));
        const int kb = (c + 1) & 1, sb = c & 1;
        const bool kwork = chunk_group && c + 1 < nch;  // chunk c + 1 (chunk group)
        const bool swork = !chunk_group && c >= 0;      // chunk c (state group)
        const int c1 = (c + 1) * KC;                    // first token of chunk c + 1
        const bool factored = __builtin_amdgcn_readfirstlane(L.pairwise) != c1 + 1;

        // ================= phase 1
        if (!chunk_group && c + 1 < nch) stage_vb(c1, tid - GT, nx);
        if (!chunk_group && c + 2 < nch) load_chunk(c1 + KC, tid - GT, nx);  // in flight until its staging
        if (kwork) {
            // element-wise operands of chunk c + 1 (arithmetic as in
            // prefill_kda_kernel), 8 tokens of one key channel per thread
            constexpr int TPT = KC * D / GT;
            static_assert(TPT == 8, "8 tokens per thread");
            const int ch = tid % D, t0 = TPT * (tid / D);
            const float gC = L.g[(KC - 1) * SG + ch], gm = L.g[kRefToken * SG + ch];
            const float egC = __builtin_amdgcn_exp2f(gC);
            const float egm = __builtin_amdgcn_exp2f(gm), emg = __builtin_amdgcn_exp2f(-gm);
            if (tid < D) L.egc[kb][ch] = egC;
            floatx4 kg0, kg1;
            bf16x8 kh8, kl8;
#pragma unroll
            for (int e = 0; e < TPT; e++) {
                const int t = t0 + e;
                const float gv = L.g[t * SG + ch];
                const float kv = (float)L.kr[t * SD + ch], qv = (float)L.qr[t * SD + ch];
                const float e1 = __builtin_amdgcn_exp2f(gv);
                const float ei = factored ? __builtin_amdgcn_exp2f(-gv) : 0.0f;
                const float e2 = factored ? egC * ei : __builtin_amdgcn_exp2f(gC - gv);
                if (e < 4) kg0[e] = kv * e1;
                else kg1[e - 4] = kv * e1;
                split(kv * e2, kh8, kl8, e);
                const float qe = qv * e1;
                const __bf16 qh = (__bf16)qe;
                L.qgh[kb][t * SD + ch] = qh;
                L.qgl[kb][t * SD + ch] = (__bf16)(qe - (float)qh);
                if (factored) {
                    const float fl = e1 * emg, fr = egm * ei;
                    L.xf[t * SG + ch] = kv * fl;
                    L.yf[t * SG + ch] = kv * fr;
                    L.zf[t * SG + ch] = qv * fl;
                }
            }
            *reinterpret_cast<floatx4 *>(&L.kgf[ch * SK + t0]) = kg0;
            *reinterpret_cast<floatx4 *>(&L.kgf[ch * SK + t0 + 4]) = kg1;
            *reinterpret_cast<bf16x8 *>(&L.kch[kb][ch * ST + t0]) = kh8;
            *reinterpret_cast<bf16x8 *>(&L.kcl[kb][ch * ST + t0]) = kl8;
        }
        floatx4 U[ET], O[ET];
        bf16x4 Vh[ET], Vl[ET];
        if (swork) {
            // U' = U - W S and O = (Q . 2^G) S for chunk c
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) U[et][r] = L.uf[sb][(4 * lg + r) * SG + e0 + 16 * et + ln];
            bf16x8 Sh[ET][KB], Sl[ET][KB];
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int k2 = 0; k2 < KB; k2++)
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        split(S[et][2 * k2][r], Sh[et][k2], Sl[et][k2], r);
                        split(S[et][2 * k2 + 1][r], Sh[et][k2], Sl[et][k2], 4 + r);
                    }
            // the three split-part products of each go to accumulators of
            // their own (chains of KB instead of 3 KB dependent products),
            // added on the VALU
            floatx4 U1[ET], U2[ET], O1[ET], O2[ET];
#pragma unroll
            for (int et = 0; et < ET; et++) {
                O[et] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                U1[et] = O[et];
                U2[et] = O[et];
                O1[et] = O[et];
                O2[et] = O[et];
            }
#pragma unroll
            for (int k2 = 0; k2 < KB; k2++) {
                const int row = ln * SD + 4 * lg + 32 * k2;
                const bf16x8 wh = ld_pair(&L.wh[sb][row]), wl = ld_pair(&L.wl[sb][row]);
                const bf16x8 qh = ld_pair(&L.qgh[sb][row]), ql = ld_pair(&L.qgl[sb][row]);
#pragma unroll
                for (int et = 0; et < ET; et++) {
                    U[et] = mma32(wh, Sh[et][k2], U[et]);
                    O[et] = mma32(qh, Sh[et][k2], O[et]);
                    U1[et] = mma32(wh, Sl[et][k2], U1[et]);
                    O1[et] = mma32(qh, Sl[et][k2], O1[et]);
                    U2[et] = mma32(wl, Sh[et][k2], U2[et]);
                    O2[et] = mma32(ql, Sh[et][k2], O2[et]);
                }
            }
#pragma unroll
            for (int et = 0; et < ET; et++) {
                U[et] += U1[et] + U2[et];
                O[et] += O1[et] + O2[et];
            }
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const floatx4 ec = ldf4(&L.egc[sb][16 * dt + 4 * lg]);
#pragma unroll
                for (int r = 0; r < 4; r++)
#pragma unroll
                    for (int et = 0; et < ET; et++) S[et][dt][r] *= ec[r];
            }
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) split(U[et][r], Vh[et], Vl[et], r);
        }
        // O += P U' (own accumulator, added on the VALU), outputs to ob
        auto outputs = [&]() {
            const bf16x4 pah = ld4(&L.ph[sb][ln * ST + 4 * lg]), pal = ld4(&L.pl[sb][ln * ST + 4 * lg]);
#pragma unroll
            for (int et = 0; et < ET; et++) {
                floatx4 pu = mma16(pah, Vh[et], floatx4{0.0f, 0.0f, 0.0f, 0.0f});
                pu = mma16(pah, Vl[et], pu);
                pu = mma16(pal, Vh[et], pu);
                O[et] += pu;
            }
#pragma unroll
            for (int et = 0; et < ET; et++)
#pragma unroll
                for (int r = 0; r < 4; r++) L.ob[(4 * lg + r) * SD + e0 + 16 * et + ln] = (__bf16)O[et][r];
        };
        // S <- diag(2^{G_C}) S + (K . 2^(G_C - G))^T U' (S already decayed)
        auto state_update = [&]() {
#pragma unroll
            for (int dt = 0; dt < DT; dt++) {
                const bf16x4 kah = ld4(&L.kch[sb][(16 * dt + ln) * ST + 4 * lg]);
                const bf16x4 kal = ld4(&L.kcl[sb][(16 * dt + ln) * ST + 4 * lg]);
#pragma unroll
                for (int et = 0; et < ET; et++) {
                    S[et][dt] = mma16(kah, Vh[et], S[et][dt]);
                    S[et][dt] = mma16(kah, Vl[et], S[et][dt]);
                    S[et][dt] = mma16(kal, Vh[et], S[et][dt]);
                }
            }
        };
        __syncthreads();  // B1: operands of chunk c + 1 staged

        // ================= phase 2 (and 3)
        if (factored) {
            // decayed Gram sums of chunk c + 1, factored (waves 0-3 as in
            // prefill_kda_kernel)
            floatx4 m = {0.0f, 0.0f, 0.0f, 0.0f};
            const bool isp = wave >= 2, first = (wave & 1) == 0;
            if (kwork) {
                constexpr int CPG = D / 8;
                const int cb = (wave & 1) * (D / 2) + CPG * lg;
                const float *xa = (isp ? L.yf : L.xf) + ln * SG + cb;
                const float *yb = (isp ? L.zf : L.yf) + ln * SG + cb;
                floatx4 m0 = {0.0f, 0.0f, 0.0f, 0.0f}, m1 = m0;
#pragma unroll
                for (int s4 = 0; s4 < CPG; s4 += 4) {
                    const floatx4 xv = ldf4(xa + s4), yv = ldf4(yb + s4);
                    m0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[0], yv[0], m0, 0, 0, 0);
                    m1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[1], yv[1], m1, 0, 0, 0);
                    m0 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[2], yv[2], m0, 0, 0, 0);
                    m1 = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[3], yv[3], m1, 0, 0, 0);
                }
                m = m0 + m1;
                if (!first) *reinterpret_cast<floatx4 *>(&L.gp[isp][ln * SA + 4 * lg]) = m;
            }
            __syncthreads();  // B2: second halves staged
            if (kwork && first) {
                m += ldf4(&L.gp[isp][ln * SA + 4 * lg]);
                if (!isp) {
                    const floatx4 bi = ldf4(&L.beta[4 * lg]);
                    floatx4 w;
#pragma unroll
                    for (int r = 0; r < 4; r++) w[r] = 4 * lg + r > ln ? bi[r] * m[r] : 0.0f;
                    *reinterpret_cast<floatx4 *>(&L.at[ln * SA + 4 * lg]) = w;
                } else {
                    bf16x4 h, l;
#pragma unroll
                    for (int r = 0; r < 4; r++) split(ln >= 4 * lg + r ? m[r] : 0.0f, h, l, r);
                    *reinterpret_cast<bf16x4 *>(&L.ph[kb][ln * ST + 4 * lg]) = h;
                    *reinterpret_cast<bf16x4 *>(&L.pl[kb][ln * ST + 4 * lg]) = l;
                }
            }
            if (swork) outputs();
        } else {
            if (kwork) {
                // decayed Gram sums of chunk c + 1, pair by pair: D/8 lanes per
                // pair, 8 key channels each, in batches of three passes (the
                // reads of a batch go out first)
                constexpr int LPP = D / 8, PPI = GT / LPP;
                constexpr int NP = (NPAIR + PPI - 1) / PPI, NB = 3;
                const int cb = tid % LPP, slot = tid / LPP, c8 = 8 * cb;
#pragma unroll
                for (int n0 = 0; n0 < NP; n0 += NB) {
                    int pi[NB], pj[NB];
                    bf16x8 kiv[NB], qiv[NB], kjv[NB];
                    floatx4 gi0[NB], gi1[NB], gj0[NB], gj1[NB];
#pragma unroll
                    for (int n = 0; n < NB; n++) {
                        const int ij = L.pij[min((n0 + n) * PPI + slot, NPAIR - 1)];
                        pi[n] = ij & 15;
                        pj[n] = ij >> 4;
                    }
#pragma unroll
                    for (int n = 0; n < NB; n++) {
                        kiv[n] = ld8(&L.kr[pi[n] * SD + c8]);
                        qiv[n] = ld8(&L.qr[pi[n] * SD + c8]);
                        kjv[n] = ld8(&L.kr[pj[n] * SD + c8]);
                        gi0[n] = ldf4(&L.g[pi[n] * SG + c8]);
                        gi1[n] = ldf4(&L.g[pi[n] * SG + c8 + 4]);
                        gj0[n] = ldf4(&L.g[pj[n] * SG + c8]);
                        gj1[n] = ldf4(&L.g[pj[n] * SG + c8 + 4]);
                    }
#pragma unroll
                    for (int n = 0; n < NB; n++) {
                        const int i = pi[n], j = pj[n];
                        float sa = 0.0f, sp = 0.0f;
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const float gi = e < 4 ? gi0[n][e] : gi1[n][e - 4];
                            const float gj = e < 4 ? gj0[n][e] : gj1[n][e - 4];
                            const float t = (float)kjv[n][e] * __builtin_amdgcn_exp2f(gi - gj);
                            sa = fmaf((float)kiv[n][e], t, sa);
                            sp = fmaf((float)qiv[n][e], t, sp);
                        }
                        sa = group_sum<LPP>(sa);
                        sp = group_sum<LPP>(sp);
                        if (cb == 0 && (n0 + n) * PPI + slot < NPAIR) {
                            if (j < i) L.at[j * SA + i] = L.beta[i] * sa;
                            const __bf16 h = (__bf16)sp;
                            L.ph[kb][i * ST + j] = h;
                            L.pl[kb][i * ST + j] = (__bf16)(sp - (float)h);
                        }
                    }
                }
            }
            if (swork) outputs();
        }
        __syncthreads();  // B3: A^T and P of chunk c + 1 complete; ob of chunk c complete

        // ================= phase 4
        if (kwork) {
            // U = T1 V and W = T1 (K . 2^G) of chunk c + 1 by forward
            // substitution (as in prefill_kda_kernel)
            const bool isw = tid >= D;  // wave-uniform
            const int ch = isw ? tid - D : tid;
            float y[KC];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const floatx4 bq = ldf4(&L.beta[4 * q]);
                if (isw) {
                    const floatx4 rq = ldf4(&L.kgf[ch * SK + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; e++) y[4 * q + e] = bq[e] * rq[e];
                } else {
                    const bf16x4 rq = ld4(&L.vt[ch * ST + 4 * q]);
#pragma unroll
                    for (int e = 0; e < 4; e++) y[4 * q + e] = bq[e] * (float)rq[e];
                }
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                constexpr int HS = KC / 2;
                floatx4 col[HS][4];
#pragma unroll
                for (int s = h * HS; s < min(KC - 1, (h + 1) * HS); s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++) col[s - h * HS][q] = ldf4(&L.at[s * SA + 4 * q]);
#pragma unroll
                for (int s = h * HS; s < min(KC - 1, (h + 1) * HS); s++)
#pragma unroll
                    for (int q = (s + 1) / 4; q < 4; q++)
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            if (4 * q + e > s) y[4 * q + e] = fmaf(-col[s - h * HS][q][e], y[s], y[4 * q + e]);
            }
            if (isw) {
#pragma unroll
                for (int t = 0; t < KC; t++) {
                    const float w = -y[t];
                    const __bf16 h = (__bf16)w;
                    L.wh[kb][t * SD + ch] = h;
                    L.wl[kb][t * SD + ch] = (__bf16)(w - (float)h);
                }
            } else {
#pragma unroll
                for (int t = 0; t < KC; t++) L.uf[kb][t * SG + ch] = y[t];
            }
        }
        if (swork) state_update();
        if (swork) {
            // the workgroup's columns: PW 16-byte pieces per token row
            constexpr int PW = D / NS / 8;
            const int c0 = c * KC, nv = min(KC, T - c0);
            const int x = tid - GT, t = x / PW, c8 = part * (D / NS) + 8 * (x % PW);
            static_assert(KC * PW <= ST_T, "one 16-byte output piece per state-group thread");
            if (x < KC * PW && t < nv)
                *reinterpret_cast<u32x4 *>(og + (size_t)(c0 + t) * tv + c8) =
                    *reinterpret_cast<const u32x4 *>(&L.ob[t * SD + c8]);
        }
        if (!chunk_group && c + 2 < nch) stage_kqg(c1 + KC, tid - GT, nx);  // chunk c + 1 reads K, Q, G no more
        __syncthreads();  // B4: U, -W of chunk c + 1 complete; chunk c + 2's K, Q, G staged
    }

    if (!chunk_group) {
#pragma unroll
        for (int et = 0; et < ET; et++)
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    Sg[(size_t)(16 * dt + 4 * lg + r) * D + e0 + 16 * et + ln] = S[et][dt][r];
    }
}

hipError_t launch_prefill_kda(const gdnq_desc &d, float *S, const void *q, const void *k, const void *v,
                              const float *a, const float *b, void *o, int T, hipStream_t st)
{
    const int hk = d.hk ? d.hk : d.H;
    PrefillKdaArgs A{S,
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
        if (grid * 4u <= (unsigned)ncu)
            hipLaunchKernelGGL((prefill_kda_ws_kernel<128, 4>), dim3(grid * 4), dim3(kda_ws_threads<4>()), 0, st, A);
        else if (grid * 2u <= (unsigned)ncu)
            hipLaunchKernelGGL((prefill_kda_ws_kernel<128, 2>), dim3(grid * 2), dim3(kda_ws_threads<2>()), 0, st, A);
        else
            hipLaunchKernelGGL((prefill_kda_ws_kernel<128, 1>), dim3(grid), dim3(kda_ws_threads<1>()), 0, st, A);
    } else {
        hipLaunchKernelGGL(prefill_kda_kernel<64>, dim3(grid), dim3(kda_threads<64>()), 0, st, A);
    }
    return hipGetLastError();
}

}  // namespace gdnq
