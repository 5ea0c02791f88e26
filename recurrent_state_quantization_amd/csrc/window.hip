// window.hip -- per-window decode step and window flush.
//
// LeapQuant project page, per-window quantization paragraph: the low-bit
// state of the window start stays fixed, each token's high-precision
// update is buffered, outputs come from the fixed state plus the buffer,
// and only at the window end is the full state rebuilt and requantized.
// Compensator Tokens paragraph: the compensators are rank-1 terms of the
// same form as token updates and ride on the same path (here: slots of the
// fixed state that decay with it).
//
// Let G_t = a_1 ... a_t (per key channel; one value per head for the scalar
// gate) be the gate product since the window start and X_0 the fixed state
// (dequantized codes + DAMP fp16 rows + compensators).  Unrolling the
// recurrence from X_0:
//   S_t = diag(G_t) X_0 + sum_{l<=t} ((G_t/G_l) . k_l) u_l^T
// so
//   S'^T k_t = X_0^T (G_t . k_t) + sum_{l<t} u_l (((G_t/G_l) . k_l) . k_t)
//   o_t      = X_0^T (G_t . q_t) + sum_{l<t} u_l (((G_t/G_l) . k_l) . q_t) + u_t (k_t . q_t)
//   S_W      = diag(G_W) X_0 + sum_{l<=n} ((G_W/G_l) . k_l) u_l^T
// A gate product can leave fp32's range long before the ratios G_t/G_l
// (all <= 1) do, so each is kept as G_t = m_t 2^(e_t): a mantissa m_t in
// [0.5, 1) (the running product of the gates' mantissas, renormalized each
// step, so it rounds exactly like a plain fp32 product) and an integer
// exponent e_t.  The buffer holds k^_l = k_l / m_l and e_l; a ratio times a
// key is then k^_l m_t scaled by 2^(e_t - e_l), an exact ldexp (a result
// below fp32's range rounds to a subnormal or zero, the value it has).
// Every rank-1 piece of X_0 (compensator p w^T, DAMP row e_i h_i^T) is a
// "slot" with key-side vector and value-side vector, like a buffered token.
#include "codec.hpp"
#include "launch.hpp"
#include "launchers.hpp"

namespace gdnq {

constexpr int MAX_SLOTS = MAX_R + MAX_HP + MAX_W;

typedef float floatx4 __attribute__((ext_vector_type(4)));

struct WinArgs {
    const void *q, *k, *v;
    const float *a, *b;
    void *o;
    const int8_t *codes;
    const float *row_scale, *col_scale;
    const float *comp_k, *comp_v;
    float *buf_k, *buf_u;
    int32_t *buf_g;
    float *g_cur;
    const uint16_t *hp_rows;
    const int32_t *hp_idx;
    int r, n_hp, W, t;
    HeadMap map;
};

// sum over the 16 lanes of a DPP row
__device__ __forceinline__ float sum16(float x)
{
    x += dpp<DPP_XOR1>(x);
    x += dpp<DPP_XOR2>(x);
    x += dpp<DPP_HALF_MIRROR>(x);
    x += dpp<DPP_MIRROR>(x);
    return x;
}

__device__ __forceinline__ void load_f16x8(const uint16_t *p, float (&out)[8])
{
    const uint4 raw = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        out[2 * i] = f16_to_f32((uint16_t)(w[i] & 0xFFFFu));
        out[2 * i + 1] = f16_to_f32((uint16_t)(w[i] >> 16));
    }
}

// Gate product after one more gate: (m, e) with m in [0.5, 1) from the
// previous (mp, ep) (the window start is m = 1, e = 0) and a gate a in
// (0, 1].  Both mantissas lie in [0.5, 1], so their product is a normal
// number and rounds once, like the plain product of the two values.
struct GateProd {
    float m;
    int e;
};

__device__ __forceinline__ GateProd gate_step(float mp, int ep, float a)
{
    const float p = mp * __builtin_amdgcn_frexp_mantf(a);
    return GateProd{__builtin_amdgcn_frexp_mantf(p),
                    ep + __builtin_amdgcn_frexp_expf(a) + __builtin_amdgcn_frexp_expf(p)};
}

__device__ __forceinline__ float ldexp_f(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

template <class G>
struct WinLds {
    alignas(16) float sgk[G::DK];  // s_i G_i k_i and s_i G_i q_i (s = 1 for DAMP), read as float4
    alignas(16) float sgq[G::DK];
    alignas(16) float cs[G::DV];   // column scales
    // raw k, q; m k, m q (token slots); G k, G q (fixed state, compensator
    // and DAMP slots); per-row mantissa and exponent of G
    float ks[G::DK], qs[G::DK], mk[G::DK], mq[G::DK], gk[G::DK], gq[G::DK], gm[G::DK];
    int ge[G::DK];
    float alpha[MAX_SLOTS + 1], beta[MAX_SLOTS + 1];
    int hp[MAX_HP];
    float red[G::NW][2][G::DV];
};

// Key-side vector of slot l (a compensator or a buffered token), entries
// l16*PER .. l16*PER+PER-1; false (nothing read) for a DAMP-row slot, the
// k.q slot and l >= NS.
template <class G>
__device__ __forceinline__ bool slot_kvec(const WinArgs &A, size_t h, int l, int NS, int n_hp, int l16,
                                          float (&x)[G::DK / 16])
{
    constexpr int PER = G::DK / 16;
    const int r = A.r;
    if (l >= NS || (l >= r && l < r + n_hp)) return false;
    const float *vec = (l < r) ? A.comp_k + ((h * r + l) * G::DK) : A.buf_k + (h * A.W + (l - r - n_hp)) * G::DK;
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
        const float4 v = *reinterpret_cast<const float4 *>(vec + l16 * PER + e);
        x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
    }
    return true;
}

// Gate exponents of buffered token j (slot r + n_hp + j): entries
// l16*PER .. +PER-1 for KDA, the head's one value for the scalar gate.
template <class G, bool KDA>
__device__ __forceinline__ void slot_kexp(const WinArgs &A, size_t h, int j, int l16, int (&xe)[G::DK / 16])
{
    constexpr int PER = G::DK / 16;
    const size_t tok = h * A.W + j;
    if constexpr (KDA) {
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
            const int4 v = *reinterpret_cast<const int4 *>(A.buf_g + tok * G::DK + l16 * PER + e);
            xe[e] = v.x; xe[e + 1] = v.y; xe[e + 2] = v.z; xe[e + 3] = v.w;
        }
    } else {
        xe[0] = A.buf_g[tok];
    }
}

// Value-side entries col..col+7 of slot l (l < NS), loaded as raw bits so
// that nothing waits for them until slot_vvec_use: eight fp32 words, or
// (returns true) eight fp16 halves in raw[0..3] for a DAMP-row slot.
template <class G>
__device__ __forceinline__ bool slot_vvec_load(const WinArgs &A, size_t h, int l, int n_hp, int col,
                                               uint4 (&raw)[2])
{
    const int r = A.r;
    const bool f16 = l >= r && l < r + n_hp;
    // one load path (a second load into the same registers on another
    // path would make the first one be waited for)
    const uint4 *p = f16 ? reinterpret_cast<const uint4 *>(A.hp_rows + (h * n_hp + (l - r)) * G::DV + col)
                   : reinterpret_cast<const uint4 *>((l < r) ? A.comp_v + (h * r + l) * G::DV + col
                                                             : A.buf_u + (h * A.W + (l - r - n_hp)) * G::DV + col);
    raw[0] = p[0];
    if (!f16) raw[1] = p[1];
    return f16;
}

__device__ __forceinline__ void slot_vvec_use(const uint4 (&raw)[2], bool f16, float (&uv)[8])
{
    if (f16) {
        const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uv[2 * i] = f16_to_f32((uint16_t)(w[i] & 0xFFFFu));
            uv[2 * i + 1] = f16_to_f32((uint16_t)(w[i] >> 16));
        }
    } else {
        const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int j = 0; j < 8; j++) uv[j] = __uint_as_float(w[j]);
    }
}

// This thread's 8 code rows of the fixed tile (DAMP rows carry no codes).
template <class G, bool DAMP, int BITS>
__device__ __forceinline__ void load_tile_codes(const int8_t *codes, const Lane &c, const RowMap &rm,
                                                CodeWord (&qraw)[8])
{
    constexpr int RB = code_row_bytes<G, BITS>();
#pragma unroll
    for (int k = 0; k < 8; k++) {
        if (!DAMP || rm.slot[k] < 0) {
            const int row = DAMP ? rm.crow[k] : row_of<G>(c, k);
            qraw[k] = load_code8<G, BITS>(codes + (size_t)row * RB, c.cb);
        } else {
            qraw[k] = CodeWord{0u, 0u};
        }
    }
}

// 8 workgroups per CU (64 VGPRs, no spills; the column scales wait in LDS
// so the prefetched slot vectors fit beside the codes): 2048 heads run as
// one round over the 256 CUs, 8192 as four.  The 6-bit unpack needs more
// temporaries, and the per-channel gate its tokens' gate exponents: 7 per
// CU (72 VGPRs) keeps those from spilling.
template <int BITS, bool KDA>
constexpr int step_min_blocks() { return (BITS == 6 || KDA) ? 7 : 8; }

template <class G, bool BF16, bool KDA, bool DAMP, int BITS>
__global__ __launch_bounds__(G::NT, (step_min_blocks<BITS, KDA>())) void window_step_kernel(WinArgs A)
{
    static_assert(!DAMP || BITS == 8, "the DAMP layout keeps 8-bit codes");
    __shared__ WinLds<G> L;
    const Lane c = lane_coords<G>();
    HeadIdx x;
    if (!map_head(A.map, A.t, 0, A.W - 1, x)) return;  // uniform per workgroup, before any barrier
    const size_t h = x.state, hi = x.in, hk = x.key;  // state, input and key head
    const int t = x.pos;
    const int n_hp = DAMP ? A.n_hp : 0;
    const int r = A.r;

    // Every load that does not depend on LDS is issued before the first
    // barrier, the small ones first so that the barrier waits for them
    // only: the per-row inputs (thread t < DK owns row t; rows wrap for
    // t >= DK), the scales, the DAMP row indices, then the first slot
    // vectors and the codes.
    const int tr = c.t % G::DK;
    const float kv = load1<BF16>(A.k, hk * G::DK + tr);
    const float qv = load1<BF16>(A.q, hk * G::DK + tr);
    const float av = KDA ? A.a[hi * G::DK + tr] : A.a[hi];
    // gate product of the previous token (the window start: 1 = 0.5 * 2^1)
    float mprev = 1.0f;
    int eprev = 0;
    if (t > 0) {
        mprev = KDA ? A.g_cur[h * G::DK + tr] : A.g_cur[h];
        eprev = KDA ? A.buf_g[(h * A.W + (t - 1)) * G::DK + tr] : A.buf_g[h * A.W + (t - 1)];
    }
    const float srow = DAMP ? 1.0f : A.row_scale[h * G::DK + tr];
    // column scales go through LDS (thread t < DV owns column t) so they
    // hold no registers during the mat-vecs
    const float cj = A.col_scale[h * G::DV + (c.t % G::DV)];
    int hpi = 0;
    if (DAMP && c.t < n_hp) hpi = A.hp_idx[h * n_hp + c.t];
    __builtin_amdgcn_sched_barrier(0);
    // the first slot each 16-lane group dots (key side) and each row group
    // adds (value side); later ones, if any, load in their loops
    const int NS = r + n_hp + t;
    constexpr int PER = G::DK / 16;
    const int l16 = c.t & 15;
    float xk[PER];
    const bool xk0 = slot_kvec<G>(A, h, c.t >> 4, NS, n_hp, l16, xk);
    constexpr int NRG = G::NW * G::RGW;
    const int rg = c.w * G::RGW + c.rgl;
    uint4 uvraw[2];
    bool uv16 = false;
    // (with the per-channel gate this load waits until after the slot dot
    // products, whose per-channel exponents need the registers)
    if (!KDA && rg < NS) uv16 = slot_vvec_load<G>(A, h, rg, n_hp, c.cb * 8, uvraw);
    __builtin_amdgcn_sched_barrier(0);

    // fixed INT8 tile (DAMP: its row map from the head's row list in global
    // memory, so that these loads too go out before the first barrier)
    const size_t nrows_c = (size_t)(G::DK - n_hp);
    const int8_t *codes = A.codes + h * nrows_c * code_row_bytes<G, BITS>();
    CodeWord qraw[8];
    RowMap rm;
    if constexpr (DAMP) rm = row_map<G>(c, A.hp_idx + h * n_hp, n_hp);
    load_tile_codes<G, DAMP, BITS>(codes, c, rm, qraw);

    // per-row vectors: gate product, gated k and q (and times the row scale)
    if (c.t < G::DK) {
        const GateProd g = gate_step(mprev, eprev, av);
        const float mk = g.m * kv, mq = g.m * qv;
        const float gk = ldexp_f(mk, g.e), gq = ldexp_f(mq, g.e);
        L.ks[c.t] = kv;
        L.qs[c.t] = qv;
        L.mk[c.t] = mk;
        L.mq[c.t] = mq;
        L.gm[c.t] = g.m;
        L.ge[c.t] = g.e;
        L.gk[c.t] = gk;
        L.gq[c.t] = gq;
        L.sgk[c.t] = srow * gk;
        L.sgq[c.t] = srow * gq;
    }
    if (c.t < G::DV) L.cs[c.t] = cj;
    if (DAMP && c.t < n_hp) L.hp[c.t] = hpi;
    __syncthreads();

    // slot dot products.  A buffered token l gives
    //   alpha_l = ((G_t/G_l) . k_l) . k_t = sum_c k^_l,c m_t,c k_t,c 2^(e_t,c - e_l,c)
    // (beta_l with q_t), and a compensator p, part of the fixed state, the
    // same with k^ = p and e_l = 0: (G_t . p) . k_t.  A DAMP row i gives
    // G_t,i k_t,i; slot NS is k . q.  16 lanes per slot.
    for (int base = 0; base <= NS; base += G::NT / 16) {
        const int l = base + (c.t >> 4);
        if (l > NS) break;  // whole 16-lane groups leave together
        const bool has = base == 0 ? xk0 : slot_kvec<G>(A, h, l, NS, n_hp, l16, xk);
        float al = 0.0f, be = 0.0f;
        if (l == NS) {
#pragma unroll
            for (int e = 0; e < PER; e++) al = fmaf(L.ks[l16 * PER + e], L.qs[l16 * PER + e], al);
        } else if (!has) {  // DAMP row slot: e_i . (G.k) = G_i k_i
            if (l16 == 0) {
                const int i = L.hp[l - r];
                al = L.gk[i];
                be = L.gq[i];
            }
        } else {
            // the slot's gate exponents (zero for a compensator; loaded here,
            // not held across the first barrier with the prefetched vector)
            int xe[PER];
            if (l >= r) {
                slot_kexp<G, KDA>(A, h, l - r - n_hp, l16, xe);
            } else {
#pragma unroll
                for (int e = 0; e < PER; e++) xe[e] = 0;
            }
            if constexpr (KDA) {
#pragma unroll
                for (int e = 0; e < PER; e++) {
                    const int i = l16 * PER + e;
                    const float x = ldexp_f(xk[e], L.ge[i] - xe[e]);
                    al = fmaf(x, L.mk[i], al);
                    be = fmaf(x, L.mq[i], be);
                }
            } else {
#pragma unroll
                for (int e = 0; e < PER; e++) {
                    al = fmaf(xk[e], L.mk[l16 * PER + e], al);
                    be = fmaf(xk[e], L.mq[l16 * PER + e], be);
                }
                // the scalar gate's ratio, once per slot
                al = ldexp_f(al, L.ge[0] - xe[0]);
                be = ldexp_f(be, L.ge[0] - xe[0]);
            }
        }
        al = sum16(al);
        be = sum16(be);
        if (l16 == 0) {
            L.alpha[l] = al;
            L.beta[l] = be;
        }
    }

    if (KDA && rg < NS) uv16 = slot_vvec_load<G>(A, h, rg, n_hp, c.cb * 8, uvraw);
    // fixed-state mat-vecs straight off the codes
    float gsk[8], gsq[8];
    load_rows_f32<G>(&L.sgk[row0_of<G>(c)], gsk);
    load_rows_f32<G>(&L.sgq[row0_of<G>(c)], gsq);
    float R[8], O[8];
    {
        float X[8];
        unpack_code8<BITS>(qraw[0], X);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            R[j] = X[j] * gsk[0];
            O[j] = X[j] * gsq[0];
        }
#pragma unroll
        for (int k = 1; k < 8; k++) {
            unpack_code8<BITS>(qraw[k], X);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                R[j] = fmaf(X[j], gsk[k], R[j]);
                O[j] = fmaf(X[j], gsq[k], O[j]);
            }
        }
    }
    {
        float cc[8];
        load_f32x8(&L.cs[c.cb * 8], cc);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            R[j] *= cc[j];
            O[j] *= cc[j];
        }
    }
    __syncthreads();  // alpha / beta ready

    // slot value-side terms, slots spread over the row groups
    for (int l = rg; l < NS; l += NRG) {
        const float al = L.alpha[l], be = L.beta[l];
        if (l != rg) uv16 = slot_vvec_load<G>(A, h, l, n_hp, c.cb * 8, uvraw);
        float uv[8];
        slot_vvec_use(uvraw, uv16, uv);
#pragma unroll
        for (int j = 0; j < 8; j++) {
            R[j] = fmaf(al, uv[j], R[j]);
            O[j] = fmaf(be, uv[j], O[j]);
        }
    }
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
            L.red[c.w][idx >> 3][c.cb * 8 + (idx & 7)] = z[p];
        }
    }
    __syncthreads();
    if (c.t < G::DV) {
        float ret = L.red[0][0][c.t], ot = L.red[0][1][c.t];
#pragma unroll
        for (int w = 1; w < G::NW; w++) {
            ret += L.red[w][0][c.t];
            ot += L.red[w][1][c.t];
        }
        const float u = A.b[hi] * (load1<BF16>(A.v, hi * G::DV + c.t) - ret);
        store1<BF16>(A.o, hi * G::DV + c.t, fmaf(u, L.alpha[NS], ot));
        A.buf_u[(h * A.W + t) * G::DV + c.t] = u;
    }
    if (c.t < G::DK) {
        const float m = L.gm[c.t];
        A.buf_k[(h * A.W + t) * G::DK + c.t] = L.ks[c.t] / m;
        if (KDA) {
            A.buf_g[(h * A.W + t) * G::DK + c.t] = L.ge[c.t];
            A.g_cur[h * G::DK + c.t] = m;
        } else if (c.t == 0) {
            A.buf_g[h * A.W + t] = L.ge[0];
            A.g_cur[h] = m;
        }
    }
}

// -------------------------------------------------------------------------
struct FlushArgs {
    int8_t *codes;
    float *row_scale, *col_scale, *comp_k, *comp_v;
    const float *buf_k, *buf_u;
    const int32_t *buf_g;
    float *g_cur;
    uint16_t *hp_rows;
    const int32_t *hp_idx;
    float *prequant;
    int r, n_hp, W, n, iters;
    HeadMap map;
};

template <class G>
struct FlushLds {
    float gs[G::DK];   // G_n per row (a subnormal or zero when it underflows)
    float gm[G::DK];   // its mantissa m_n and exponent e_n
    int ge[G::DK];
    int hp[MAX_HP];
};

// Key-side value of slot l at row i (already multiplied by G_n,i; a token's
// (G_n/G_l)_i k_l,i = m_n,i k^_l,i 2^(e_n,i - e_l,i)) and the 8 value-side
// entries at columns col..col+7.  Slots: r compensators, n_hp DAMP rows,
// n buffered tokens; l >= K is a zero pad.
template <class G, bool KDA>
__device__ __forceinline__ float slot_key(const FlushArgs &A, const FlushLds<G> &L, size_t h, int l, int i, int K)
{
    if (l >= K) return 0.0f;
    if (l < A.r) return L.gs[i] * A.comp_k[(h * A.r + l) * G::DK + i];
    if (l < A.r + A.n_hp) return (L.hp[l - A.r] == i) ? L.gs[i] : 0.0f;
    const size_t tok = h * A.W + (l - A.r - A.n_hp);
    const int el = KDA ? A.buf_g[tok * G::DK + i] : A.buf_g[tok];
    return ldexp_f(L.gm[i] * A.buf_k[tok * G::DK + i], L.ge[i] - el);
}

template <class G>
__device__ __forceinline__ void slot_val(const FlushArgs &A, size_t h, int l, int col, int K, float (&out)[8])
{
    if (l >= K) {
#pragma unroll
        for (int j = 0; j < 8; j++) out[j] = 0.0f;
    } else if (l < A.r) {
        load_f32x8(A.comp_v + (h * A.r + l) * G::DV + col, out);
    } else if (l < A.r + A.n_hp) {
        load_f16x8(A.hp_rows + (h * A.n_hp + (l - A.r)) * G::DV + col, out);
    } else {
        load_f32x8(A.buf_u + (h * A.W + (l - A.r - A.n_hp)) * G::DV + col, out);
    }
}

// Occupancy: the 128x128 rowcol flush fits 128 VGPRs without spilling, so
// it asks for 4 workgroups per CU (4 waves per SIMD: the power iteration
// is VALU-bound and its per-step barrier is hidden by the other
// workgroups); the DAMP and 64-row or 64-column variants would spill at that bound
// and ask for 2 (3 waves per SIMD at their register counts).
template <class G, bool DAMP>
constexpr int flush_min_blocks() { return (G::DK == 128 && G::DV == 128 && !DAMP) ? 4 : 2; }

template <class G, bool KDA, bool DAMP, int BITS>
__global__ __launch_bounds__(G::NT, (flush_min_blocks<G, DAMP>())) void flush_kernel(FlushArgs A)
{
    static_assert(!DAMP || BITS == 8, "the DAMP layout keeps 8-bit codes");
    constexpr int RB = code_row_bytes<G, BITS>();
    __shared__ CodecLds<G> L;
    __shared__ FlushLds<G> F;
    const Lane c = lane_coords<G>();
    HeadIdx x;
    if (!map_head(A.map, A.n, 1, A.W, x)) return;  // uniform per workgroup, before any barrier
    const size_t h = x.state;
    const int n = x.pos;
    const int n_hp = DAMP ? A.n_hp : 0;
    if (!DAMP) A.n_hp = 0;
    if (c.t < G::DK) {
        // the gate product after the window's last token, n - 1
        const float m = KDA ? A.g_cur[h * G::DK + c.t] : A.g_cur[h];
        const int e = KDA ? A.buf_g[(h * A.W + (n - 1)) * G::DK + c.t] : A.buf_g[h * A.W + (n - 1)];
        F.gm[c.t] = m;
        F.ge[c.t] = e;
        F.gs[c.t] = ldexp_f(m, e);
    }
    if (DAMP && c.t < n_hp) F.hp[c.t] = A.hp_idx[h * n_hp + c.t];
    __syncthreads();

    RowMap rm;
    if constexpr (DAMP) rm = row_map<G>(c, F.hp, n_hp);
    const size_t nrows_c = (size_t)(G::DK - n_hp);
    int8_t *codes = A.codes + h * nrows_c * RB;
    float cc[8];
    load_f32x8(A.col_scale + h * G::DV + c.cb * 8, cc);
    float P[8][8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int i = row_of<G>(c, k);
        if (!DAMP || rm.slot[k] < 0) {
            const int row = DAMP ? rm.crow[k] : i;
            float X[8];
            unpack_code8<BITS>(load_code8<G, BITS>(codes + (size_t)row * RB, c.cb), X);
            const float s = DAMP ? 1.0f : A.row_scale[h * G::DK + i];
            const float g = F.gs[i];
#pragma unroll
            for (int j = 0; j < 8; j++) P[k][j] = DAMP ? (X[j] * cc[j]) * g : ((X[j] * cc[j]) * s) * g;
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) P[k][j] = 0.0f;
        }
    }

    // rank-K update with the slots (compensators, DAMP rows, tokens)
    const int K = A.r + n_hp + n;
    if constexpr (G::DV == 128) {
        // 16x16x4 fp32 MFMA.  MFMA row m of block hb of wave w is tile row
        // w*32 + hb*16 + m; MFMA column n of block nb is tile column
        // 8*n + nb, so the accumulator of (hb, nb) holds P[hb*4 + i][nb].
        floatx4 acc[2][8];
#pragma unroll
        for (int hb = 0; hb < 2; hb++)
#pragma unroll
            for (int nb = 0; nb < 8; nb++)
#pragma unroll
                for (int i = 0; i < 4; i++) acc[hb][nb][i] = P[hb * 4 + i][nb];
        const int lm = c.lane & 15, lk = c.lane >> 4;
        for (int kk = 0; kk < K; kk += 4) {
            const int l = kk + lk;
            float av[2], bv[8];
#pragma unroll
            for (int hb = 0; hb < 2; hb++) av[hb] = slot_key<G, KDA>(A, F, h, l, c.w * 32 + hb * 16 + lm, K);
            slot_val<G>(A, h, l, 8 * lm, K, bv);
#pragma unroll
            for (int hb = 0; hb < 2; hb++)
#pragma unroll
                for (int nb = 0; nb < 8; nb++)
                    acc[hb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[hb], bv[nb], acc[hb][nb], 0, 0, 0);
        }
#pragma unroll
        for (int hb = 0; hb < 2; hb++)
#pragma unroll
            for (int nb = 0; nb < 8; nb++)
#pragma unroll
                for (int i = 0; i < 4; i++) P[hb * 4 + i][nb] = acc[hb][nb][i];
    } else {
        for (int l = 0; l < K; l++) {
            float kv[8], uv[8];
#pragma unroll
            for (int k = 0; k < 8; k++) kv[k] = slot_key<G, KDA>(A, F, h, l, row_of<G>(c, k), K);
            slot_val<G>(A, h, l, c.cb * 8, K, uv);
#pragma unroll
            for (int k = 0; k < 8; k++)
#pragma unroll
                for (int j = 0; j < 8; j++) P[k][j] = fmaf(kv[k], uv[j], P[k][j]);
        }
    }

    power_deflate<G, !DAMP>(P, c, L, A.r, A.iters, A.comp_k + h * A.r * G::DK, A.comp_v + h * A.r * G::DV);
    if (A.prequant) {
        float *pq = A.prequant + h * (size_t)G::DK * G::DV;
#pragma unroll
        for (int k = 0; k < 8; k++) store_f32x8(pq + (size_t)row_of<G>(c, k) * G::DV + c.cb * 8, P[k]);
    }
    __syncthreads();  // every read of codes / scales / DAMP rows is done
    if constexpr (DAMP)
        codec_damp<G>(P, c, L, rm, codes, A.col_scale + h * G::DV, A.hp_rows + h * n_hp * G::DV);
    else
        codec_rowcol<G, false, BITS>(P, c, L, codes, A.row_scale + h * G::DK, A.col_scale + h * G::DV);
    if (c.t < G::DK) {
        if (KDA) A.g_cur[h * G::DK + c.t] = 1.0f;
        else if (c.t == 0) A.g_cur[h] = 1.0f;
    }
}

hipError_t launch_window_step(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, const void *q,
                              const void *k, const void *v, const float *a, const float *b, void *o,
                              int t_in_window, hipStream_t st)
{
    WinArgs A{q, k, v, a, b, o, s.codes, s.row_scale, s.col_scale, s.comp_k, s.comp_v,
              s.buf_k, s.buf_u, s.buf_g, s.g_cur, s.hp_rows, s.hp_idx, d.r, d.n_hp, d.W, t_in_window, m};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.io_dtype == GDNQ_IO_BF16, [&](auto bf) {
            return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
                return with_bool(d.layout == GDNQ_LAYOUT_DAMP, [&](auto damp) {
                    return with_bits(d.bits, [&](auto bits) {
                        constexpr bool DAMP = decltype(damp)::value;
                        constexpr int BITS = decltype(bits)::value;
                        if constexpr (DAMP && BITS != 8) {
                            return hipErrorInvalidValue;
                        } else {
                            hipLaunchKernelGGL((window_step_kernel<G, decltype(bf)::value, decltype(kda)::value,
                                                                   DAMP, BITS>),
                                               dim3(nh), dim3(G::NT), 0, st, A);
                            return hipGetLastError();
                        }
                    });
                });
            });
        });
    });
}

hipError_t launch_flush(const gdnq_desc &d, const HeadMap &m, const gdnq_state &s, int n_tokens, hipStream_t st)
{
    FlushArgs A{s.codes, s.row_scale, s.col_scale, s.comp_k, s.comp_v, s.buf_k, s.buf_u, s.buf_g, s.g_cur,
                s.hp_rows, s.hp_idx, (d.flags & GDNQ_DEBUG_PREQUANT) ? s.prequant_out : nullptr,
                d.r, d.n_hp, d.W, n_tokens, d.power_iters, m};
    const unsigned nh = (unsigned)d.B * (unsigned)d.H;
    return with_dims(d.dk, d.dv, [&](auto DK, auto DV) {
        using G = Geom<decltype(DK)::value, decltype(DV)::value>;
        return with_bool(d.decay == GDNQ_DECAY_CHANNEL, [&](auto kda) {
            return with_bool(d.layout == GDNQ_LAYOUT_DAMP, [&](auto damp) {
                return with_bits(d.bits, [&](auto bits) {
                    constexpr bool DAMP = decltype(damp)::value;
                    constexpr int BITS = decltype(bits)::value;
                    if constexpr (DAMP && BITS != 8) {
                        return hipErrorInvalidValue;
                    } else {
                        hipLaunchKernelGGL((flush_kernel<G, decltype(kda)::value, DAMP, BITS>), dim3(nh),
                                           dim3(G::NT), 0, st, A);
                        return hipGetLastError();
                    }
                });
            });
        });
    });
}

}  // namespace gdnq
