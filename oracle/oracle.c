/*
 * oracle.c -- plain, slow, single-threaded fp64 CPU oracle for quantized
 * Gated-DeltaNet / Kimi-Delta-Attention recurrent-state decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's
 * cpu_baseline leg do.  It shares no code, header, table or constant with
 * the HIP library and includes none of its files.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -std=c11 oracle.c -lm
 * (-ffp-contract=off: no fused multiply-add, every operation is rounded on
 * its own, so the fp32 emulation below is exact.)
 *
 * Sources (web pages this follows; the method is given there in prose only):
 *  [LEAP]  "LeapQuant: Efficient Linear Attention with Accurate Recurrent
 *          State Quantization" (project page): the paragraphs on the
 *          per-token state load/update/write-back, on per-window
 *          quantization, on Compensator Tokens and on residual smoothing.
 *  [LINQ]  "LinQuant: Functional Invariances for Low-Precision Linear
 *          Recurrences", appendix Table 3 (state-update rules of DeltaNet,
 *          Gated DeltaNet, KDA) and Table 1 (invariances).
 *  [STEP]  "How does STEPQuant compress recurrent states without losing
 *          accuracy?": key-row and value-column scales.
 *  [DAMP]  "DAMP: Decay-Aware Mixed-Precision Recurrent-State
 *          Quantization", abstract: high-risk channels picked offline from
 *          quantization-error energy and decay persistence, kept at higher
 *          precision, the rest in INT8.
 *
 * Orientation.  [LINQ] Table 3 writes the state as dv x dk with
 *   S_t = alpha_t S_{t-1} (I - beta_t k k^T) + beta_t v k^T   (GDN).
 * This file stores its transpose, dk x dv, row i = key channel, column j =
 * value channel, row-major:
 *   S' = a S (GDN) or diag(a) S (KDA);  u = b (v - S'^T k);
 *   S_t = S' + k u^T;                    o = S_t^T q.
 * Expanding (I - b k k^T) shows the two forms are the same matrix.
 *
 * Readings taken where the pages are silent (each is repeated where used):
 *  - smoothing scale of key row i: s_i = sqrt(max_j |X_ij|); rows are
 *    divided by s_i before the value-column scales are taken;
 *  - value-column scales are symmetric: c_j = m_j / Qb, codes in
 *    [-Qb, Qb] with Qb = 2^(b-1) - 1 for a code width of b bits (127 for
 *    the INT8 state; 31 and 7 for the 6- and 4-bit states the LeapQuant
 *    accuracy table reports), round half to even;
 *  - codes of b < 8 bits are stored packed (orc_pack_codes): 4 bits as two
 *    two's-complement nibbles per byte, even column in the low nibble; 6
 *    bits as one 48-bit record per block of 8 columns (column 8k+e in bits
 *    6e..6e+5), the records' low 32 bits in a first plane and their high
 *    16 bits in a second;
 *  - every codec step is one IEEE fp32 operation rounded to nearest even,
 *    in the order written below, with no fused multiply-add, except the
 *    last: the code is the integer nearest to the exact product
 *    Y_ij * iota_j (ties to even), with no intermediate rounding;
 *  - zero rows/columns get scale 0, reciprocal 0 and code 0; a column whose
 *    reciprocal scale Qb/m_j overflows fp32 is treated as a zero column;
 *  - the output of a per-step quantized decode is taken from the updated
 *    state before it is requantized;
 *  - Compensator Tokens: sequential deflation, each term found by
 *    `iters` power-iteration steps v <- R^T(R v)/|R^T(R v)| from the
 *    all-equal unit vector; the stored pair is p = R v (fp32, key side)
 *    and w = v (fp32, unit, value side); deflation uses the stored fp32
 *    pair so that compensators + residual rebuild the state;
 *  - inside a window the compensators are part of the fixed state (they
 *    decay with it), matching "no separate state update";
 *  - DAMP rows: the listed high-precision key rows are stored as IEEE
 *    half (round to nearest even, saturating at +-65504); the other rows
 *    are INT8 with per-value-column scales over those rows only and no
 *    row smoothing.
 *
 * Emulating one fp32 operation: the operands are fp32 values, the exact
 * result is computed in fp64 and rounded once to fp32.  A product of two
 * fp32 values is exact in fp64; for a quotient or square root the fp64
 * result is already rounded once, and rounding it again to fp32 gives the
 * correctly rounded fp32 result because 53 >= 2*24 + 2 (S. A. Figueroa,
 * "When is double rounding innocuous?", SIGNUM Newsletter 30(3), 1995).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- one correctly rounded fp32 operation, computed in fp64 ----------- */
static float f32_mul(float x, float y) { return (float)((double)x * (double)y); }
static float f32_div(float x, float y) { return (float)((double)x / (double)y); }
static float f32_sqrt(float x) { return (float)sqrt((double)x); }

/* round to nearest integer, ties to even (the C default rounding mode) */
static double round_half_even(double t) { return nearbyint(t); }

/* ======================================================================
 * c2: the state codec, layout 0 (row smoothing + value-column scales).
 * [LEAP] residual-smoothing paragraph: rows are balanced before
 * quantization and the smoothing scales are recomputed at every window
 * boundary.  [STEP]: key-row and value-column scales.
 * X is one dk x dv fp32 tile.  Outputs: codes Q (int8, dk x dv), row
 * smoothing scales s (dk), column scales c (dv).
 * ==================================================================== */
static void quantize_tile(int dk, int dv, int qmax, const float *X, int8_t *Q, float *s, float *c)
{
    const float qm = (float)qmax;
    float *Y = (float *)malloc(sizeof(float) * (size_t)dk * dv);
    for (int i = 0; i < dk; i++) {
        float r = 0.0f;                                   /* r_i = max_j |X_ij| */
        for (int j = 0; j < dv; j++) {
            float a = fabsf(X[i * dv + j]);
            if (a > r) r = a;
        }
        float si = (r > 0.0f) ? f32_sqrt(r) : 0.0f;      /* s_i = sqrt(r_i)   */
        float rho = (si > 0.0f) ? f32_div(1.0f, si) : 0.0f; /* rho_i = 1/s_i */
        s[i] = si;
        for (int j = 0; j < dv; j++)                      /* Y_ij = X_ij rho_i */
            Y[i * dv + j] = f32_mul(X[i * dv + j], rho);
    }
    for (int j = 0; j < dv; j++) {
        float m = 0.0f;                                   /* m_j = max_i |Y_ij| */
        for (int i = 0; i < dk; i++) {
            float a = fabsf(Y[i * dv + j]);
            if (a > m) m = a;
        }
        float cj = 0.0f, iota = 0.0f;
        if (m > 0.0f) {
            iota = f32_div(qm, m);                        /* iota_j = Qb/m_j   */
            if (isinf(iota)) iota = 0.0f;                 /* overflow: zero column */
            else cj = f32_div(m, qm);                     /* c_j = m_j/Qb      */
        }
        c[j] = cj;
        for (int i = 0; i < dk; i++) {
            /* exact product of two fp32 values (fits in fp64), rounded once */
            double qv = round_half_even((double)Y[i * dv + j] * (double)iota);
            if (qv > qmax) qv = qmax;
            if (qv < -qmax) qv = -qmax;
            Q[i * dv + j] = (int8_t)qv;
        }
    }
    free(Y);
}

/* Dequantize one tile: X_ij = (Q_ij * c_j) * s_i, two rounded fp32 products. */
static void dequantize_tile(int dk, int dv, const int8_t *Q, const float *s, const float *c, float *X)
{
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++)
            X[i * dv + j] = f32_mul(f32_mul((float)Q[i * dv + j], c[j]), s[i]);
}

/* largest code of a b-bit state: 2^(b-1) - 1 (b = 8, 6 or 4) */
static int code_qmax(int bits) { return (1 << (bits - 1)) - 1; }

/* ======================================================================
 * Packed code layout of one row of dv codes (b = 8, 6, 4 bits), as stored
 * in memory; rows follow each other, dv*b/8 bytes apart.
 *   b = 8: one byte per code.
 *   b = 4: code j in byte j/2, bits 4*(j%2)..+3 (two's complement nibble).
 *   b = 6: block k = columns 8k..8k+7 forms a 48-bit little-endian record,
 *          code 8k+e (6-bit two's complement) in record bits 6e..6e+5;
 *          record bits 0..31 go to bytes 4k..4k+3, bits 32..47 to bytes
 *          dv/2 + 2k .. dv/2 + 2k + 1.
 * ==================================================================== */
static void pack_row(int dv, int bits, const int8_t *Q, uint8_t *P)
{
    int nb = dv * bits / 8;
    memset(P, 0, (size_t)nb);
    for (int j = 0; j < dv; j++) {
        unsigned u = (unsigned)(uint8_t)Q[j];            /* two's complement byte */
        if (bits == 8) {
            P[j] = (uint8_t)u;
        } else if (bits == 4) {
            P[j / 2] |= (uint8_t)((u & 0xFu) << (4 * (j % 2)));
        } else {
            int k = j / 8, pos = 6 * (j % 8);             /* record bit of the field */
            for (int t = 0; t < 6; t++) {
                int rb = pos + t;                         /* record bit */
                int byte = rb < 32 ? 4 * k + rb / 8 : dv / 2 + 2 * k + (rb - 32) / 8;
                P[byte] |= (uint8_t)(((u >> t) & 1u) << (rb % 8));
            }
        }
    }
}

static void unpack_row(int dv, int bits, const uint8_t *P, int8_t *Q)
{
    for (int j = 0; j < dv; j++) {
        int v = 0;
        if (bits == 8) {
            v = (int8_t)P[j];
        } else {
            if (bits == 4) {
                v = (P[j / 2] >> (4 * (j % 2))) & 0xF;
            } else {
                int k = j / 8, pos = 6 * (j % 8);
                for (int t = 0; t < 6; t++) {
                    int rb = pos + t;
                    int byte = rb < 32 ? 4 * k + rb / 8 : dv / 2 + 2 * k + (rb - 32) / 8;
                    v |= ((P[byte] >> (rb % 8)) & 1) << t;
                }
            }
            if (v >= (1 << (bits - 1))) v -= 1 << bits;  /* sign of the b-bit field */
        }
        Q[j] = (int8_t)v;
    }
}

/* ======================================================================
 * IEEE binary16 conversion, round to nearest even, saturating at +-65504.
 * [DAMP] abstract: high-risk channels are kept at higher precision.
 * Written from the binary16 definition: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits; subnormals have quantum 2^-24.
 * ==================================================================== */
static uint16_t f32_to_f16_bits(float x)
{
    double a = fabs((double)x);
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (a == 0.0) return sign;
    double q;                                    /* a rounded to the fp16 grid */
    if (a < ldexp(1.0, -14)) {
        q = round_half_even(a / ldexp(1.0, -24)) * ldexp(1.0, -24);
    } else {
        int e;
        (void)frexp(a, &e);                      /* a = f * 2^e, f in [0.5,1) */
        double ulp = ldexp(1.0, (e - 1) - 10);   /* 10 fraction bits */
        q = round_half_even(a / ulp) * ulp;
    }
    if (q > 65504.0) q = 65504.0;                /* saturate, never inf */
    if (q == 0.0) return sign;
    if (q < ldexp(1.0, -14)) {                   /* subnormal encoding */
        return (uint16_t)(sign | (uint16_t)(q / ldexp(1.0, -24)));
    }
    int e;
    double f = frexp(q, &e);                     /* q = f * 2^e */
    int E = (e - 1) + 15;                        /* biased exponent */
    int frac = (int)((f * 2.0 - 1.0) * 1024.0);  /* exact: q is on the grid */
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)frac);
}

static float f16_bits_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1, E = (h >> 10) & 31, frac = h & 1023;
    double v;
    if (E == 0) v = ldexp((double)frac, -24);
    else if (E == 31) v = frac ? NAN : INFINITY;
    else v = ldexp(1.0 + frac / 1024.0, E - 15);
    return (float)(sign ? -v : v);
}

static int is_hp_row(int i, int n_hp, const int32_t *hp_idx)
{
    for (int t = 0; t < n_hp; t++)
        if (hp_idx[t] == i) return 1;
    return 0;
}

/* ======================================================================
 * c6 (split): the DAMP layout of one tile.  Rows listed in hp_idx are
 * stored as fp16; the remaining rows (in ascending row order) are INT8
 * with value-column scales taken over those rows only, and no smoothing
 * (s = 1), following the same per-column steps as the layout-0 codec.
 * Qc holds (dk - n_hp) x dv codes; hp_rows holds n_hp x dv fp16 values in
 * the order of hp_idx.
 * ==================================================================== */
static void quantize_tile_damp(int dk, int dv, int n_hp, const int32_t *hp_idx, const float *X,
                               int8_t *Qc, float *c, uint16_t *hp_rows)
{
    for (int t = 0; t < n_hp; t++)
        for (int j = 0; j < dv; j++)
            hp_rows[t * dv + j] = f32_to_f16_bits(X[hp_idx[t] * dv + j]);
    for (int j = 0; j < dv; j++) {
        float m = 0.0f;
        for (int i = 0; i < dk; i++) {
            if (is_hp_row(i, n_hp, hp_idx)) continue;
            float a = fabsf(X[i * dv + j]);
            if (a > m) m = a;
        }
        float cj = 0.0f, iota = 0.0f;
        if (m > 0.0f) {
            iota = f32_div(127.0f, m);
            if (isinf(iota)) iota = 0.0f;
            else cj = f32_div(m, 127.0f);
        }
        c[j] = cj;
        int row = 0;
        for (int i = 0; i < dk; i++) {
            if (is_hp_row(i, n_hp, hp_idx)) continue;
            double qv = round_half_even((double)X[i * dv + j] * (double)iota);
            if (qv > 127.0) qv = 127.0;
            if (qv < -127.0) qv = -127.0;
            Qc[row * dv + j] = (int8_t)qv;
            row++;
        }
    }
}

static void dequantize_tile_damp(int dk, int dv, int n_hp, const int32_t *hp_idx, const int8_t *Qc,
                                 const float *c, const uint16_t *hp_rows, float *X)
{
    int row = 0;
    for (int i = 0; i < dk; i++) {
        int slot = -1;
        for (int t = 0; t < n_hp; t++)
            if (hp_idx[t] == i) slot = t;
        if (slot >= 0) {
            for (int j = 0; j < dv; j++) X[i * dv + j] = f16_bits_to_f32(hp_rows[slot * dv + j]);
        } else {
            for (int j = 0; j < dv; j++) X[i * dv + j] = f32_mul((float)Qc[row * dv + j], c[j]);
            row++;
        }
    }
}

/* ======================================================================
 * c1: one step of the unquantized recurrence on a fp64 state.
 * [LINQ] Table 3, Gated DeltaNet and KDA rows, in the dk x dv orientation.
 * kda = 0: a is one scalar (a[0]); kda = 1: a has dk entries, diag(a)
 * scales key row i by a_i.  o may be NULL.  u (dv) may be NULL.
 * ==================================================================== */
static void recur_step(int dk, int dv, int kda, double *S, const float *q, const float *k,
                       const float *v, const float *a, float b, double *o, double *u_out)
{
    for (int i = 0; i < dk; i++) {                       /* S' = a S or diag(a) S */
        double ai = kda ? (double)a[i] : (double)a[0];
        for (int j = 0; j < dv; j++) S[i * dv + j] *= ai;
    }
    double *u = (double *)malloc(sizeof(double) * dv);
    for (int j = 0; j < dv; j++) {                       /* w = S'^T k           */
        double w = 0.0;
        for (int i = 0; i < dk; i++) w += S[i * dv + j] * (double)k[i];
        u[j] = (double)b * ((double)v[j] - w);           /* u = b (v - w)        */
    }
    for (int i = 0; i < dk; i++)                         /* S = S' + k u^T       */
        for (int j = 0; j < dv; j++) S[i * dv + j] += (double)k[i] * u[j];
    if (o) {
        for (int j = 0; j < dv; j++) {                   /* o = S^T q            */
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += S[i * dv + j] * (double)q[i];
            o[j] = acc;
        }
    }
    if (u_out) memcpy(u_out, u, sizeof(double) * dv);
    free(u);
}

/* ======================================================================
 * Exported entry points.  Arrays are contiguous, row-major, head-major:
 * a "head" is one (batch, head) state.  Per-step inputs are laid out
 * [step][head][...] .  a has 1 (GDN) or dk (KDA) entries per head-step.
 * ==================================================================== */

/* c2 / layout 0 over nh heads, b-bit codes (unpacked, one int8 each) */
void orc_quantize(int nh, int dk, int dv, int bits, const float *X, int8_t *Q, float *s, float *c)
{
    size_t E = (size_t)dk * dv;
    for (int h = 0; h < nh; h++)
        quantize_tile(dk, dv, code_qmax(bits), X + h * E, Q + h * E, s + (size_t)h * dk,
                      c + (size_t)h * dv);
}

/* n_rows rows of dv codes: unpacked int8 <-> the packed layout above */
void orc_pack_codes(int n_rows, int dv, int bits, const int8_t *Q, uint8_t *P)
{
    size_t nb = (size_t)dv * bits / 8;
    for (int r = 0; r < n_rows; r++) pack_row(dv, bits, Q + (size_t)r * dv, P + r * nb);
}

void orc_unpack_codes(int n_rows, int dv, int bits, const uint8_t *P, int8_t *Q)
{
    size_t nb = (size_t)dv * bits / 8;
    for (int r = 0; r < n_rows; r++) unpack_row(dv, bits, P + r * nb, Q + (size_t)r * dv);
}

void orc_dequantize(int nh, int dk, int dv, const int8_t *Q, const float *s, const float *c, float *X)
{
    size_t E = (size_t)dk * dv;
    for (int h = 0; h < nh; h++)
        dequantize_tile(dk, dv, Q + h * E, s + (size_t)h * dk, c + (size_t)h * dv, X + h * E);
}

/* c6 split over nh heads; hp_idx is [nh][n_hp], Qc [nh][dk-n_hp][dv] */
void orc_quantize_damp(int nh, int dk, int dv, int n_hp, const int32_t *hp_idx, const float *X,
                       int8_t *Qc, float *c, uint16_t *hp_rows)
{
    size_t E = (size_t)dk * dv, Ec = (size_t)(dk - n_hp) * dv, Eh = (size_t)n_hp * dv;
    for (int h = 0; h < nh; h++)
        quantize_tile_damp(dk, dv, n_hp, hp_idx + (size_t)h * n_hp, X + h * E, Qc + h * Ec,
                           c + (size_t)h * dv, hp_rows + h * Eh);
}

void orc_dequantize_damp(int nh, int dk, int dv, int n_hp, const int32_t *hp_idx, const int8_t *Qc,
                         const float *c, const uint16_t *hp_rows, float *X)
{
    size_t E = (size_t)dk * dv, Ec = (size_t)(dk - n_hp) * dv, Eh = (size_t)n_hp * dv;
    for (int h = 0; h < nh; h++)
        dequantize_tile_damp(dk, dv, n_hp, hp_idx + (size_t)h * n_hp, Qc + h * Ec,
                             c + (size_t)h * dv, hp_rows + h * Eh, X + h * E);
}

void orc_f32_to_f16(int n, const float *x, uint16_t *h)
{
    for (int t = 0; t < n; t++) h[t] = f32_to_f16_bits(x[t]);
}

void orc_f16_to_f32(int n, const uint16_t *h, float *x)
{
    for (int t = 0; t < n; t++) x[t] = f16_bits_to_f32(h[t]);
}

/* c1 over n steps and nh heads.  S: fp64 [nh][dk][dv], updated in place.
 * o: [n][nh][dv] (may be NULL).  u: [n][nh][dv] (may be NULL). */
void orc_recur(int nh, int dk, int dv, int kda, int n, double *S, const float *q, const float *k,
               const float *v, const float *a, const float *b, double *o, double *u)
{
    size_t E = (size_t)dk * dv;
    int na = kda ? dk : 1;
    for (int t = 0; t < n; t++)
        for (int h = 0; h < nh; h++) {
            size_t hs = (size_t)t * nh + h;
            recur_step(dk, dv, kda, S + h * E, q ? q + hs * dk : k + hs * dk, k + hs * dk,
                       v + hs * dv, a + hs * na, b[hs], o ? o + hs * dv : NULL,
                       u ? u + hs * dv : NULL);
        }
}

/* ======================================================================
 * c3: per-step quantized decode (window of one token, no compensators).
 * [LEAP] opening paragraphs: per token the layer loads the state, applies
 * a light update and writes it back.  Steps: X = D(Q); one c1 step in
 * fp64; o from the fp64 updated state (before requantization); round the
 * state to fp32; requantize with the layout-0 codec; store in place.
 * S_pre (nullable) receives the fp64 updated state, S_f32 (nullable) the
 * fp32 tensor handed to the codec.
 * ==================================================================== */
void orc_quant_step(int nh, int dk, int dv, int kda, int bits, int8_t *Q, float *s, float *c,
                    const float *q, const float *k, const float *v, const float *a, const float *b,
                    double *o, double *S_pre, float *S_f32)
{
    size_t E = (size_t)dk * dv;
    int na = kda ? dk : 1;
    float *X = (float *)malloc(sizeof(float) * E);
    double *S = (double *)malloc(sizeof(double) * E);
    for (int h = 0; h < nh; h++) {
        int8_t *Qh = Q + h * E;
        float *sh = s + (size_t)h * dk, *ch = c + (size_t)h * dv;
        dequantize_tile(dk, dv, Qh, sh, ch, X);
        for (size_t e = 0; e < E; e++) S[e] = (double)X[e];
        recur_step(dk, dv, kda, S, q + (size_t)h * dk, k + (size_t)h * dk, v + (size_t)h * dv,
                   a + (size_t)h * na, b[h], o + (size_t)h * dv, NULL);
        if (S_pre) memcpy(S_pre + h * E, S, sizeof(double) * E);
        for (size_t e = 0; e < E; e++) X[e] = (float)S[e];
        if (S_f32) memcpy(S_f32 + h * E, X, sizeof(float) * E);
        quantize_tile(dk, dv, code_qmax(bits), X, Qh, sh, ch);
    }
    free(X);
    free(S);
}

/* ======================================================================
 * The fixed state at a window start, in fp64:
 *   X_0 = D(Q) + sum_c p_c w_c^T
 * layout 0: D(Q) from (Q, s, c); layout 1: DAMP rows (Qc, c, hp rows).
 * [LEAP] Compensator Tokens paragraph: each is an outer product of two
 * high-precision vectors that is removed before quantization and added
 * back on the update path.
 * p: [nh][r][dk], w: [nh][r][dv].
 * ==================================================================== */
void orc_state_base(int nh, int dk, int dv, int r, int layout, int n_hp, const int8_t *Q,
                    const float *s, const float *c, const int32_t *hp_idx, const uint16_t *hp_rows,
                    const float *p, const float *w, double *X0)
{
    size_t E = (size_t)dk * dv;
    float *X = (float *)malloc(sizeof(float) * E);
    for (int h = 0; h < nh; h++) {
        if (layout == 0)
            dequantize_tile(dk, dv, Q + h * E, s + (size_t)h * dk, c + (size_t)h * dv, X);
        else
            dequantize_tile_damp(dk, dv, n_hp, hp_idx + (size_t)h * n_hp,
                                 Q + h * (size_t)(dk - n_hp) * dv, c + (size_t)h * dv,
                                 hp_rows + h * (size_t)n_hp * dv, X);
        double *Xh = X0 + h * E;
        for (size_t e = 0; e < E; e++) Xh[e] = (double)X[e];
        for (int cc = 0; cc < r; cc++) {
            const float *pc = p + ((size_t)h * r + cc) * dk;
            const float *wc = w + ((size_t)h * r + cc) * dv;
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++) Xh[i * dv + j] += (double)pc[i] * (double)wc[j];
        }
    }
    free(X);
}

/* cumulative decay from after token `from` through token `to` (1-based),
 * prod_{from < j <= to} a_j, for key channel i; the empty product is 1. */
static double decay_ratio(int kda, int dk, int nh, int h, const float *a, int from, int to, int i)
{
    int na = kda ? dk : 1;
    double g = 1.0;
    for (int j = from + 1; j <= to; j++) {
        const float *aj = a + ((size_t)(j - 1) * nh + h) * na;
        g *= kda ? (double)aj[i] : (double)aj[0];
    }
    return g;
}

/* ======================================================================
 * c4 + the rebuild half of c5: per-window decode.
 * [LEAP] per-window quantization paragraph: the low-precision state is
 * held fixed for the window, higher-precision token updates are
 * buffered, every output is computed from the fixed state plus the
 * buffer, and the full state is rebuilt only at the window end.
 *
 * For token t = 1..n of the window (G_t = a_1 ... a_t per key channel):
 *   retrieval_t = X_0^T (G_t . k_t) + sum_{i<t} u_i ((G_t/G_i) . k_i)^T k_t
 *   u_t = b_t (v_t - retrieval_t)
 *   o_t = X_0^T (G_t . q_t) + sum_{i<=t} u_i ((G_t/G_i) . k_i)^T q_t
 * G_t/G_i is the direct product of the gates after token i.  These are the
 * sequential recurrence from X_0 unrolled; diag(a_t) diag(G_{t-1}) = diag(G_t).
 * At the end: S_W = diag(G_n) X_0 + sum_i ((G_n/G_i) . k_i) u_i^T.
 * X0: fp64 [nh][dk][dv]; inputs [n][nh][..]; o, u: [n][nh][dv]; SW: [nh][dk][dv].
 * ==================================================================== */
void orc_window(int nh, int dk, int dv, int kda, int n, const double *X0, const float *q,
                const float *k, const float *v, const float *a, const float *b, double *o,
                double *u, double *SW)
{
    size_t E = (size_t)dk * dv;
    double *gk = (double *)malloc(sizeof(double) * dk);
    double *gq = (double *)malloc(sizeof(double) * dk);
    for (int h = 0; h < nh; h++) {
        const double *X = X0 + h * E;
        for (int t = 1; t <= n; t++) {
            size_t hs = (size_t)(t - 1) * nh + h;
            const float *kt = k + hs * dk, *qt = q + hs * dk, *vt = v + hs * dv;
            for (int i = 0; i < dk; i++) {
                double g = decay_ratio(kda, dk, nh, h, a, 0, t, i);
                gk[i] = g * (double)kt[i];
                gq[i] = g * (double)qt[i];
            }
            double *ut = u + hs * dv, *ot = o + hs * dv;
            for (int j = 0; j < dv; j++) {
                double ret = 0.0, out = 0.0;
                for (int i = 0; i < dk; i++) {
                    ret += X[i * dv + j] * gk[i];
                    out += X[i * dv + j] * gq[i];
                }
                ut[j] = ret;                           /* fixed-state part for now */
                ot[j] = out;
            }
            for (int ii = 1; ii < t; ii++) {           /* buffered tokens i < t */
                size_t hi = (size_t)(ii - 1) * nh + h;
                const float *ki = k + hi * dk;
                double alpha = 0.0, beta = 0.0;
                for (int i = 0; i < dk; i++) {
                    double kr = decay_ratio(kda, dk, nh, h, a, ii, t, i) * (double)ki[i];
                    alpha += kr * (double)kt[i];
                    beta += kr * (double)qt[i];
                }
                const double *ui = u + hi * dv;
                for (int j = 0; j < dv; j++) {
                    ut[j] += alpha * ui[j];
                    ot[j] += beta * ui[j];
                }
            }
            for (int j = 0; j < dv; j++) ut[j] = (double)b[hs] * ((double)vt[j] - ut[j]);
            double kq = 0.0;                           /* token t itself: G_t/G_t = 1 */
            for (int i = 0; i < dk; i++) kq += (double)kt[i] * (double)qt[i];
            for (int j = 0; j < dv; j++) ot[j] += kq * ut[j];
        }
        if (SW) {                                      /* rebuild at the window end */
            double *S = SW + h * E;
            for (int i = 0; i < dk; i++) {
                double g = decay_ratio(kda, dk, nh, h, a, 0, n, i);
                for (int j = 0; j < dv; j++) S[i * dv + j] = g * X[i * dv + j];
            }
            for (int ii = 1; ii <= n; ii++) {
                size_t hi = (size_t)(ii - 1) * nh + h;
                const float *ki = k + hi * dk;
                const double *ui = u + hi * dv;
                for (int i = 0; i < dk; i++) {
                    double kr = decay_ratio(kda, dk, nh, h, a, ii, n, i) * (double)ki[i];
                    for (int j = 0; j < dv; j++) S[i * dv + j] += kr * ui[j];
                }
            }
        }
    }
    free(gk);
    free(gq);
}

/* ======================================================================
 * c5 (compress half): Compensator Tokens + residual + codec.
 * [LEAP] Compensator Tokens and residual-smoothing paragraphs.
 * Input: the rebuilt fp64 state S_W of each head.  For c = 1..r:
 *   v <- 1/sqrt(dv) (all entries); repeat `iters` times:
 *     y <- R^T (R v); if |y| = 0: on the first step, restart from the unit
 *     vector of R's largest column (lowest index on ties) when R != 0,
 *     otherwise stop; v <- y / |y|.
 *   p_c = fp32(R v), w_c = fp32(v); R <- R - p_c w_c^T (stored fp32 pair).
 * R == 0 gives p_c = w_c = 0.  The residual is rounded to fp32 (R_out),
 * then coded by layout 0 (Q, s, c) or the DAMP split (Q, c, hp_rows).
 * p: [nh][r][dk], w: [nh][r][dv], R_out (nullable): fp32 [nh][dk][dv].
 * ==================================================================== */
void orc_compress(int nh, int dk, int dv, int r, int iters, int layout, int n_hp, int bits,
                  const int32_t *hp_idx, const double *SW, int8_t *Q, float *s, float *c,
                  uint16_t *hp_rows, float *p, float *w, float *R_out)
{
    size_t E = (size_t)dk * dv;
    double *R = (double *)malloc(sizeof(double) * E);
    double *vv = (double *)malloc(sizeof(double) * dv);
    double *x = (double *)malloc(sizeof(double) * dk);
    double *y = (double *)malloc(sizeof(double) * dv);
    float *Rf = (float *)malloc(sizeof(float) * E);
    for (int h = 0; h < nh; h++) {
        memcpy(R, SW + h * E, sizeof(double) * E);
        for (int cc = 0; cc < r; cc++) {
            float *pc = p + ((size_t)h * r + cc) * dk;
            float *wc = w + ((size_t)h * r + cc) * dv;
            int nonzero = 0;
            for (size_t e = 0; e < E; e++)
                if (R[e] != 0.0) nonzero = 1;
            if (!nonzero) {                             /* zero compensator */
                for (int i = 0; i < dk; i++) pc[i] = 0.0f;
                for (int j = 0; j < dv; j++) wc[j] = 0.0f;
                continue;
            }
            for (int j = 0; j < dv; j++) vv[j] = 1.0 / sqrt((double)dv);
            int restarted = 0;
            for (int it = 0; it < iters; it++) {
                for (int i = 0; i < dk; i++) {          /* x = R v   */
                    double acc = 0.0;
                    for (int j = 0; j < dv; j++) acc += R[i * dv + j] * vv[j];
                    x[i] = acc;
                }
                double n2 = 0.0;
                for (int j = 0; j < dv; j++) {          /* y = R^T x */
                    double acc = 0.0;
                    for (int i = 0; i < dk; i++) acc += R[i * dv + j] * x[i];
                    y[j] = acc;
                    n2 += acc * acc;
                }
                if (n2 == 0.0) {
                    if (it > 0 || restarted) break;     /* keep the current v */
                    int jbest = 0;                      /* largest column of R */
                    double best = -1.0;
                    for (int j = 0; j < dv; j++) {
                        double cn = 0.0;
                        for (int i = 0; i < dk; i++) cn += R[i * dv + j] * R[i * dv + j];
                        if (cn > best) { best = cn; jbest = j; }
                    }
                    for (int j = 0; j < dv; j++) vv[j] = (j == jbest) ? 1.0 : 0.0;
                    restarted = 1;
                    it = -1;                            /* restart the full count */
                    continue;
                }
                double nrm = sqrt(n2);
                for (int j = 0; j < dv; j++) vv[j] = y[j] / nrm;
            }
            for (int i = 0; i < dk; i++) {              /* p = R v  */
                double acc = 0.0;
                for (int j = 0; j < dv; j++) acc += R[i * dv + j] * vv[j];
                pc[i] = (float)acc;
            }
            for (int j = 0; j < dv; j++) wc[j] = (float)vv[j];
            for (int i = 0; i < dk; i++)                /* deflate with the stored pair */
                for (int j = 0; j < dv; j++) R[i * dv + j] -= (double)pc[i] * (double)wc[j];
        }
        for (size_t e = 0; e < E; e++) Rf[e] = (float)R[e];
        if (R_out) memcpy(R_out + h * E, Rf, sizeof(float) * E);
        if (layout == 0)
            quantize_tile(dk, dv, code_qmax(bits), Rf, Q + h * E, s + (size_t)h * dk,
                          c + (size_t)h * dv);
        else
            quantize_tile_damp(dk, dv, n_hp, hp_idx + (size_t)h * n_hp, Rf,
                               Q + h * (size_t)(dk - n_hp) * dv, c + (size_t)h * dv,
                               hp_rows + h * (size_t)n_hp * dv);
    }
    free(R);
    free(vv);
    free(x);
    free(y);
    free(Rf);
}

/* ======================================================================
 * c6 (calibration): pick the high-precision key rows of each head.
 * [DAMP] abstract: channels are scored offline by quantization-error
 * energy and by decay-based persistence.  Reading taken:
 *   run n_steps of the recurrence from S0 (fp32 [nh][dk][dv]);
 *   after each step quantize the fp32-rounded state with value-column
 *   scales over all rows and no smoothing; E_i += sum_j (S_ij - D_ij)^2;
 *   abar_i = mean over steps of the key-channel gate a_i;
 *   score_i = E_i / max(1 - abar_i, 1e-6);
 *   keep the n_hp largest scores (lower index first on ties), listed in
 *   ascending row order.
 * hp_idx: [nh][n_hp]; score (nullable): fp64 [nh][dk].
 * ==================================================================== */
void orc_calibrate(int nh, int dk, int dv, int kda, int n_steps, int n_hp, const float *S0,
                   const float *k, const float *v, const float *a, const float *b,
                   int32_t *hp_idx, double *score)
{
    size_t E = (size_t)dk * dv;
    int na = kda ? dk : 1;
    double *S = (double *)malloc(sizeof(double) * E);
    float *X = (float *)malloc(sizeof(float) * E);
    int8_t *Qc = (int8_t *)malloc(E);
    float *cc = (float *)malloc(sizeof(float) * dv);
    double *En = (double *)malloc(sizeof(double) * dk);
    double *Ab = (double *)malloc(sizeof(double) * dk);
    double *sc = (double *)malloc(sizeof(double) * dk);
    int *taken = (int *)malloc(sizeof(int) * dk);
    for (int h = 0; h < nh; h++) {
        for (size_t e = 0; e < E; e++) S[e] = (double)S0[h * E + e];
        for (int i = 0; i < dk; i++) { En[i] = 0.0; Ab[i] = 0.0; }
        for (int t = 0; t < n_steps; t++) {
            size_t hs = (size_t)t * nh + h;
            const float *at = a + hs * na;
            recur_step(dk, dv, kda, S, NULL, k + hs * dk, v + hs * dv, at, b[hs], NULL, NULL);
            for (size_t e = 0; e < E; e++) X[e] = (float)S[e];
            quantize_tile_damp(dk, dv, 0, NULL, X, Qc, cc, NULL);
            for (int i = 0; i < dk; i++) {
                for (int j = 0; j < dv; j++) {
                    double d = S[i * dv + j] - (double)f32_mul((float)Qc[i * dv + j], cc[j]);
                    En[i] += d * d;
                }
                Ab[i] += kda ? (double)at[i] : (double)at[0];
            }
        }
        for (int i = 0; i < dk; i++) {
            double abar = Ab[i] / (double)n_steps;
            double den = 1.0 - abar;
            if (den < 1e-6) den = 1e-6;
            sc[i] = En[i] / den;
            taken[i] = 0;
            if (score) score[(size_t)h * dk + i] = sc[i];
        }
        int32_t *out = hp_idx + (size_t)h * n_hp;
        for (int t = 0; t < n_hp; t++) {                /* repeated arg-max */
            int best = -1;
            for (int i = 0; i < dk; i++) {
                if (taken[i]) continue;
                if (best < 0 || sc[i] > sc[best]) best = i;
            }
            taken[best] = 1;
        }
        int n = 0;
        for (int i = 0; i < dk; i++)
            if (taken[i]) out[n++] = i;
    }
    free(S);
    free(X);
    free(Qc);
    free(cc);
    free(En);
    free(Ab);
    free(sc);
    free(taken);
}

/* ======================================================================
 * f4: static scales.  [STEP] (opening section): key-row and value-column
 * scales are fitted jointly and offline, from the state distribution and
 * from each key row's impact on the output error; precision follows the
 * error's size and how long it persists.  The page gives no formula.
 * Reading taken:
 *  - a head's stored parameters are s (dk), rho = 1/s (dk), c (dv) and
 *    iota (dv), with c_j = mc_j / Qb and iota_j = Qb / mc_j for a column
 *    range mc_j (zero column: c = iota = 0);
 *  - codes of a state X under fixed parameters: Y_ij = X_ij rho_i (one fp32
 *    product), Q_ij = the integer nearest to the exact product Y_ij iota_j
 *    (ties to even), clamped to [-Qb, Qb]; dequantization as in c2;
 *  - the fit runs n steps of the recurrence from S0 and takes the fp32
 *    state after each step as a calibration state X_t:
 *      s_i   = sqrt(max_t max_j |X_t,ij|), rho_i = 1/s_i (0 for a zero row);
 *      m_j   = max_t max_i |X_t,ij rho_i|;
 *      candidate ranges mc_j(k) = m_j (16-k)/16, k = 0..8 (one fp32 product);
 *      omega_i = (mean_t q_t,i^2) / max(1 - abar_i, 1e-6): the weight of key
 *      row i in the output o = S^T q times the lifetime of an error in that
 *      row under its gate (abar_i = mean gate of key channel i);
 *      E_j(k) = sum_t sum_i omega_i (X_t,ij - D_t,ij(k))^2 with the codes
 *      and dequantized values of column j under candidate k;
 *      keep the candidate with the least E_j (smallest k on ties).
 * ==================================================================== */
static void quantize_tile_static(int dk, int dv, int qmax, const float *X, const float *rho,
                                 const float *iota, int8_t *Q)
{
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) {
            float Y = f32_mul(X[i * dv + j], rho[i]);                 /* Y_ij = X_ij rho_i */
            double qv = round_half_even((double)Y * (double)iota[j]); /* exact product    */
            if (qv > qmax) qv = qmax;
            if (qv < -qmax) qv = -qmax;
            Q[i * dv + j] = (int8_t)qv;
        }
}

/* codes of nh tiles X [nh][dk][dv] under fixed rho [nh][dk], iota [nh][dv] */
void orc_quantize_static(int nh, int dk, int dv, int bits, const float *X, const float *rho, const float *iota,
                         int8_t *Q)
{
    size_t E = (size_t)dk * dv;
    for (int h = 0; h < nh; h++)
        quantize_tile_static(dk, dv, code_qmax(bits), X + h * E, rho + (size_t)h * dk, iota + (size_t)h * dv,
                             Q + h * E);
}

/* Fit of the reading above.  q, k: [n][nh][dk], v: [n][nh][dv], a: [n][nh][1|dk],
 * b: [n][nh].  Outputs per head: s, rho [nh][dk]; c, iota [nh][dv]; choice
 * [nh][dv] (the chosen k); err (nullable) [nh][9][dv] the E_j(k); cand_c and
 * cand_iota (nullable) [nh][9][dv] the candidates' scales. */
void orc_fit_static(int nh, int dk, int dv, int kda, int bits, int n, const float *S0, const float *q,
                    const float *k, const float *v, const float *a, const float *b, float *s, float *rho,
                    float *c, float *iota, int32_t *choice, double *err, float *cand_c, float *cand_iota)
{
    size_t E = (size_t)dk * dv;
    int na = kda ? dk : 1;
    const int qmax = code_qmax(bits);
    const float qm = (float)qmax;
    double *S = (double *)malloc(sizeof(double) * E);
    float *X = (float *)malloc(sizeof(float) * E);
    double *om = (double *)malloc(sizeof(double) * dk);
    double *Ej = (double *)malloc(sizeof(double) * 9 * dv);
    float *cc = (float *)malloc(sizeof(float) * 9 * dv);
    float *ci = (float *)malloc(sizeof(float) * 9 * dv);
    for (int h = 0; h < nh; h++) {
        float *sh = s + (size_t)h * dk, *rh = rho + (size_t)h * dk;
        float *ch = c + (size_t)h * dv, *ih = iota + (size_t)h * dv;
        /* pass 1: row maxima, output weights and gate means */
        for (int i = 0; i < dk; i++) { sh[i] = 0.0f; om[i] = 0.0; }
        double *ab = (double *)calloc((size_t)dk, sizeof(double));
        for (size_t e = 0; e < E; e++) S[e] = (double)S0[h * E + e];
        for (int t = 0; t < n; t++) {
            size_t hs = (size_t)t * nh + h;
            recur_step(dk, dv, kda, S, NULL, k + hs * dk, v + hs * dv, a + hs * na, b[hs], NULL, NULL);
            for (int i = 0; i < dk; i++) {
                for (int j = 0; j < dv; j++) {
                    float x = fabsf((float)S[i * dv + j]);
                    if (x > sh[i]) sh[i] = x;        /* sh holds the running max */
                }
                double qi = (double)q[hs * dk + i];
                om[i] += qi * qi;
                ab[i] += kda ? (double)a[hs * na + i] : (double)a[hs * na];
            }
        }
        for (int i = 0; i < dk; i++) {
            float r = sh[i];
            sh[i] = (r > 0.0f) ? f32_sqrt(r) : 0.0f;
            rh[i] = (sh[i] > 0.0f) ? f32_div(1.0f, sh[i]) : 0.0f;
            double den = 1.0 - ab[i] / (double)n;
            if (den < 1e-6) den = 1e-6;
            om[i] = (om[i] / (double)n) / den;
        }
        free(ab);
        /* pass 2: column maxima of the smoothed states */
        float *m = (float *)calloc((size_t)dv, sizeof(float));
        for (size_t e = 0; e < E; e++) S[e] = (double)S0[h * E + e];
        for (int t = 0; t < n; t++) {
            size_t hs = (size_t)t * nh + h;
            recur_step(dk, dv, kda, S, NULL, k + hs * dk, v + hs * dv, a + hs * na, b[hs], NULL, NULL);
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++) {
                    float y = fabsf(f32_mul((float)S[i * dv + j], rh[i]));
                    if (y > m[j]) m[j] = y;
                }
        }
        for (int j = 0; j < dv; j++)
            for (int kk = 0; kk < 9; kk++) {
                float mc = f32_mul(m[j], (float)(16 - kk) / 16.0f);
                float cj = 0.0f, io = 0.0f;
                if (mc > 0.0f) {
                    io = f32_div(qm, mc);
                    if (isinf(io)) io = 0.0f;
                    else cj = f32_div(mc, qm);
                }
                cc[kk * dv + j] = cj;
                ci[kk * dv + j] = io;
                Ej[kk * dv + j] = 0.0;
            }
        free(m);
        /* pass 3: weighted error of every candidate */
        for (size_t e = 0; e < E; e++) S[e] = (double)S0[h * E + e];
        for (int t = 0; t < n; t++) {
            size_t hs = (size_t)t * nh + h;
            recur_step(dk, dv, kda, S, NULL, k + hs * dk, v + hs * dv, a + hs * na, b[hs], NULL, NULL);
            for (size_t e = 0; e < E; e++) X[e] = (float)S[e];
            for (int i = 0; i < dk; i++)
                for (int j = 0; j < dv; j++) {
                    float Y = f32_mul(X[i * dv + j], rh[i]);
                    for (int kk = 0; kk < 9; kk++) {
                        double qv = round_half_even((double)Y * (double)ci[kk * dv + j]);
                        if (qv > qmax) qv = qmax;
                        if (qv < -qmax) qv = -qmax;
                        float D = f32_mul(f32_mul((float)qv, cc[kk * dv + j]), sh[i]);
                        double d = (double)X[i * dv + j] - (double)D;
                        Ej[kk * dv + j] += om[i] * d * d;
                    }
                }
        }
        for (int j = 0; j < dv; j++) {
            int best = 0;
            for (int kk = 1; kk < 9; kk++)
                if (Ej[kk * dv + j] < Ej[best * dv + j]) best = kk;
            ch[j] = cc[best * dv + j];
            ih[j] = ci[best * dv + j];
            choice[(size_t)h * dv + j] = best;
        }
        if (err) memcpy(err + (size_t)h * 9 * dv, Ej, sizeof(double) * 9 * dv);
        if (cand_c) memcpy(cand_c + (size_t)h * 9 * dv, cc, sizeof(float) * 9 * dv);
        if (cand_iota) memcpy(cand_iota + (size_t)h * 9 * dv, ci, sizeof(float) * 9 * dv);
    }
    free(S);
    free(X);
    free(om);
    free(Ej);
    free(cc);
    free(ci);
}

/* c3 with static scales: X = D(Q) with the fixed s, c; one c1 step in fp64;
 * o from the updated fp64 state; round to fp32; codes under the fixed rho,
 * iota (s, c, rho, iota unchanged).  S_f32 (nullable) receives the fp32
 * tensor handed to the codec. */
void orc_quant_step_static(int nh, int dk, int dv, int kda, int bits, int8_t *Q, const float *s, const float *c,
                           const float *rho, const float *iota, const float *q, const float *k, const float *v,
                           const float *a, const float *b, double *o, float *S_f32)
{
    size_t E = (size_t)dk * dv;
    int na = kda ? dk : 1;
    float *X = (float *)malloc(sizeof(float) * E);
    double *S = (double *)malloc(sizeof(double) * E);
    for (int h = 0; h < nh; h++) {
        int8_t *Qh = Q + h * E;
        dequantize_tile(dk, dv, Qh, s + (size_t)h * dk, c + (size_t)h * dv, X);
        for (size_t e = 0; e < E; e++) S[e] = (double)X[e];
        recur_step(dk, dv, kda, S, q + (size_t)h * dk, k + (size_t)h * dk, v + (size_t)h * dv,
                   a + (size_t)h * na, b[h], o + (size_t)h * dv, NULL);
        for (size_t e = 0; e < E; e++) X[e] = (float)S[e];
        if (S_f32) memcpy(S_f32 + h * E, X, sizeof(float) * E);
        quantize_tile_static(dk, dv, code_qmax(bits), X, rho + (size_t)h * dk, iota + (size_t)h * dv, Qh);
    }
    free(X);
    free(S);
}
