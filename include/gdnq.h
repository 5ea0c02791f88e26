/*
 * gdnq.h -- C ABI of libgdnq.so: quantized recurrent-state decode for
 * Gated-DeltaNet (GDN) and Kimi-Delta-Attention (KDA) linear-attention
 * layers on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are web pages; the method is given
 * there in prose, the formulas below are the readings this library takes):
 *
 *  - Recurrence ("LinQuant: Functional Invariances for Low-Precision Linear
 *    Recurrences", appendix Table 3, Gated DeltaNet and KDA rows).  The
 *    state of one (batch, head) is S in R^{dk x dv}, key channel i = row,
 *    value channel j = column (the transpose of Table 3's dv x dk form):
 *        S' = a S  (GDN, scalar gate)   or  diag(a) S  (KDA, a in R^dk)
 *        u  = b (v - S'^T k),   S_t = S' + k u^T,   o = S_t^T q.
 *
 *  - Per-token state traffic ("LeapQuant: Efficient Linear Attention with
 *    Accurate Recurrent State Quantization", project page, opening
 *    paragraphs): each token loads the state from HBM, applies a light
 *    update and writes it back; the state is kept in 8 bits here.
 *
 *  - State codec (LeapQuant, residual-smoothing paragraph; STEPQuant page,
 *    key-row and value-column scales).  Layout 0, per head, every step one
 *    IEEE fp32 operation rounded to nearest even, no fused multiply-add:
 *        r_i = max_j |X_ij|,  s_i = sqrt(r_i),  rho_i = 1/s_i,
 *        Y_ij = X_ij rho_i,   m_j = max_i |Y_ij|,
 *        c_j = m_j/127,  iota_j = 127/m_j,  Q_ij = rint_even(Y_ij iota_j)
 *    clamped to [-127, 127] (zero rows/columns: scale 0, code 0; a column
 *    whose 127/m_j overflows fp32 is a zero column).  Dequantized value:
 *        D(Q)_ij = (Q_ij c_j) s_i   (two rounded fp32 products).
 *
 *  - Per-window mode (LeapQuant, per-window quantization paragraph): the
 *    INT8 state of the window start stays fixed for W tokens, each token's
 *    rank-1 update (k_t, u_t) is buffered in fp32, outputs are computed
 *    from the fixed state plus the buffer, and the state is rebuilt and
 *    requantized only at the window end (gdn_quant_window_flush).
 *
 *  - Compensator Tokens (LeapQuant, Compensator Tokens paragraph): before
 *    quantization, r rank-1 terms p_c w_c^T (fp32) are taken out of the
 *    state by `power_iters` steps of power iteration each (start: the
 *    all-equal unit vector; v <- R^T R v / |R^T R v|; p = R v, w = v;
 *    sequential deflation R <- R - p w^T with the stored fp32 pair).  They
 *    are part of the fixed state inside a window and decay with it.
 *
 *  - DAMP rows ("DAMP: Decay-Aware Mixed-Precision Recurrent-State
 *    Quantization", abstract).  Layout 1: n_hp key rows per head, chosen
 *    offline by calibrate_scales, are stored as IEEE fp16 (round to nearest
 *    even, saturating at +-65504); the other rows are INT8 with
 *    value-column scales over those rows only and no row smoothing.
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are caller-allocated, contiguous, 16-byte
 *    aligned device buffers; the library allocates nothing, keeps no state
 *    between calls except a thread-local error string, and is reentrant.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  The library never synchronizes.
 *  - State arrays are updated in place.  q, k, v, a, b, o must not overlap
 *    any state array; overlapping buffers are rejected.
 *  - Return value: GDNQ_OK, or an error code with a message readable from
 *    gdnq_last_error().  Argument errors are found on the host before any
 *    launch, so a failed call has not touched device memory.
 *  - Inputs that are NaN or infinite give undefined results.  Gates must
 *    satisfy 0 < a <= 1 (fp32 subnormal gates included); a window's gate
 *    products may fall below fp32's range: the window buffer keeps each
 *    product as a mantissa and a separate integer exponent.
 *  - bf16 inputs are widened exactly; a bf16 output is rounded to nearest
 *    even from fp32.
 */
#ifndef GDNQ_H
#define GDNQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GDNQ_OK = 0,
    GDNQ_EINVAL = 1,      /* invalid argument (null, misaligned, overlap, range) */
    GDNQ_EUNSUPPORTED = 2,/* shape or mode the library does not implement       */
    GDNQ_ELAUNCH = 3      /* the HIP runtime reported an error at launch        */
};

enum { GDNQ_DECAY_SCALAR = 0, GDNQ_DECAY_CHANNEL = 1 };
enum { GDNQ_IO_F32 = 0, GDNQ_IO_BF16 = 1 };
enum { GDNQ_LAYOUT_ROWCOL = 0, GDNQ_LAYOUT_DAMP = 1 };

/* flags */
#define GDNQ_DEBUG_PREQUANT 1u  /* also store the fp32 tensor the codec consumed */
#define GDNQ_STATIC_SCALES 2u   /* keep fitted static scales (calibrate_static_scales);
                                   per-step mode of layout 0 only */

/* Problem description shared by all calls. */
typedef struct {
    int32_t B, H;         /* batch and heads: B*H independent states           */
    int32_t dk, dv;       /* key / value head dims, each 64 or 128             */
    int32_t W;            /* window length, >= 1                               */
    int32_t r;            /* Compensator Tokens per head, 0..8                 */
    int32_t decay;        /* GDNQ_DECAY_SCALAR or GDNQ_DECAY_CHANNEL           */
    int32_t io_dtype;     /* GDNQ_IO_F32 or GDNQ_IO_BF16 for q, k, v and o     */
    int32_t layout;       /* GDNQ_LAYOUT_ROWCOL or GDNQ_LAYOUT_DAMP            */
    int32_t n_hp;         /* DAMP fp16 rows per head (layout 1), 1..dk/2       */
    int32_t power_iters;  /* power-iteration steps per compensator, 1..64      */
    uint32_t flags;       /* GDNQ_DEBUG_PREQUANT | GDNQ_STATIC_SCALES, or 0    */
    int32_t bits;         /* code width b: 8 (0 also means 8), 6 or 4; layout 1
                             keeps 8-bit codes (DAMP: the rest in INT8)        */
    int32_t hk;           /* key/query heads, dividing H (0 means H): value
                             head hh reads key head hh / (H / hk) of its batch
                             entry; q and k are [B,hk,dk]                      */
} gdnq_desc;

/*
 * Quantized state of B*H heads (all device pointers; NULL where unused).
 * Per-step mode is W == 1 && r == 0; everything else is window mode.
 *   codes       int8   layout 0: [B,H,dk,dv]; layout 1: [B,H,dk-n_hp,dv]
 *                      (the non-DAMP rows in ascending row order); row-major.
 *                      With b = 6 or 4 bits (layout 0) each row of dv
 *                      codes takes dv*b/8 bytes: b = 4: code j in byte
 *                      j/2, bits 4(j%2)..+3, two's complement; b = 6: the
 *                      codes of columns 8k..8k+7 form a 48-bit record
 *                      (column 8k+e in bits 6e..6e+5, two's complement),
 *                      its bits 0..31 in bytes 4k..4k+3 and its bits
 *                      32..47 in bytes dv/2+2k, +1.  Codes lie in [-(2^(b-1)-1),
 *                      2^(b-1)-1] (LeapQuant accuracy table: 8, 6 and 4
 *                      bit states), column scales c = m / (2^(b-1)-1).
 *   row_scale   fp32   [B,H,dk]        layout 0 only (smoothing scales s); with
 *                                      GDNQ_STATIC_SCALES two planes [2][B,H,dk]:
 *                                      s, then rho = 1/s
 *   col_scale   fp32   [B,H,dv]        value-column scales c; with
 *                                      GDNQ_STATIC_SCALES two planes [2][B,H,dv]:
 *                                      c = range/Qb, then iota = Qb/range for
 *                                      the fitted column range
 *   comp_k      fp32   [B,H,r,dk]      compensator key-side vectors p (r > 0)
 *   comp_v      fp32   [B,H,r,dv]      compensator value-side unit vectors w
 *   With G_t the gate product a_1 ... a_t since the window start (one
 *   value per head for the scalar gate, one per key channel for KDA),
 *   written G_t = m_t 2^(e_t) with mantissa m_t in [0.5, 1) and integer
 *   exponent e_t (so no product over- or underflows):
 *   buf_k       fp32   [B,H,W,dk]      window buffer keys k_t / m_t
 *   buf_u       fp32   [B,H,W,dv]      window buffer updates u_t
 *   buf_g       int32  [B,H,W] (scalar) or [B,H,W,dk] (channel): e_t
 *   g_cur       fp32   [B,H] (scalar) or [B,H,dk] (channel): m_t of the
 *                                      last token (1 at a window start)
 *   hp_rows     uint16 [B,H,n_hp,dv]   layout 1: fp16 bit patterns
 *   hp_idx      int32  [B,H,n_hp]      layout 1: row indices, strictly
 *                                      ascending, in [0, dk)
 *   prequant_out fp32  [B,H,dk,dv]     with GDNQ_DEBUG_PREQUANT: the fp32
 *                                      tensor handed to the codec
 * Buffers for window mode (buf_k, buf_u, buf_g, g_cur) are needed when
 * W > 1, r > 0 or layout == GDNQ_LAYOUT_DAMP.
 */
typedef struct {
    int8_t *codes;
    float *row_scale;
    float *col_scale;
    float *comp_k;
    float *comp_v;
    float *buf_k;
    float *buf_u;
    int32_t *buf_g;
    float *g_cur;
    uint16_t *hp_rows;
    int32_t *hp_idx;
    float *prequant_out;
} gdnq_state;

/*
 * One decode token for all B*H heads.
 *   q, k   device, io_dtype, [B,hk,dk] (hk = H unless set); v device, io_dtype, [B,H,dv]
 *   a      device fp32 [B,H] (scalar decay) or [B,H,dk] (channel decay)
 *   b      device fp32 [B,H]
 *   o      device, io_dtype, [B,H,dv]    output o_t = S_t^T q_t
 *   t_in_window: position of this token in the current window, 0..W-1
 *               (all heads move in lockstep; must be 0 in per-step mode).
 * Per-step mode: dequantize, update, emit o from the updated fp32 state,
 * requantize and store codes and scales in place (one fused kernel).
 * Window mode: read the fixed state, compensators and the t_in_window
 * buffered tokens, emit o, append (k_t / m_t, u_t, e_t) to buffer slot
 * t_in_window and store m_t in g_cur; the codes are not written.
 * Per-step mode with layout 1 runs the window step and a one-token flush.
 */
int gdn_quant_decode_step(const gdnq_desc *desc, const gdnq_state *state, const void *q,
                          const void *k, const void *v, const float *a, const float *b,
                          void *o, int32_t t_in_window, void *stream);

/*
 * Window end: rebuild S_W = diag(G) (D(Q) + sum_c p_c w_c^T) +
 * sum_{t<n} ((G/G_t) . k_t) u_t^T from the first n_tokens buffer slots
 * (fp32 MFMA rank-(n+r) product; G = G_n, each ratio G/G_t formed as
 * (m_n / m_t) 2^(e_n - e_t)), take r new Compensator Tokens out of it,
 * requantize the residual, store codes, scales and compensators, and reset
 * g_cur to 1.  n_tokens in 1..W; n_tokens < W gives a self-contained
 * snapshot of a partial window.  In per-step mode this is a no-op.
 */
int gdn_quant_window_flush(const gdnq_desc *desc, const gdnq_state *state, int32_t n_tokens,
                           void *stream);

/*
 * Serving pool form of the decode step and the flush, for engines that keep
 * the states of many requests or cached prefixes in one pool (LeapQuant
 * project page, opening paragraphs: one recurrent state per cached prefix).
 * The state arrays hold n_slots*H heads, sized as for a descriptor with
 * B = n_slots; the call serves desc->B batch entries.  Entry b (0 <= b < B)
 * uses pool slot slots[b] (device int32 [B]): state head slots[b]*H + hh,
 * while q, k, v, a, b and o keep the [B,...] layout of the plain call.
 *   t_pos     device int32 [B]: window position of each entry, 0..W-1
 *             (window mode; entries may sit at different positions; NULL
 *             in per-step mode).
 *   n_tokens  device int32 [B]: tokens to flush for each entry, 1..W; 0
 *             leaves the entry untouched (so one call can flush the
 *             entries that reached their window end).
 * An entry whose slot is outside [0, n_slots), or whose position or token
 * count is outside its range, is skipped on the device (nothing read or
 * written for it).  Slots of one call must be distinct: two entries on one
 * slot race.  The plain calls are the case slots[b] = b, t_pos[b] = t.
 */
int gdn_quant_decode_step_pool(const gdnq_desc *desc, const gdnq_state *state, int32_t n_slots,
                               const int32_t *slots, const int32_t *t_pos, const void *q,
                               const void *k, const void *v, const float *a, const float *b,
                               void *o, void *stream);
int gdn_quant_window_flush_pool(const gdnq_desc *desc, const gdnq_state *state, int32_t n_slots,
                                const int32_t *slots, const int32_t *n_tokens, void *stream);

/*
 * Encode fp32 states S [B,H,dk,dv] (device): r compensators, then the
 * residual through the codec of desc->layout (layout 1 reads
 * state->hp_idx).  Writes codes, scales, compensators; sets g_cur to 1
 * when given.  This is the back half of the flush.
 * Defining passages: LeapQuant project page, residual-smoothing paragraph
 * (key rows balanced by their smoothing scales before the low-bit codes)
 * and Compensator Tokens paragraph (high-precision rank-1 terms taken out
 * first); STEPQuant page (key-row and value-column scales); DAMP abstract
 * (layout 1).  The codec's steps are the ones listed at the top of this
 * header.  Errors: GDNQ_EINVAL for a NULL, misaligned or overlapping
 * buffer; S is read only.
 */
int gdn_state_quantize(const gdnq_desc *desc, const float *S, const gdnq_state *state,
                       void *stream);

/*
 * Decode the stored state: S_out [B,H,dk,dv] fp32 (device) =
 * D(Q) + sum_c p_c w_c^T, i.e. the fixed state of the window start
 * (LeapQuant project page, per-window quantization paragraph: the
 * low-bit state the window's outputs are computed from; residual-smoothing
 * and Compensator Tokens paragraphs for its parts).  D(Q)_ij = (Q_ij c_j)
 * s_i (layout 0) or Q_ij c_j and the fp16 rows (layout 1).  Only the
 * state arrays are read; S_out must not overlap them.
 */
int gdn_state_dequantize(const gdnq_desc *desc, const gdnq_state *state, float *S_out,
                         void *stream);

/*
 * DAMP calibration (DAMP abstract: error energy and decay persistence
 * pick the high-risk channels offline).  Runs n_steps of the fp32
 * recurrence from S0 [B,H,dk,dv]; after each step quantizes every head
 * with value-column scales over all rows and no smoothing and accumulates
 * E_i = sum_t sum_j (S_ij - D_ij)^2; abar_i = mean gate of key channel i;
 * score_i = E_i / max(1 - abar_i, 1e-6).  Writes the n_hp highest-scoring
 * rows per head (lower index first on ties), ascending, to hp_idx_out
 * [B,H,n_hp] int32, and the scores to row_score_out [B,H,dk] fp32 when
 * not NULL.  k: io_dtype [n_steps,B,hk,dk], v: io_dtype [n_steps,B,H,dv]; a fp32 [n_steps,B,H] or
 * [n_steps,B,H,dk]; b fp32 [n_steps,B,H].  All device pointers.
 */
int calibrate_scales(const gdnq_desc *desc, const float *S0, const void *k, const void *v,
                     const float *a, const float *b, int32_t n_steps, int32_t *hp_idx_out,
                     float *row_score_out, void *stream);

/*
 * Static scales (STEPQuant page, opening section: key-row and value-column
 * scales fitted jointly and offline from the state distribution and each key
 * row's impact on the output error; no formula is given, the reading here is
 * the library's).  Needs desc->flags & GDNQ_STATIC_SCALES (per-step mode,
 * layout 0).  Runs n_steps of the fp32 recurrence from S0 [B,H,dk,dv] three
 * times over the calibration inputs q, k (io_dtype [n_steps,B,hk,dk]), v
 * (io_dtype [n_steps,B,H,dv]), a (fp32 [n_steps,B,H] or [n_steps,B,H,dk]), b
 * (fp32 [n_steps,B,H]), all device pointers, and writes both planes of
 * state->row_scale and state->col_scale:
 *   s_i = sqrt(max_t max_j |S_t,ij|), rho_i = 1/s_i;
 *   m_j = max_t max_i |S_t,ij rho_i|; candidate ranges m_j (16-k)/16,
 *   k = 0..8, each with c = range/Qb and iota = Qb/range;
 *   omega_i = (mean_t q_t,i^2) / max(1 - mean_t a_t,i, 1e-6);
 *   E_j(k) = sum_t sum_i omega_i (S_t,ij - D_t,ij(k))^2 with
 *   D = (Q c) s, Q = clamp(rint((S rho) iota), -Qb, Qb); the candidate with
 *   the least E_j is kept (smallest k on ties).
 * With the flag set, gdn_quant_decode_step (and its pool form) and
 * gdn_state_quantize store codes under these fixed scales (the integer
 * nearest to the exact product (x rho_i) iota_j, clamped to [-Qb, Qb]) and
 * leave every scale unchanged; gdn_state_dequantize reads the first planes.
 */
int calibrate_static_scales(const gdnq_desc *desc, const float *S0, const void *q, const void *k,
                            const void *v, const float *a, const float *b, int32_t n_steps,
                            const gdnq_state *state, void *stream);

/*
 * Baseline: one decode token on fp32 states S [B,H,dk,dv] (device, in
 * place), same inputs and output as gdn_quant_decode_step.  This is the
 * comparator the pages measure against (LeapQuant project page,
 * kernel-speed paragraph: the quantized kernel's speedups are stated over
 * the FP32 recurrent state; the update is LinQuant's appendix Table 3).
 * Per head it reads and writes the dk x dv fp32 state once.  Errors:
 * GDNQ_EINVAL for a NULL, misaligned or overlapping buffer.
 */
int gdn_fp32_decode_step(const gdnq_desc *desc, float *S, const void *q, const void *k,
                         const void *v, const float *a, const float *b, void *o, void *stream);

/*
 * Prefill ("LinQuant: Functional Invariances for Low-Precision Linear
 * Recurrences", abstract: chunkwise-parallel prefill casts most of the
 * recurrence as dense matrix products; appendix Table 3, Gated DeltaNet and
 * KDA rows).  Runs T tokens of the recurrence for all B*H heads at once,
 * chunk by chunk on the matrix cores (32 tokens per chunk for the scalar
 * gate at dk = 128, 64 at dk = 64, 16 for the per-channel gate), and writes
 * every token's output:
 *   S      device fp32 [B,H,dk,dv], in place: the state before token 0 on
 *          entry (zeros for a new sequence, gdn_state_dequantize's output to
 *          continue a cached prefix), the state after token T-1 on return.
 *   q, k   device bf16 [B,T,hk,dk] (hk = H unless set); v device bf16 [B,T,H,dv]
 *   a      device fp32, 0 < a <= 1: [B,T,H] for GDNQ_DECAY_SCALAR, [B,T,H,dk]
 *          for GDNQ_DECAY_CHANNEL (no bound on the product of gates: the
 *          chunk forms work with log-gates and only non-positive exponents)
 *   b      device fp32 [B,T,H]
 *   o      device bf16 [B,T,H,dv], o_t = S_t^T q_t
 * Supported: io_dtype GDNQ_IO_BF16, either decay, dk == dv (64 or 128);
 * other descriptors return GDNQ_EUNSUPPORTED.  W, r, layout,
 * n_hp, bits and the state struct play no part.  Products run in bf16 with
 * fp32 accumulation, fp32 operands split into two bf16 parts, so results
 * stay near fp32 accuracy.  T == 0 is a no-op (the buffers may be NULL).
 * Follow with gdn_state_quantize(desc, S, state) to store the prefilled
 * state in the quantized form for decoding.
 */
int gdn_prefill(const gdnq_desc *desc, float *S, const void *q, const void *k, const void *v,
                const float *a, const float *b, void *o, int32_t T, void *stream);

/*
 * Byte sizes of the 12 gdnq_state arrays for this descriptor, in field
 * order (codes, row_scale, col_scale, comp_k, comp_v, buf_k, buf_u, buf_g,
 * g_cur, hp_rows, hp_idx, prequant_out); 0 where the array is unused.
 */
int gdnq_state_sizes(const gdnq_desc *desc, size_t bytes_out[12]);

/* Message of the last error on this thread ("" if none). */
const char *gdnq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDNQ_H */
