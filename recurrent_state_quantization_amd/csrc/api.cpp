// api.cpp -- the C ABI of libgdnq.so (include/gdnq.h): argument checks on
// the host, then one launch per call on the caller's stream.  Nothing is
// allocated and nothing is synchronized.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdnq.h"
#include "launch.hpp"
#include "launchers.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return GDNQ_OK;
}

struct Span {
    const void *p;
    size_t n;
    const char *name;
};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const Span &a, const Span &b)
{
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

size_t io_size(const gdnq_desc &d) { return d.io_dtype == GDNQ_IO_BF16 ? 2 : 4; }
size_t nheads(const gdnq_desc &d) { return (size_t)d.B * (size_t)d.H; }
bool per_step(const gdnq_desc &d) { return d.W == 1 && d.r == 0; }
int code_bits(const gdnq_desc &d) { return d.bits == 0 ? 8 : d.bits; }
size_t nkheads(const gdnq_desc &d) { return (size_t)d.B * (size_t)(d.hk ? d.hk : d.H); }
size_t agate(const gdnq_desc &d) { return d.decay == GDNQ_DECAY_CHANNEL ? (size_t)d.dk : 1; }  // gate values per head

int check_desc(const gdnq_desc *d)
{
    if (!d) return fail(GDNQ_EINVAL, "desc is NULL");
    if (d->B < 1 || d->H < 1) return fail(GDNQ_EINVAL, "B and H must be >= 1 (got B=%d H=%d)", d->B, d->H);
    if ((long long)d->B * d->H > 0x7fffffffLL) return fail(GDNQ_EINVAL, "B*H too large");
    if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128))
        return fail(GDNQ_EUNSUPPORTED, "dk and dv must each be 64 or 128 (got dk=%d dv=%d)", d->dk, d->dv);
    if (d->W < 1 || d->W > gdnq::MAX_W) return fail(GDNQ_EINVAL, "W must be in [1, %d] (got %d)", gdnq::MAX_W, d->W);
    if (d->r < 0 || d->r > gdnq::MAX_R) return fail(GDNQ_EINVAL, "r must be in [0, %d] (got %d)", gdnq::MAX_R, d->r);
    if (d->decay != GDNQ_DECAY_SCALAR && d->decay != GDNQ_DECAY_CHANNEL)
        return fail(GDNQ_EINVAL, "decay must be GDNQ_DECAY_SCALAR or GDNQ_DECAY_CHANNEL (got %d)", d->decay);
    if (d->io_dtype != GDNQ_IO_F32 && d->io_dtype != GDNQ_IO_BF16)
        return fail(GDNQ_EINVAL, "io_dtype must be GDNQ_IO_F32 or GDNQ_IO_BF16 (got %d)", d->io_dtype);
    if (d->layout != GDNQ_LAYOUT_ROWCOL && d->layout != GDNQ_LAYOUT_DAMP)
        return fail(GDNQ_EINVAL, "layout must be GDNQ_LAYOUT_ROWCOL or GDNQ_LAYOUT_DAMP (got %d)", d->layout);
    if (d->layout == GDNQ_LAYOUT_DAMP) {
        if (d->n_hp < 1 || d->n_hp > d->dk / 2 || d->n_hp > gdnq::MAX_HP)
            return fail(GDNQ_EINVAL, "n_hp must be in [1, min(dk/2, %d)] for the DAMP layout (got %d)",
                        gdnq::MAX_HP, d->n_hp);
    }
    if (d->r > 0 && (d->power_iters < 1 || d->power_iters > 64))
        return fail(GDNQ_EINVAL, "power_iters must be in [1, 64] when r > 0 (got %d)", d->power_iters);
    if (d->flags & ~(GDNQ_DEBUG_PREQUANT | GDNQ_STATIC_SCALES))
        return fail(GDNQ_EINVAL, "unknown flag bits 0x%x", d->flags);
    if ((d->flags & GDNQ_STATIC_SCALES) && (d->layout != GDNQ_LAYOUT_ROWCOL || d->W != 1 || d->r != 0))
        return fail(GDNQ_EUNSUPPORTED, "static scales are for the per-step mode of layout 0 (W == 1, r == 0)");
    if (d->bits != 0 && d->bits != 8 && d->bits != 6 && d->bits != 4)
        return fail(GDNQ_EINVAL, "bits must be 8, 6 or 4 (0 means 8; got %d)", d->bits);
    if (d->layout == GDNQ_LAYOUT_DAMP && code_bits(*d) != 8)
        return fail(GDNQ_EUNSUPPORTED, "the DAMP layout keeps 8-bit codes (got bits=%d)", d->bits);
    if (d->hk < 0 || (d->hk > 0 && d->H % d->hk != 0))
        return fail(GDNQ_EINVAL, "hk must divide H (0 means H; got hk=%d, H=%d)", d->hk, d->H);
    return GDNQ_OK;
}

// byte sizes of the 12 state arrays, 0 where unused
constexpr int NSTATE = 12;

void state_sizes(const gdnq_desc &d, size_t out[NSTATE])
{
    const size_t nh = nheads(d);
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    const bool window = !per_step(d) || damp;
    const size_t rows = damp ? (size_t)(d.dk - d.n_hp) : (size_t)d.dk;
    out[0] = nh * rows * d.dv * code_bits(d) / 8;                          // codes
    const size_t planes = (d.flags & GDNQ_STATIC_SCALES) ? 2 : 1;        // static: s | rho, c | iota
    out[1] = damp ? 0 : planes * nh * d.dk * 4;                            // row_scale
    out[2] = planes * nh * d.dv * 4;                                       // col_scale
    out[3] = nh * (size_t)d.r * d.dk * 4;                                  // comp_k
    out[4] = nh * (size_t)d.r * d.dv * 4;                                  // comp_v
    out[5] = window ? nh * (size_t)d.W * d.dk * 4 : 0;                     // buf_k
    out[6] = window ? nh * (size_t)d.W * d.dv * 4 : 0;                     // buf_u
    out[7] = window ? nh * (size_t)d.W * agate(d) * 4 : 0;                 // buf_g
    out[8] = window ? nh * agate(d) * 4 : 0;                               // g_cur
    out[9] = damp ? nh * (size_t)d.n_hp * d.dv * 2 : 0;                   // hp_rows
    out[10] = damp ? nh * (size_t)d.n_hp * 4 : 0;                          // hp_idx
    out[11] = (d.flags & GDNQ_DEBUG_PREQUANT) ? nh * d.dk * d.dv * 4 : 0;  // prequant_out
}

const char *kStateNames[NSTATE] = {"codes", "row_scale", "col_scale", "comp_k", "comp_v", "buf_k",
                                   "buf_u", "buf_g",     "g_cur",     "hp_rows", "hp_idx", "prequant_out"};

void state_ptrs(const gdnq_state &s, const void *out[NSTATE])
{
    out[0] = s.codes;
    out[1] = s.row_scale;
    out[2] = s.col_scale;
    out[3] = s.comp_k;
    out[4] = s.comp_v;
    out[5] = s.buf_k;
    out[6] = s.buf_u;
    out[7] = s.buf_g;
    out[8] = s.g_cur;
    out[9] = s.hp_rows;
    out[10] = s.hp_idx;
    out[11] = s.prequant_out;
}

// Which state arrays a call reads or writes.
struct Need {
    bool v[NSTATE];
};

// codes, scales and compensators (+ DAMP rows); `window` adds the window
// buffer and gate arrays, `prequant` the debug output
Need need_of(const gdnq_desc &d, bool window, bool prequant)
{
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    return Need{{true, !damp, true, d.r > 0, d.r > 0, window, window, window, window, damp, damp, prequant}};
}

// Check the state arrays that `need[]` marks as used: non-NULL, 16-byte
// aligned, pairwise disjoint; append them to `spans` for overlap checks
// against the per-call buffers.
int check_state(const gdnq_desc &d, const gdnq_state *s, const Need &need, std::vector<Span> &spans)
{
    if (!s) return fail(GDNQ_EINVAL, "state is NULL");
    size_t sz[NSTATE];
    const void *p[NSTATE];
    state_sizes(d, sz);
    state_ptrs(*s, p);
    for (int i = 0; i < NSTATE; i++) {
        if (!need.v[i] || sz[i] == 0) continue;
        if (!p[i]) return fail(GDNQ_EINVAL, "state->%s is NULL but required here", kStateNames[i]);
        if (!aligned16(p[i])) return fail(GDNQ_EINVAL, "state->%s is not 16-byte aligned", kStateNames[i]);
        Span sp{p[i], sz[i], kStateNames[i]};
        for (const Span &o : spans)
            if (overlap(sp, o)) return fail(GDNQ_EINVAL, "state->%s overlaps %s", kStateNames[i], o.name);
        spans.push_back(sp);
    }
    return GDNQ_OK;
}

int check_buf(const void *p, size_t n, const char *name, std::vector<Span> &spans, bool nullable = false)
{
    if (!p) {
        if (nullable) return GDNQ_OK;
        return fail(GDNQ_EINVAL, "%s is NULL", name);
    }
    if (!aligned16(p)) return fail(GDNQ_EINVAL, "%s is not 16-byte aligned", name);
    Span sp{p, n, name};
    for (const Span &o : spans)
        if (overlap(sp, o)) return fail(GDNQ_EINVAL, "%s overlaps %s", name, o.name);
    spans.push_back(sp);
    return GDNQ_OK;
}

// a and b may share storage with nothing written by the call; q, k, v are
// read-only and may alias each other.
int check_step_io(const gdnq_desc &d, const void *q, const void *k, const void *v, const float *a,
                  const float *b, void *o, std::vector<Span> &spans)
{
    const size_t nh = nheads(d), es = io_size(d);
    int rc;
    // inputs: checked against the state (written) and against o, not each other
    std::vector<Span> written = spans;
    if ((rc = check_buf(o, nh * d.dv * es, "o", written))) return rc;
    const size_t na = d.decay == GDNQ_DECAY_CHANNEL ? (size_t)d.dk : 1;
    struct In {
        const void *p;
        size_t n;
        const char *name;
    } ins[5] = {{q, nkheads(d) * d.dk * es, "q"}, {k, nkheads(d) * d.dk * es, "k"}, {v, nh * d.dv * es, "v"},
                {a, nh * na * 4, "a"}, {b, nh * 4, "b"}};
    for (const In &in : ins) {
        std::vector<Span> tmp = written;
        if ((rc = check_buf(in.p, in.n, in.name, tmp))) return rc;
    }
    spans = written;
    return GDNQ_OK;
}

int launched(hipError_t e)
{
    if (e != hipSuccess) return fail(GDNQ_ELAUNCH, "HIP launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char *gdnq_last_error(void) { return g_err; }

int gdnq_state_sizes(const gdnq_desc *desc, size_t bytes_out[12])
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!bytes_out) return fail(GDNQ_EINVAL, "bytes_out is NULL");
    state_sizes(*desc, bytes_out);
    return ok();
}

int gdn_quant_decode_step(const gdnq_desc *desc, const gdnq_state *state, const void *q, const void *k,
                          const void *v, const float *a, const float *b, void *o, int32_t t_in_window,
                          void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    const bool fused = per_step(d) && !damp;
    if (t_in_window < 0 || t_in_window >= d.W)
        return fail(GDNQ_EINVAL, "t_in_window must be in [0, W-1] (got %d, W=%d)", t_in_window, d.W);
    // the debug output is written by the fused step and by the flush that
    // follows a DAMP per-step decode
    const Need need = need_of(d, !fused, (fused || per_step(d)) && (d.flags & GDNQ_DEBUG_PREQUANT));
    std::vector<Span> spans;
    if ((rc = check_state(d, state, need, spans))) return rc;
    if ((rc = check_step_io(d, q, k, v, a, b, o, spans))) return rc;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (fused) return launched(gdnq::launch_step_fused(d, gdnq::plain_map(d), *state, q, k, v, a, b, o, st));
    hipError_t e = gdnq::launch_window_step(d, gdnq::plain_map(d), *state, q, k, v, a, b, o, t_in_window, st);
    if (e == hipSuccess && per_step(d)) e = gdnq::launch_flush(d, gdnq::plain_map(d), *state, 1, st);
    return launched(e);
}

int gdn_quant_window_flush(const gdnq_desc *desc, const gdnq_state *state, int32_t n_tokens, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    if (per_step(d) && !damp) {
        if (n_tokens < 0 || n_tokens > 1) return fail(GDNQ_EINVAL, "n_tokens must be 0 or 1 in per-step mode");
        return ok();
    }
    if (per_step(d) && damp) return ok();  // the decode step already flushed
    if (n_tokens < 1 || n_tokens > d.W)
        return fail(GDNQ_EINVAL, "n_tokens must be in [1, W] (got %d, W=%d)", n_tokens, d.W);
    const Need need = need_of(d, true, (d.flags & GDNQ_DEBUG_PREQUANT) != 0);
    std::vector<Span> spans;
    if ((rc = check_state(d, state, need, spans))) return rc;
    return launched(gdnq::launch_flush(d, gdnq::plain_map(d), *state, n_tokens, reinterpret_cast<hipStream_t>(stream)));
}

int gdn_quant_decode_step_pool(const gdnq_desc *desc, const gdnq_state *state, int32_t n_slots,
                               const int32_t *slots, const int32_t *t_pos, const void *q, const void *k,
                               const void *v, const float *a, const float *b, void *o, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (n_slots < 1) return fail(GDNQ_EINVAL, "n_slots must be >= 1 (got %d)", n_slots);
    if ((long long)n_slots * desc->H > 0x7fffffffLL) return fail(GDNQ_EINVAL, "n_slots*H too large");
    gdnq_desc pool = *desc;   // the state arrays are sized for n_slots entries
    pool.B = n_slots;
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    const bool fused = per_step(d) && !damp;
    const Need need = need_of(d, !fused, (fused || per_step(d)) && (d.flags & GDNQ_DEBUG_PREQUANT));
    std::vector<Span> spans;
    if ((rc = check_state(pool, state, need, spans))) return rc;
    if ((rc = check_step_io(d, q, k, v, a, b, o, spans))) return rc;
    if ((rc = check_buf(slots, (size_t)d.B * 4, "slots", spans))) return rc;
    if (!per_step(d) && (rc = check_buf(t_pos, (size_t)d.B * 4, "t_pos", spans))) return rc;
    gdnq::HeadMap m = gdnq::plain_map(d);
    m.slots = slots;
    m.n_slots = n_slots;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (fused) return launched(gdnq::launch_step_fused(d, m, *state, q, k, v, a, b, o, st));
    if (per_step(d)) {   // DAMP per-step: window step at position 0, then a one-token flush
        hipError_t e = gdnq::launch_window_step(d, m, *state, q, k, v, a, b, o, 0, st);
        if (e == hipSuccess) e = gdnq::launch_flush(d, m, *state, 1, st);
        return launched(e);
    }
    m.pos = t_pos;
    return launched(gdnq::launch_window_step(d, m, *state, q, k, v, a, b, o, 0, st));
}

int gdn_quant_window_flush_pool(const gdnq_desc *desc, const gdnq_state *state, int32_t n_slots,
                                const int32_t *slots, const int32_t *n_tokens, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (n_slots < 1) return fail(GDNQ_EINVAL, "n_slots must be >= 1 (got %d)", n_slots);
    if ((long long)n_slots * desc->H > 0x7fffffffLL) return fail(GDNQ_EINVAL, "n_slots*H too large");
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    if (per_step(d)) return ok();   // per-step mode has no window to flush
    gdnq_desc pool = d;
    pool.B = n_slots;
    const Need need = need_of(d, true, (d.flags & GDNQ_DEBUG_PREQUANT) != 0);
    std::vector<Span> spans;
    if ((rc = check_state(pool, state, need, spans))) return rc;
    if ((rc = check_buf(slots, (size_t)d.B * 4, "slots", spans))) return rc;
    if ((rc = check_buf(n_tokens, (size_t)d.B * 4, "n_tokens", spans))) return rc;
    gdnq::HeadMap m = gdnq::plain_map(d);
    m.slots = slots;
    m.pos = n_tokens;
    m.n_slots = n_slots;
    return launched(gdnq::launch_flush(d, m, *state, 1, reinterpret_cast<hipStream_t>(stream)));
}

int gdn_state_quantize(const gdnq_desc *desc, const float *S, const gdnq_state *state, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    const Need need = need_of(d, false, (d.flags & GDNQ_DEBUG_PREQUANT) != 0);
    std::vector<Span> spans;
    if ((rc = check_state(d, state, need, spans))) return rc;
    if ((rc = check_buf(S, nheads(d) * d.dk * d.dv * 4, "S", spans))) return rc;
    // g_cur is optional here: reset to 1 when given
    if (state->g_cur) {
        size_t sz[NSTATE];
        state_sizes(d, sz);
        size_t gsz = nheads(d) * agate(d) * 4;
        if ((rc = check_buf(state->g_cur, sz[8] ? sz[8] : gsz, "state->g_cur", spans))) return rc;
    }
    return launched(gdnq::launch_quantize(d, S, *state, reinterpret_cast<hipStream_t>(stream)));
}

int gdn_state_dequantize(const gdnq_desc *desc, const gdnq_state *state, float *S_out, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    const bool damp = d.layout == GDNQ_LAYOUT_DAMP;
    const Need need = need_of(d, false, false);
    std::vector<Span> spans;
    if ((rc = check_state(d, state, need, spans))) return rc;
    if ((rc = check_buf(S_out, nheads(d) * d.dk * d.dv * 4, "S_out", spans))) return rc;
    return launched(gdnq::launch_dequantize(d, *state, S_out, reinterpret_cast<hipStream_t>(stream)));
}

int calibrate_scales(const gdnq_desc *desc, const float *S0, const void *k, const void *v, const float *a,
                     const float *b, int32_t n_steps, int32_t *hp_idx_out, float *row_score_out,
                     void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    if (d.n_hp < 1 || d.n_hp > d.dk / 2 || d.n_hp > gdnq::MAX_HP)
        return fail(GDNQ_EINVAL, "n_hp must be in [1, min(dk/2, %d)] (got %d)", gdnq::MAX_HP, d.n_hp);
    if (n_steps < 1) return fail(GDNQ_EINVAL, "n_steps must be >= 1 (got %d)", n_steps);
    const size_t nh = nheads(d), es = io_size(d), ns = (size_t)n_steps;
    const size_t na = d.decay == GDNQ_DECAY_CHANNEL ? (size_t)d.dk : 1;
    std::vector<Span> spans;
    if ((rc = check_buf(hp_idx_out, nh * d.n_hp * 4, "hp_idx_out", spans))) return rc;
    if ((rc = check_buf(row_score_out, nh * d.dk * 4, "row_score_out", spans, true))) return rc;
    struct In {
        const void *p;
        size_t n;
        const char *name;
    } ins[5] = {{S0, nh * d.dk * d.dv * 4, "S0"}, {k, ns * nkheads(d) * d.dk * es, "k"}, {v, ns * nh * d.dv * es, "v"},
                {a, ns * nh * na * 4, "a"}, {b, ns * nh * 4, "b"}};
    for (const In &in : ins) {
        std::vector<Span> tmp = spans;
        if ((rc = check_buf(in.p, in.n, in.name, tmp))) return rc;
    }
    return launched(gdnq::launch_calibrate(d, S0, k, v, a, b, n_steps, hp_idx_out, row_score_out,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int gdn_fp32_decode_step(const gdnq_desc *desc, float *S, const void *q, const void *k, const void *v,
                         const float *a, const float *b, void *o, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    std::vector<Span> spans;
    if ((rc = check_buf(S, nheads(d) * d.dk * d.dv * 4, "S", spans))) return rc;
    if ((rc = check_step_io(d, q, k, v, a, b, o, spans))) return rc;
    return launched(gdnq::launch_step_fp32(d, S, q, k, v, a, b, o, reinterpret_cast<hipStream_t>(stream)));
}

int calibrate_static_scales(const gdnq_desc *desc, const float *S0, const void *q, const void *k, const void *v,
                            const float *a, const float *b, int32_t n_steps, const gdnq_state *state, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    if (!(d.flags & GDNQ_STATIC_SCALES))
        return fail(GDNQ_EINVAL, "calibrate_static_scales needs a descriptor with GDNQ_STATIC_SCALES");
    if (n_steps < 1) return fail(GDNQ_EINVAL, "n_steps must be >= 1 (got %d)", n_steps);
    const size_t nh = nheads(d), es = io_size(d), ns = (size_t)n_steps;
    const size_t na = d.decay == GDNQ_DECAY_CHANNEL ? (size_t)d.dk : 1;
    std::vector<Span> spans;
    Need need{};
    need.v[1] = need.v[2] = true;  // row_scale, col_scale (both planes)
    if ((rc = check_state(d, state, need, spans))) return rc;
    struct In {
        const void *p;
        size_t n;
        const char *name;
    } ins[6] = {{S0, nh * d.dk * d.dv * 4, "S0"},         {q, ns * nkheads(d) * d.dk * es, "q"},
                {k, ns * nkheads(d) * d.dk * es, "k"},    {v, ns * nh * d.dv * es, "v"},
                {a, ns * nh * na * 4, "a"},               {b, ns * nh * 4, "b"}};
    for (const In &in : ins) {
        std::vector<Span> tmp = spans;
        if ((rc = check_buf(in.p, in.n, in.name, tmp))) return rc;
    }
    return launched(gdnq::launch_fit_static(d, S0, q, k, v, a, b, n_steps, state->row_scale, state->col_scale,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int gdn_prefill(const gdnq_desc *desc, float *S, const void *q, const void *k, const void *v, const float *a,
                const float *b, void *o, int32_t T, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    const gdnq_desc &d = *desc;
    if (d.io_dtype != GDNQ_IO_BF16) return fail(GDNQ_EUNSUPPORTED, "gdn_prefill takes bf16 q, k, v and o");
    if (d.dk != d.dv) return fail(GDNQ_EUNSUPPORTED, "gdn_prefill needs dk == dv (got %d, %d)", d.dk, d.dv);
    if (T < 0) return fail(GDNQ_EINVAL, "T must be >= 0 (got %d)", T);
    const size_t nh = nheads(d), nt = (size_t)T;
    if (nt * nh > 0x7fffffffULL) return fail(GDNQ_EINVAL, "B*T*H too large");
    std::vector<Span> spans;
    if ((rc = check_buf(S, nh * d.dk * d.dv * 4, "S", spans))) return rc;
    if ((rc = check_buf(o, nt * nh * d.dv * 2, "o", spans, T == 0))) return rc;
    struct In {
        const void *p;
        size_t n;
        const char *name;
    } ins[5] = {{q, nt * nkheads(d) * d.dk * 2, "q"}, {k, nt * nkheads(d) * d.dk * 2, "k"},
                {v, nt * nh * d.dv * 2, "v"}, {a, nt * nh * agate(d) * 4, "a"}, {b, nt * nh * 4, "b"}};
    for (const In &in : ins) {
        std::vector<Span> tmp = spans;
        if ((rc = check_buf(in.p, in.n, in.name, tmp, T == 0))) return rc;
    }
    if (T == 0) return ok();
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (d.decay == GDNQ_DECAY_CHANNEL) return launched(gdnq::launch_prefill_kda(d, S, q, k, v, a, b, o, T, st));
    return launched(gdnq::launch_prefill(d, S, q, k, v, a, b, o, T, st));
}

}  // extern "C"
