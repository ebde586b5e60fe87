// api.cpp -- the C ABI of libnhmamba: argument validation, workspace layout, launches.
//
// Every entry point validates all of its arguments before it enqueues anything, so a call
// that returns an error has no side effect.  Nothing here allocates device memory or
// synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/nhmamba.h"
#include "nh_device.hpp"
#include "nh_kernels.hpp"

using namespace nh;

namespace nh {
ProfEvents &prof_next()
{
    static thread_local ProfEvents p;
    return p;
}
}  // namespace nh

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_prof_ev[6];
thread_local int g_prof_on = 0;

// arm the start/stop events of the step's kernel i (0 in_proj, 1 SSM, 2 out_proj)
void prof_arm(int i)
{
    if (g_prof_on) prof_next() = ProfEvents{g_prof_ev[2 * i], g_prof_ev[2 * i + 1]};
}

nh_status fail(nh_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

nh_status ok()
{
    g_err.clear();
    return NH_OK;
}

nh_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) return fail(NH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define NH_TRY(expr)                         \
    do {                                     \
        nh_status s__ = (expr);              \
        if (s__ != NH_OK) return s__;        \
    } while (0)

#define NH_HIP(expr, what)                                          \
    do {                                                            \
        hipError_t e__ = (expr);                                    \
        if (e__ != hipSuccess) return hip_status(e__, what);        \
    } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

nh_status need_ptr(const void *p, const char *name)
{
    if (!p) return fail(NH_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned16(p)) return fail(NH_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return NH_OK;
}

nh_status opt_ptr(const void *p, const char *name)
{
    if (p && !aligned16(p)) return fail(NH_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
    return NH_OK;
}

nh_status need_dtype(int t, const char *name)
{
    if (t != NH_BF16 && t != NH_F32) return fail(NH_ERR_INVALID_ARGUMENT, "%s: unknown dtype %d", name, t);
    return NH_OK;
}

nh_status check_w4(const nh_w4_matrix *W, const char *name)
{
    if (!W) return fail(NH_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    NH_TRY(need_ptr(W->qweight, "qweight"));
    NH_TRY(need_ptr(W->scales, "scales"));
    NH_TRY(need_ptr(W->biases, "biases"));
    if (W->group_size != 64)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "%s: group_size %d (only 64)", name, W->group_size);
    if (W->n_out < 1 || W->k_in < 64 || W->k_in % 64 != 0 || W->k_in > 16384)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "%s: n_out %d, k_in %d (need n_out >= 1, k_in %% 64 == 0, "
                    "64 <= k_in <= 16384)", name, W->n_out, W->k_in);
    // the kernels address the packed matrix through one 32-bit buffer range
    if ((long long)W->n_out * (W->k_in / 2) >= (1LL << 31))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "%s: packed matrix of %d x %d is 2 GiB or more", name,
                    W->n_out, W->k_in);
    return NH_OK;
}

W4 view(const nh_w4_matrix *W) { return W4{W->qweight, W->scales, W->biases, W->n_out, W->k_in}; }

nh_status check_dims(const nh_mamba_dims *d, bool need_chunk)
{
    if (!d) return fail(NH_ERR_INVALID_ARGUMENT, "dims is NULL");
    if (d->hidden != HIDDEN || d->n_heads != NHEADS || d->head_dim != HDIM || d->d_state != DSTATE ||
        d->n_groups != NGROUPS || d->conv_k != CONVK)
        return fail(NH_ERR_UNSUPPORTED_SHAPE,
                    "dims (%d,%d,%d,%d,%d,%d) differ from the supported Nemotron-H mixer "
                    "(4480,128,80,128,8,4)", d->hidden, d->n_heads, d->head_dim, d->d_state,
                    d->n_groups, d->conv_k);
    if (!(d->eps > 0.f) || !std::isfinite(d->eps))
        return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive and finite");
    if (need_chunk && (d->chunk < 1 || d->chunk > QMAX))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "chunk %d outside 1..%d", d->chunk, QMAX);
    return NH_OK;
}

nh_status check_weights(const nh_mamba_weights *w)
{
    if (!w) return fail(NH_ERR_INVALID_ARGUMENT, "weights is NULL");
    NH_TRY(need_ptr(w->norm_w, "norm_w"));
    NH_TRY(check_w4(&w->in_proj, "in_proj"));
    NH_TRY(need_ptr(w->conv_w, "conv_w"));
    NH_TRY(need_ptr(w->conv_b, "conv_b"));
    NH_TRY(need_ptr(w->dt_bias, "dt_bias"));
    NH_TRY(need_ptr(w->A_log, "A_log"));
    NH_TRY(need_ptr(w->D, "D"));
    NH_TRY(need_ptr(w->gnorm_w, "gnorm_w"));
    NH_TRY(check_w4(&w->out_proj, "out_proj"));
    if (w->in_proj.n_out != NIN || w->in_proj.k_in != HIDDEN)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "in_proj is %dx%d, expected %dx%d", w->in_proj.n_out,
                    w->in_proj.k_in, NIN, HIDDEN);
    if (w->out_proj.n_out != HIDDEN || w->out_proj.k_in != DINNER)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "out_proj is %dx%d, expected %dx%d", w->out_proj.n_out,
                    w->out_proj.k_in, HIDDEN, DINNER);
    return NH_OK;
}

// ---------------------------------------------------------------- workspace layout
struct Carve {
    char *base;
    size_t off = 0;
    template <class T>
    T *take(size_t count)
    {
        off = (off + 255) & ~size_t(255);
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

struct StepWs {
    uint16_t *z, *xc, *dtr;
    float *gate, *part, *osum;
};

StepWs carve_step(void *ws, int B, size_t *bytes)
{
    Carve c{reinterpret_cast<char *>(ws)};
    StepWs s;
    s.z = c.take<uint16_t>((size_t)B * DINNER);
    s.xc = c.take<uint16_t>((size_t)B * CONVDIM);
    s.dtr = c.take<uint16_t>((size_t)B * NHEADS);
    s.gate = c.take<float>((size_t)B * DINNER);
    s.part = c.take<float>((size_t)B * NHEADS * 2);
    s.osum = c.take<float>(outproj_partial_floats(B));
    *bytes = c.off;
    return s;
}

struct SeqWs {
    uint16_t *u, *zx, *xc, *y, *o, *cs;
    float *su_u, *su_o;
};

SeqWs carve_seq(void *ws, int B, int T, size_t *bytes)
{
    const size_t M = (size_t)B * T;
    Carve c{reinterpret_cast<char *>(ws)};
    SeqWs s;
    s.u = c.take<uint16_t>(M * HIDDEN);
    s.su_u = c.take<float>(M * (HIDDEN / 64));
    s.zx = c.take<uint16_t>(M * NIN);
    s.xc = c.take<uint16_t>(M * CONVDIM);
    s.y = c.take<uint16_t>(M * DINNER);
    s.o = c.take<uint16_t>(M * DINNER);
    s.su_o = c.take<float>(M * (DINNER / 64));
    s.cs = c.take<uint16_t>((size_t)B * (CONVK - 1) * CONVDIM);
    *bytes = c.off;
    return s;
}

size_t step_bytes(int B)
{
    size_t n;
    carve_step(nullptr, B, &n);
    return n;
}

size_t seq_bytes(int B, int T)
{
    size_t n;
    carve_seq(nullptr, B, T, &n);
    return n;
}

hipStream_t S(void *stream) { return reinterpret_cast<hipStream_t>(stream); }

// The block bodies, called after validation.
nh_status block_step(const nh_mamba_dims *d, const nh_mamba_weights *w, nh_mamba_state *st,
                     const void *x, int x_t, void *out, int out_t, int B, void *ws, hipStream_t s)
{
    size_t nb;
    StepWs k = carve_step(ws, B, &nb);
    prof_arm(0);
    NH_HIP(launch_inproj_step(view(&w->in_proj), x, x_t, w->norm_w, d->eps, B, k.z, k.xc, k.dtr,
                              st->conv_state, w->conv_w, w->conv_b, nullptr, 0, s),
           "in_proj step");
    prof_arm(1);
    NH_HIP(launch_ssm_step_part(k.xc, k.dtr, NHEADS, w->dt_bias, w->A_log, w->D, st->ssm_state, k.gate, k.z,
                                w->gnorm_w, k.part, B, s),
           "ssm step");
    prof_arm(2);
    NH_HIP(launch_outproj_step(view(&w->out_proj), k.gate, k.part, d->eps, B, x, x_t, out, out_t, k.osum, s),
           "out_proj step");
    prof_next() = ProfEvents{};
    return ok();
}

nh_status block_seq(const nh_mamba_dims *d, const nh_mamba_weights *w, const nh_mamba_state *init,
                    nh_mamba_state *fin, const void *x, int x_t, int T, void *out, int out_t, int B,
                    void *ws, hipStream_t s)
{
    size_t nb;
    SeqWs k = carve_seq(ws, B, T, &nb);
    const int M = B * T;
    NH_HIP(launch_rmsnorm(x, x_t, w->norm_w, k.u, 1, k.su_u, M, HIDDEN, d->eps, s), "pre-norm");
    NH_HIP(launch_w4_gemm(view(&w->in_proj), k.u, k.su_u, M, nullptr, BF16, k.zx, BF16, s), "in_proj");
    const uint16_t *cs_in = init ? init->conv_state : nullptr;
    uint16_t *cs_out = fin ? fin->conv_state : nullptr;
    if (cs_in && cs_out == cs_in) {
        NH_HIP(hipMemcpyAsync(k.cs, cs_in, (size_t)B * (CONVK - 1) * CONVDIM * 2, hipMemcpyDeviceToDevice, s),
               "conv state copy");
        cs_in = k.cs;
    }
    NH_HIP(launch_conv_seq(k.zx + DINNER, NIN, T, cs_in, cs_out, w->conv_w, w->conv_b, k.xc, B, CONVDIM, s),
           "conv");
    // the scan's workspace (C.B^T tiles, and for long chunks the B fragments and tables) takes
    // the gated norm's output region, which is written only after the scan
    if (ssd_scan_ws_bytes(B, T, d->chunk) > (size_t)M * DINNER * sizeof(uint16_t))
        return fail(NH_ERR_INVALID_ARGUMENT, "internal: scan workspace exceeds its region");
    NH_HIP(launch_ssd_scan(k.xc, k.zx + DINNER + CONVDIM, NIN, T, d->chunk, w->dt_bias, w->A_log, w->D,
                           init ? init->ssm_state : nullptr, fin ? fin->ssm_state : nullptr, k.y, BF16, B,
                           k.o, s),
           "scan");
    NH_HIP(launch_rmsnorm_gated(k.y, BF16, k.zx, NIN, w->gnorm_w, k.o, 1, k.su_o, M, DINNER, GNORM, d->eps, s),
           "gated norm");
    NH_HIP(launch_w4_gemm(view(&w->out_proj), k.o, k.su_o, M, x, x_t, out, out_t, s), "out_proj");
    return ok();
}

nh_status check_state(const nh_mamba_state *st, const char *name, bool required)
{
    if (!st) {
        if (required) return fail(NH_ERR_INVALID_ARGUMENT, "%s is NULL", name);
        return NH_OK;
    }
    NH_TRY(need_ptr(st->conv_state, "conv_state"));
    NH_TRY(need_ptr(st->ssm_state, "ssm_state"));
    return NH_OK;
}

// ---------------------------------------------------------------- attention layers
constexpr int ATT_Q = 40 * 128, ATT_KV = 8 * 128, ATT_MAX_LEN = 1 << 22;

nh_status check_attention(const nh_attention_weights *w)
{
    if (!w) return fail(NH_ERR_INVALID_ARGUMENT, "attention weights are NULL");
    NH_TRY(need_ptr(w->norm_w, "attention norm_w"));
    NH_TRY(check_w4(&w->q_proj, "q_proj"));
    NH_TRY(check_w4(&w->k_proj, "k_proj"));
    NH_TRY(check_w4(&w->v_proj, "v_proj"));
    NH_TRY(check_w4(&w->o_proj, "o_proj"));
    if (w->q_proj.n_out != ATT_Q || w->q_proj.k_in != HIDDEN || w->k_proj.n_out != ATT_KV ||
        w->k_proj.k_in != HIDDEN || w->v_proj.n_out != ATT_KV || w->v_proj.k_in != HIDDEN ||
        w->o_proj.n_out != HIDDEN || w->o_proj.k_in != ATT_Q)
        return fail(NH_ERR_UNSUPPORTED_SHAPE,
                    "attention projections q %dx%d, k %dx%d, v %dx%d, o %dx%d (need q [%d][%d], k and v "
                    "[%d][%d], o [%d][%d])",
                    w->q_proj.n_out, w->q_proj.k_in, w->k_proj.n_out, w->k_proj.k_in, w->v_proj.n_out,
                    w->v_proj.k_in, w->o_proj.n_out, w->o_proj.k_in, ATT_Q, HIDDEN, ATT_KV, HIDDEN, HIDDEN, ATT_Q);
    return NH_OK;
}

nh_status check_cache(const nh_kv_cache *c)
{
    if (!c) return fail(NH_ERR_INVALID_ARGUMENT, "kv cache is NULL");
    NH_TRY(need_ptr(c->k, "cache k"));
    NH_TRY(need_ptr(c->v, "cache v"));
    if (c->max_len < 1 || c->max_len > ATT_MAX_LEN)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "cache max_len %d outside 1..%d", c->max_len, ATT_MAX_LEN);
    return NH_OK;
}

struct AttWs {
    uint16_t *q, *o;
    float *part;
};

AttWs carve_attention(void *ws, int B, size_t *bytes)
{
    Carve c{reinterpret_cast<char *>(ws)};
    AttWs a;
    a.q = c.take<uint16_t>((size_t)B * ATT_Q);
    a.o = c.take<uint16_t>((size_t)B * ATT_Q);
    a.part = c.take<float>(attn_part_bytes(B) / sizeof(float));
    *bytes = c.off;
    return a;
}

size_t attention_bytes(int B)
{
    size_t n;
    carve_attention(nullptr, B, &n);
    return n;
}

// the four launches of one attention layer (arguments already checked)
nh_status attention_step(const nh_attention_weights *w, const nh_kv_cache *c, const int32_t *pos, const void *x,
                         int x_t, void *out, int out_t, int B, float eps, void *ws, hipStream_t s)
{
    size_t n;
    const AttWs a = carve_attention(ws, B, &n);
    NH_HIP(launch_attn_qkv(view(&w->q_proj), view(&w->k_proj), view(&w->v_proj), x, x_t, w->norm_w, eps, B, a.q,
                           c->k, c->v, pos, c->max_len, s),
           "attention q/k/v");
    NH_HIP(launch_attn_decode(a.q, c->k, c->v, pos, c->max_len, B, a.part, a.o, s), "attention");
    NH_HIP(launch_gemv(view(&w->o_proj), a.o, BF16, B, x, x_t, out, out_t, s), "attention o_proj");
    return NH_OK;
}

}  // namespace

extern "C" {

const char *nh_last_error(void) { return g_err.c_str(); }

const char *nh_version(void) { return "libnhmamba 0.1 (gfx950)"; }

nh_status nh_profile_events(void *const *events, int n)
{
    if (!events) {
        g_prof_on = 0;
        return ok();
    }
    if (n < 6) return fail(NH_ERR_INVALID_ARGUMENT, "need 6 events, got %d", n);
    for (int i = 0; i < 6; ++i) {
        if (!events[i]) return fail(NH_ERR_INVALID_ARGUMENT, "event %d is NULL", i);
        g_prof_ev[i] = reinterpret_cast<hipEvent_t>(events[i]);
    }
    g_prof_on = 1;
    return ok();
}

const char *nh_hybrid_pattern(void)
{
    // text_config.hybrid_override_pattern (issue page, section "config.json").
    return "M-M-M-MM-M-M-M*-M-M-M*-M-M-M-M*-M-M-M-M*-M-MM-M-M-M-M-M-";
}

nh_status nh_w4_gemv(const nh_w4_matrix *W, const void *x, nh_dtype x_dtype, int batch, const void *residual,
                     nh_dtype res_dtype, void *y, nh_dtype y_dtype, void *stream)
{
    NH_TRY(check_w4(W, "W"));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_ptr(y, "y"));
    NH_TRY(opt_ptr(residual, "residual"));
    NH_TRY(need_dtype(y_dtype, "y_dtype"));
    if (residual) NH_TRY(need_dtype(res_dtype, "res_dtype"));
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    NH_HIP(launch_gemv(view(W), x, x_dtype, batch, residual, res_dtype, y, y_dtype, S(stream)), "gemv");
    return ok();
}

size_t nh_mlp_workspace_bytes(int inter, int batch)
{
    if (inter < 64 || inter % 64 || inter > 16384 || batch < 1 || batch > 4) return 0;
    return ((size_t)batch * inter * sizeof(uint16_t) + 255) / 256 * 256;
}

nh_status nh_mlp_step(const uint16_t *norm_w, const nh_w4_matrix *up, const nh_w4_matrix *down, float eps,
                      const void *x, nh_dtype x_dtype, void *out, nh_dtype out_dtype, int batch, void *ws,
                      size_t ws_bytes, void *stream)
{
    NH_TRY(need_ptr(norm_w, "norm_w"));
    NH_TRY(check_w4(up, "up"));
    NH_TRY(check_w4(down, "down"));
    if (up->k_in != HIDDEN || down->n_out != HIDDEN || down->k_in != up->n_out)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "up %d x %d, down %d x %d (need up [inter][%d], down [%d][inter])",
                    up->n_out, up->k_in, down->n_out, down->k_in, HIDDEN, HIDDEN);
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_ptr(out, "out"));
    NH_TRY(need_dtype(out_dtype, "out_dtype"));
    NH_TRY(need_ptr(ws, "ws"));
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive");
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    const size_t need = nh_mlp_workspace_bytes(up->n_out, batch);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "mlp workspace %zu < %zu bytes", ws_bytes, need);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws);
    NH_HIP(launch_mlp_up_step(view(up), x, x_dtype, norm_w, eps, batch, h, S(stream)), "mlp up");
    NH_HIP(launch_gemv(view(down), h, BF16, batch, x, x_dtype, out, out_dtype, S(stream)), "mlp down");
    return ok();
}

nh_status nh_fused_embedding(const nh_w4_matrix *E, const int32_t *text_ids, const int32_t *function_ids,
                             const void *audio, nh_dtype audio_dtype, float function_weight, int batch,
                             float *out, void *stream)
{
    NH_TRY(check_w4(E, "E"));
    NH_TRY(need_ptr(text_ids, "text_ids"));
    NH_TRY(need_ptr(function_ids, "function_ids"));
    NH_TRY(need_ptr(audio, "audio"));
    NH_TRY(need_dtype(audio_dtype, "audio_dtype"));
    NH_TRY(need_ptr(out, "out"));
    if (!std::isfinite(function_weight)) return fail(NH_ERR_INVALID_ARGUMENT, "function_weight must be finite");
    if (batch < 1 || batch > 4096) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4096", batch);
    NH_HIP(launch_fused_embed(view(E), text_ids, function_ids, audio, audio_dtype, function_weight, batch, out,
                              S(stream)),
           "fused embedding");
    return ok();
}

size_t nh_head_workspace_bytes(int batch)
{
    if (batch < 1 || batch > 4) return 0;
    return head_ws_bytes(batch);
}

nh_status nh_head_argmax(const nh_w4_matrix *W, const void *x, nh_dtype x_dtype, const uint16_t *norm_w,
                         float eps, int batch, float *logits, int32_t *ids, void *ws, size_t ws_bytes,
                         void *stream)
{
    NH_TRY(check_w4(W, "W"));
    if (W->k_in != HIDDEN || W->n_out > (1 << 19))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "head %d x %d (need k_in == %d, n_out <= 524288)", W->n_out,
                    W->k_in, HIDDEN);
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_ptr(norm_w, "norm_w"));
    NH_TRY(opt_ptr(logits, "logits"));
    NH_TRY(need_ptr(ids, "ids"));
    NH_TRY(need_ptr(ws, "ws"));
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive");
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    if (ws_bytes < head_ws_bytes(batch))
        return fail(NH_ERR_WORKSPACE_TOO_SMALL, "head workspace %zu < %zu bytes", ws_bytes, head_ws_bytes(batch));
    NH_HIP(launch_head(view(W), x, x_dtype, norm_w, eps, batch, logits, ids, ws, S(stream)), "head");
    return ok();
}

size_t nh_w4_gemm_workspace_bytes(int M, int k_in)
{
    if (M < 1 || k_in < 64 || k_in % 64) return 0;
    Carve c{nullptr};
    c.take<uint16_t>((size_t)M * k_in);
    c.take<float>((size_t)M * (k_in / 64));
    return c.off;
}

nh_status nh_w4_gemm(const nh_w4_matrix *W, const uint16_t *X, int M, const void *residual,
                     nh_dtype res_dtype, void *Y, nh_dtype y_dtype, void *ws, size_t ws_bytes, void *stream)
{
    NH_TRY(check_w4(W, "W"));
    NH_TRY(need_ptr(X, "X"));
    NH_TRY(need_ptr(Y, "Y"));
    NH_TRY(opt_ptr(residual, "residual"));
    NH_TRY(need_dtype(y_dtype, "y_dtype"));
    if (residual) NH_TRY(need_dtype(res_dtype, "res_dtype"));
    if (M < 1) return fail(NH_ERR_UNSUPPORTED_SHAPE, "M %d < 1", M);
    NH_TRY(need_ptr(ws, "ws"));
    const size_t need = nh_w4_gemm_workspace_bytes(M, W->k_in);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    Carve c{reinterpret_cast<char *>(ws)};
    uint16_t *xh = c.take<uint16_t>((size_t)M * W->k_in);
    float *su = c.take<float>((size_t)M * (W->k_in / 64));
    NH_HIP(launch_to_f16(X, xh, su, M, W->k_in, S(stream)), "gemm staging");
    NH_HIP(launch_w4_gemm(view(W), xh, su, M, residual, res_dtype, Y, y_dtype, S(stream)), "gemm");
    return ok();
}

nh_status nh_rmsnorm(const void *x, nh_dtype x_dtype, const uint16_t *w, uint16_t *u, int rows, int d,
                     float eps, void *stream)
{
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(w, "w"));
    NH_TRY(need_ptr(u, "u"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    if (rows < 1 || d < 8 || d % 8 || d > 8192)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "rows %d, d %d (need rows >= 1, d %% 8 == 0, d <= 8192)", rows, d);
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive");
    NH_HIP(launch_rmsnorm(x, x_dtype, w, u, 0, nullptr, rows, d, eps, S(stream)), "rmsnorm");
    return ok();
}

nh_status nh_conv1d_step(const uint16_t *xbc, long ld, uint16_t *conv_state, const uint16_t *w,
                         const uint16_t *b, uint16_t *out, int batch, int channels, int k, void *stream)
{
    NH_TRY(need_ptr(xbc, "xbc"));
    NH_TRY(need_ptr(conv_state, "conv_state"));
    NH_TRY(need_ptr(w, "w"));
    NH_TRY(need_ptr(b, "b"));
    NH_TRY(need_ptr(out, "out"));
    if (k != CONVK) return fail(NH_ERR_UNSUPPORTED_SHAPE, "conv kernel %d (only 4)", k);
    if (batch < 1 || channels < 1 || ld < channels)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d, channels %d, ld %ld", batch, channels, ld);
    NH_HIP(launch_conv_step(xbc, ld, conv_state, w, b, out, batch, channels, S(stream)), "conv step");
    return ok();
}

nh_status nh_conv1d_seq(const uint16_t *xbc, long ld, int T, const uint16_t *state_in, uint16_t *state_out,
                        const uint16_t *w, const uint16_t *b, uint16_t *out, int batch, int channels, int k,
                        void *stream)
{
    NH_TRY(need_ptr(xbc, "xbc"));
    NH_TRY(opt_ptr(state_in, "state_in"));
    NH_TRY(opt_ptr(state_out, "state_out"));
    NH_TRY(need_ptr(w, "w"));
    NH_TRY(need_ptr(b, "b"));
    NH_TRY(need_ptr(out, "out"));
    if (k != CONVK) return fail(NH_ERR_UNSUPPORTED_SHAPE, "conv kernel %d (only 4)", k);
    if (batch < 1 || channels < 1 || ld < channels || T < 1)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d, channels %d, ld %ld, T %d", batch, channels, ld, T);
    if (state_in && state_in == state_out)
        return fail(NH_ERR_INVALID_ARGUMENT, "state_out may not alias state_in");
    NH_HIP(launch_conv_seq(xbc, ld, T, state_in, state_out, w, b, out, batch, channels, S(stream)), "conv seq");
    return ok();
}

nh_status nh_ssm_step(const nh_mamba_dims *d, const uint16_t *xc, const uint16_t *dt_raw, long ld_dt,
                      const float *dt_bias, const float *A_log, const float *D, float *ssm_state, void *y,
                      nh_dtype y_dtype, int batch, void *stream)
{
    NH_TRY(check_dims(d, false));
    NH_TRY(need_ptr(xc, "xc"));
    if (!dt_raw) return fail(NH_ERR_INVALID_ARGUMENT, "dt_raw is NULL");
    NH_TRY(need_ptr(dt_bias, "dt_bias"));
    NH_TRY(need_ptr(A_log, "A_log"));
    NH_TRY(need_ptr(D, "D"));
    NH_TRY(need_ptr(ssm_state, "ssm_state"));
    NH_TRY(need_ptr(y, "y"));
    NH_TRY(need_dtype(y_dtype, "y_dtype"));
    if (batch < 1 || batch > 64) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..64", batch);
    if (batch > 1 && ld_dt < NHEADS) return fail(NH_ERR_UNSUPPORTED_SHAPE, "ld_dt %ld < n_heads", ld_dt);
    NH_HIP(launch_ssm_step(xc, dt_raw, ld_dt, dt_bias, A_log, D, ssm_state, y, y_dtype, batch, S(stream)),
           "ssm step");
    return ok();
}

size_t nh_ssd_scan_workspace_bytes(const nh_mamba_dims *d, int batch, int T)
{
    if (!d || batch < 1 || T < 1 || d->chunk < 1 || d->chunk > QMAX) return 0;
    return ssd_scan_ws_bytes(batch, T, d->chunk);
}

nh_status nh_ssd_chunk_scan(const nh_mamba_dims *d, const uint16_t *xc, const uint16_t *dt_raw, long ld_dt,
                            int T, const float *dt_bias, const float *A_log, const float *D, const float *h0,
                            float *h_final, void *y, nh_dtype y_dtype, int batch, void *ws, size_t ws_bytes,
                            void *stream)
{
    NH_TRY(check_dims(d, true));
    NH_TRY(need_ptr(xc, "xc"));
    if (!dt_raw) return fail(NH_ERR_INVALID_ARGUMENT, "dt_raw is NULL");
    NH_TRY(need_ptr(dt_bias, "dt_bias"));
    NH_TRY(need_ptr(A_log, "A_log"));
    NH_TRY(need_ptr(D, "D"));
    NH_TRY(opt_ptr(h0, "h0"));
    NH_TRY(opt_ptr(h_final, "h_final"));
    NH_TRY(need_ptr(y, "y"));
    NH_TRY(need_dtype(y_dtype, "y_dtype"));
    if (batch < 1 || T < 1) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d, T %d", batch, T);
    if (ld_dt < 1 || (T * (long)batch > 1 && ld_dt < NHEADS))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "ld_dt %ld < n_heads", ld_dt);
    NH_TRY(need_ptr(ws, "ws"));
    const size_t need = ssd_scan_ws_bytes(batch, T, d->chunk);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    NH_HIP(launch_ssd_scan(xc, dt_raw, ld_dt, T, d->chunk, dt_bias, A_log, D, h0, h_final, y, y_dtype, batch,
                           reinterpret_cast<uint16_t *>(ws), S(stream)),
           "ssd scan");
    return ok();
}

nh_status nh_rmsnorm_gated(const void *y, nh_dtype y_dtype, const uint16_t *z, long ld_z, const uint16_t *w,
                           uint16_t *out, int rows, int d, int group, float eps, void *stream)
{
    NH_TRY(need_ptr(y, "y"));
    NH_TRY(need_dtype(y_dtype, "y_dtype"));
    NH_TRY(need_ptr(z, "z"));
    NH_TRY(need_ptr(w, "w"));
    NH_TRY(need_ptr(out, "out"));
    if (rows < 1 || group < 8 || group % 8 || d % group || group > 8192 || ld_z < d || ld_z % 8)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "rows %d, d %d, group %d, ld_z %ld", rows, d, group, ld_z);
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive");
    NH_HIP(launch_rmsnorm_gated(y, y_dtype, z, ld_z, w, out, 0, nullptr, rows, d, group, eps, S(stream)), "gated norm");
    return ok();
}

size_t nh_block_workspace_bytes(const nh_mamba_dims *d, int batch, int T, int mode)
{
    if (!d || batch < 1) return 0;
    if (mode == NH_MODE_STEP) return batch <= 4 ? step_bytes(batch) : 0;
    if (mode == NH_MODE_SEQ) return T >= 1 ? seq_bytes(batch, T) : 0;
    return 0;
}

nh_status nh_mamba_block_step(const nh_mamba_dims *d, const nh_mamba_weights *w, nh_mamba_state *state,
                              const void *x, nh_dtype x_dtype, void *out, nh_dtype out_dtype, int batch,
                              void *ws, size_t ws_bytes, void *stream)
{
    NH_TRY(check_dims(d, false));
    NH_TRY(check_weights(w));
    NH_TRY(check_state(state, "state", true));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(out, "out"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_dtype(out_dtype, "out_dtype"));
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    if (x == out) return fail(NH_ERR_INVALID_ARGUMENT, "out may not alias x");
    NH_TRY(need_ptr(ws, "ws"));
    const size_t need = step_bytes(batch);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    return block_step(d, w, state, x, x_dtype, out, out_dtype, batch, ws, S(stream));
}

nh_status nh_mamba_block_step_noalloc(const nh_mamba_dims *d, const nh_mamba_weights *w, nh_mamba_state *state,
                                      const void *x, nh_dtype x_dtype, void *out, nh_dtype out_dtype, int batch,
                                      void *stream)
{
    NH_TRY(check_dims(d, false));
    NH_TRY(check_weights(w));
    NH_TRY(check_state(state, "state", true));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(out, "out"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_dtype(out_dtype, "out_dtype"));
    if (batch < 1 || batch > 4)
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4 (the allocation-free scratch holds the "
                    "step workspace of at most 4 sequences)", batch);
    if (x == out) return fail(NH_ERR_INVALID_ARGUMENT, "out may not alias x");
    void *scr = nullptr;
    size_t cap = 0;
    NH_HIP(noalloc_scratch(&scr, &cap), "allocation-free scratch lookup");
    if (step_bytes(batch) > cap)
        return fail(NH_ERR_WORKSPACE_TOO_SMALL, "step workspace %zu exceeds the allocation-free scratch (%zu bytes)",
                    step_bytes(batch), cap);
    return block_step(d, w, state, x, x_dtype, out, out_dtype, batch, scr, S(stream));
}

nh_status nh_inproj_conv_step(const nh_mamba_dims *d, const nh_mamba_weights *w, nh_mamba_state *state,
                              const void *x, nh_dtype x_dtype, uint16_t *z, uint16_t *xc, uint16_t *dt_raw,
                              int batch, void *stream)
{
    NH_TRY(check_dims(d, false));
    NH_TRY(check_weights(w));
    NH_TRY(check_state(state, "state", true));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(z, "z"));
    NH_TRY(need_ptr(xc, "xc"));
    NH_TRY(need_ptr(dt_raw, "dt_raw"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    if (x == (const void *)z || x == (const void *)xc || x == (const void *)dt_raw)
        return fail(NH_ERR_INVALID_ARGUMENT, "outputs may not alias x");
    NH_HIP(launch_inproj_step(view(&w->in_proj), x, x_dtype, w->norm_w, d->eps, batch, z, xc, dt_raw,
                              state->conv_state, w->conv_w, w->conv_b, nullptr, 0, S(stream)),
           "in_proj step");
    return ok();
}

nh_status nh_mamba_block_seq(const nh_mamba_dims *d, const nh_mamba_weights *w, const nh_mamba_state *init,
                             nh_mamba_state *final_state, const void *x, nh_dtype x_dtype, int T, void *out,
                             nh_dtype out_dtype, int batch, void *ws, size_t ws_bytes, void *stream)
{
    NH_TRY(check_dims(d, true));
    NH_TRY(check_weights(w));
    NH_TRY(check_state(init, "init", false));
    NH_TRY(check_state(final_state, "final_state", false));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(out, "out"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_dtype(out_dtype, "out_dtype"));
    if (batch < 1 || T < 1) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d, T %d", batch, T);
    if ((long)batch * T > (1L << 24)) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch*T too large");
    if (x == out) return fail(NH_ERR_INVALID_ARGUMENT, "out may not alias x");
    NH_TRY(need_ptr(ws, "ws"));
    const size_t need = seq_bytes(batch, T);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    return block_seq(d, w, init, final_state, x, x_dtype, T, out, out_dtype, batch, ws, S(stream));
}

nh_status nh_mamba_stack(const nh_mamba_dims *d, const nh_mamba_weights *weights, nh_mamba_state *states,
                         int n_layers, int mode, const void *x, nh_dtype x_dtype, int T, float *outs, int batch,
                         void *ws, size_t ws_bytes, void *stream)
{
    if (mode != NH_MODE_STEP && mode != NH_MODE_SEQ) return fail(NH_ERR_INVALID_ARGUMENT, "mode %d", mode);
    NH_TRY(check_dims(d, mode == NH_MODE_SEQ));
    if (!weights || n_layers < 1) return fail(NH_ERR_INVALID_ARGUMENT, "weights NULL or n_layers %d", n_layers);
    if (mode == NH_MODE_STEP && !states) return fail(NH_ERR_INVALID_ARGUMENT, "states is NULL");
    for (int i = 0; i < n_layers; ++i) {
        NH_TRY(check_weights(&weights[i]));
        if (states) NH_TRY(check_state(&states[i], "state", true));
    }
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_ptr(outs, "outs"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    if (batch < 1 || T < 1) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d, T %d", batch, T);
    if (mode == NH_MODE_STEP && (T != 1 || batch > 4))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "step mode needs T == 1 and batch <= 4");
    if (x == (const void *)outs) return fail(NH_ERR_INVALID_ARGUMENT, "outs may not alias x");
    NH_TRY(need_ptr(ws, "ws"));
    const size_t need = mode == NH_MODE_STEP ? step_bytes(batch) : seq_bytes(batch, T);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    const size_t per = (size_t)batch * T * HIDDEN;
    for (int i = 0; i < n_layers; ++i) {
        const void *xi = i == 0 ? x : (const void *)(outs + (i - 1) * per);
        const int xt = i == 0 ? x_dtype : NH_F32;
        nh_status s;
        if (mode == NH_MODE_STEP)
            s = block_step(d, &weights[i], &states[i], xi, xt, outs + i * per, NH_F32, batch, ws, S(stream));
        else
            s = block_seq(d, &weights[i], states ? &states[i] : nullptr, states ? &states[i] : nullptr, xi, xt, T,
                          outs + i * per, NH_F32, batch, ws, S(stream));
        if (s != NH_OK) return s;
    }
    return ok();
}

size_t nh_attention_workspace_bytes(int batch)
{
    if (batch < 1 || batch > 4) return 0;
    return attention_bytes(batch);
}

nh_status nh_attention_step(const nh_attention_weights *w, const nh_kv_cache *cache, const int32_t *positions,
                            const void *x, nh_dtype x_dtype, void *out, nh_dtype out_dtype, int batch, float eps,
                            void *ws, size_t ws_bytes, void *stream)
{
    NH_TRY(check_attention(w));
    NH_TRY(check_cache(cache));
    NH_TRY(need_ptr(positions, "positions"));
    NH_TRY(need_ptr(x, "x"));
    NH_TRY(need_dtype(x_dtype, "x_dtype"));
    NH_TRY(need_ptr(out, "out"));
    NH_TRY(need_dtype(out_dtype, "out_dtype"));
    NH_TRY(need_ptr(ws, "ws"));
    if (out == x) return fail(NH_ERR_INVALID_ARGUMENT, "out may not alias x");
    if (!(eps > 0.f) || !std::isfinite(eps)) return fail(NH_ERR_INVALID_ARGUMENT, "eps must be positive");
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    const size_t need = attention_bytes(batch);
    if (ws_bytes < need)
        return fail(NH_ERR_WORKSPACE_TOO_SMALL, "attention workspace %zu < %zu bytes", ws_bytes, need);
    NH_TRY(attention_step(w, cache, positions, x, x_dtype, out, out_dtype, batch, eps, ws, S(stream)));
    return ok();
}

size_t nh_attention_decode_workspace_bytes(int batch)
{
    if (batch < 1 || batch > 64) return 0;
    return attn_part_bytes(batch);
}

nh_status nh_attention_decode(const uint16_t *q, const nh_kv_cache *cache, const int32_t *positions, uint16_t *o,
                              int batch, void *ws, size_t ws_bytes, void *stream)
{
    NH_TRY(need_ptr(q, "q"));
    NH_TRY(check_cache(cache));
    NH_TRY(need_ptr(positions, "positions"));
    NH_TRY(need_ptr(o, "o"));
    NH_TRY(need_ptr(ws, "ws"));
    if (batch < 1 || batch > 64) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..64", batch);
    const size_t need = attn_part_bytes(batch);
    if (ws_bytes < need)
        return fail(NH_ERR_WORKSPACE_TOO_SMALL, "attention workspace %zu < %zu bytes", ws_bytes, need);
    NH_HIP(launch_attn_decode(q, cache->k, cache->v, positions, cache->max_len, batch,
                              reinterpret_cast<float *>(ws), o, S(stream)),
           "attention");
    return ok();
}

static const int NH_N_MAMBA = 27, NH_N_MLP = 25, NH_N_ATT = 4;

size_t nh_lm_workspace_bytes(const nh_mamba_dims *d, int inter, int batch)
{
    if (!d || batch < 1 || batch > 4 || nh_mlp_workspace_bytes(inter, batch) == 0) return 0;
    size_t scratch = step_bytes(batch);
    scratch = std::max(scratch, nh_mlp_workspace_bytes(inter, batch));
    scratch = std::max(scratch, head_ws_bytes(batch));
    scratch = std::max(scratch, attention_bytes(batch));
    Carve c{nullptr};
    c.take<float>((size_t)batch * HIDDEN);
    c.take<float>((size_t)batch * HIDDEN);
    c.take<char>(scratch);
    return c.off;
}

nh_status nh_lm_step(const nh_mamba_dims *d, const nh_lm_weights *w, nh_mamba_state *states,
                     const nh_kv_cache *caches, const int32_t *positions, const int32_t *text_ids,
                     const int32_t *function_ids, const void *audio, nh_dtype audio_dtype, int batch,
                     float *hidden_out, int32_t *text_out, int32_t *function_out, void *ws, size_t ws_bytes,
                     void *stream)
{
    NH_TRY(check_dims(d, false));
    if (!w || !w->mamba || !w->mlp || !w->attn || !states || !caches)
        return fail(NH_ERR_INVALID_ARGUMENT, "weights, their layer arrays, states and caches must be non-NULL");
    NH_TRY(check_w4(&w->embed, "embed"));
    NH_TRY(check_w4(&w->lm_head, "lm_head"));
    NH_TRY(check_w4(&w->function_head, "function_head"));
    if (w->embed.k_in != HIDDEN || w->lm_head.k_in != HIDDEN || w->function_head.k_in != HIDDEN ||
        w->lm_head.n_out > (1 << 19) || w->function_head.n_out > (1 << 19))
        return fail(NH_ERR_UNSUPPORTED_SHAPE, "embedding and heads need k_in == %d and heads n_out <= 524288", HIDDEN);
    NH_TRY(need_ptr(w->norm_f, "norm_f"));
    if (!std::isfinite(w->function_weight)) return fail(NH_ERR_INVALID_ARGUMENT, "function_weight must be finite");
    for (int i = 0; i < NH_N_MAMBA; ++i) {
        NH_TRY(check_weights(&w->mamba[i]));
        NH_TRY(check_state(&states[i], "state", true));
    }
    const int inter = w->mlp[0].up.n_out;
    for (int i = 0; i < NH_N_MLP; ++i) {
        const nh_mlp_weights &m = w->mlp[i];
        NH_TRY(need_ptr(m.norm_w, "mlp norm_w"));
        NH_TRY(check_w4(&m.up, "mlp up"));
        NH_TRY(check_w4(&m.down, "mlp down"));
        if (m.up.k_in != HIDDEN || m.down.n_out != HIDDEN || m.up.n_out != inter || m.down.k_in != inter)
            return fail(NH_ERR_UNSUPPORTED_SHAPE, "mlp layer %d: up %d x %d, down %d x %d", i, m.up.n_out, m.up.k_in,
                        m.down.n_out, m.down.k_in);
    }
    for (int i = 0; i < NH_N_ATT; ++i) {
        NH_TRY(check_attention(&w->attn[i]));
        NH_TRY(check_cache(&caches[i]));
    }
    NH_TRY(need_ptr(positions, "positions"));
    NH_TRY(need_ptr(text_ids, "text_ids"));
    NH_TRY(need_ptr(function_ids, "function_ids"));
    NH_TRY(need_ptr(audio, "audio"));
    NH_TRY(need_dtype(audio_dtype, "audio_dtype"));
    NH_TRY(opt_ptr(hidden_out, "hidden_out"));
    NH_TRY(need_ptr(text_out, "text_out"));
    NH_TRY(need_ptr(function_out, "function_out"));
    NH_TRY(need_ptr(ws, "ws"));
    if (batch < 1 || batch > 4) return fail(NH_ERR_UNSUPPORTED_SHAPE, "batch %d outside 1..4", batch);
    const size_t need = nh_lm_workspace_bytes(d, inter, batch);
    if (need == 0) return fail(NH_ERR_UNSUPPORTED_SHAPE, "mlp width %d", inter);
    if (ws_bytes < need) return fail(NH_ERR_WORKSPACE_TOO_SMALL, "lm workspace %zu < %zu bytes", ws_bytes, need);

    Carve c{reinterpret_cast<char *>(ws)};
    float *cur = c.take<float>((size_t)batch * HIDDEN);
    float *nxt = c.take<float>((size_t)batch * HIDDEN);
    void *scratch = c.take<char>(1);
    const hipStream_t s = S(stream);
    NH_HIP(launch_fused_embed(view(&w->embed), text_ids, function_ids, audio, audio_dtype, w->function_weight, batch,
                              cur, s),
           "input row");
    const char *pat = nh_hybrid_pattern();
    int mi = 0, li = 0, ai = 0;
    for (const char *p = pat; *p; ++p) {
        if (*p == 'M') {
            NH_TRY(block_step(d, &w->mamba[mi], &states[mi], cur, NH_F32, nxt, NH_F32, batch, scratch, s));
            ++mi;
        } else if (*p == '-') {
            const nh_mlp_weights &m = w->mlp[li++];
            uint16_t *h = reinterpret_cast<uint16_t *>(scratch);
            NH_HIP(launch_mlp_up_step(view(&m.up), cur, F32, m.norm_w, d->eps, batch, h, s), "mlp up");
            NH_HIP(launch_gemv(view(&m.down), h, BF16, batch, cur, F32, nxt, F32, s), "mlp down");
        } else {
            NH_TRY(attention_step(&w->attn[ai], &caches[ai], positions, cur, F32, nxt, F32, batch, d->eps, scratch,
                                  s));
            ++ai;
        }
        std::swap(cur, nxt);
    }
    if (hidden_out)
        NH_HIP(hipMemcpyAsync(hidden_out, cur, (size_t)batch * HIDDEN * sizeof(float), hipMemcpyDeviceToDevice, s),
               "hidden copy");
    NH_HIP(launch_head(view(&w->lm_head), cur, F32, w->norm_f, d->eps, batch, nullptr, text_out, scratch, s),
           "lm_head");
    NH_HIP(launch_head(view(&w->function_head), cur, F32, w->norm_f, d->eps, batch, nullptr, function_out, scratch,
                       s),
           "function_head");
    return ok();
}

}  // extern "C"
