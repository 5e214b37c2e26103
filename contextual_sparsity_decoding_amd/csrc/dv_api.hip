// C-ABI entry points of libdv: argument validation (host only, before any
// launch), workspace sizing and the order of kernel launches.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157); ByteCross = "Where Activation Sparsity
// and KV-Cache Sparsity Cross in LLM Decoding" (arXiv 2609.33889v1).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "pred.h"
#include "topk_split.h"
#include "w4.h"

namespace dvh {

static thread_local char g_err[512];

dv_status fail(dv_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

// dv_time_launches state (per host thread)
struct LaunchTiming {
    int kind = 0;
    hipEvent_t* ev = nullptr;
    int n = 0, used = 0;
    bool armed = false, taken = false;
};
static thread_local LaunchTiming g_timing;

// The role's events: the start is recorded on the stream at once; the first
// launch through DV_LAUNCH inside the role takes both, so that they mark that
// kernel's own start and end; otherwise the end is recorded after the role.
void timed_begin(int kind, hipStream_t s) {
    if (kind != 0 && kind == g_timing.kind && g_timing.used + 2 <= g_timing.n) {
        (void)hipEventRecord(g_timing.ev[g_timing.used], s);
        g_timing.armed = true;
        g_timing.taken = false;
    }
}
bool timed_take(hipEvent_t* ev) {
    if (!g_timing.armed) return false;
    g_timing.armed = false;
    g_timing.taken = true;
    ev[0] = g_timing.ev[g_timing.used];
    ev[1] = g_timing.ev[g_timing.used + 1];
    return true;
}
void timed_end(int kind, hipStream_t s) {
    if (kind != 0 && kind == g_timing.kind && g_timing.used + 2 <= g_timing.n) {
        if (!g_timing.taken) (void)hipEventRecord(g_timing.ev[g_timing.used + 1], s);
        g_timing.used += 2;
    }
    g_timing.armed = g_timing.taken = false;
}

int elt_bytes(int wdt) { return wdt == DV_F16 ? 2 : 4; }

static bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool wdt_ok(int wdt) { return wdt == DV_F16 || wdt == DV_F32; }
static bool dh_ok(int d_h) { return d_h == 32 || d_h == 64 || d_h == 128 || d_h == 256; }
// one counter per output column slice (64 lanes x 16 bytes) must fit the counter block
static bool d_ok(int d) { return d >= 1 && (long)d <= (long)(kMaxCounters - 1) * 256; }
static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const char* x = (const char*)a;
    const char* y = (const char*)b;
    return a && b && x < y + nb && y < x + na;
}

#define REQ(cond, code, ...)                 \
    do {                                     \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)
#define TRY(expr)                            \
    do {                                     \
        dv_status st_ = (expr);              \
        if (st_ != DV_OK) return st_;        \
    } while (0)
#define HIP_TRY(expr)                                                                   \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) return fail(DV_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// ---- workspace layouts ------------------------------------------------------

static size_t predict_ws(int B, int d, int r, int wdt) {
    return kCounterBytes + align_up(pred_partials(B, d, r, wdt) * 4, 256);
}
static float* predict_part(void* ws) { return ws ? (float*)((char*)ws + kCounterBytes) : nullptr; }

struct MlpWs {
    float* a;
    float* partial;
    float* mpart;             // the matrix-core fc1's partial sums (batches of 8-16), or NULL
    size_t bytes;
};
static MlpWs mlp_ws(void* ws, int B, int d, int n_idx_max, int wdt, bool need_a) {
    Carve cv(ws);
    MlpWs w;
    w.a = need_a ? cv.take<float>((size_t)B * (n_idx_max > 0 ? n_idx_max : 1)) : nullptr;
    const AxpyPlan p = axpy_plan(d, n_idx_max, wdt);
    w.partial = cv.take<float>(axpy_ws_floats(p, B, d));
    w.mpart = rowdot_mfma_ok(B, d, wdt) ? cv.take<float>(rowdot_mfma_part_floats(n_idx_max)) : nullptr;
    w.bytes = align_up(cv.off, 256);
    return w;
}

struct ProjWs {
    float* partial;
    size_t bytes;
};
static ProjWs proj_ws(void* ws, int mode, int B, int d, int n_sel, int d_h, int wdt) {
    Carve cv(ws);
    ProjWs w{nullptr, 0};
    if (mode == DV_PROJ_OUT) {
        const AxpyPlan p = axpy_plan(d, n_sel * d_h, wdt);
        w.partial = cv.take<float>(axpy_ws_floats(p, B, d));
    }
    w.bytes = align_up(cv.off, 256);
    return w;
}

static size_t splitk_ws(int B, int n_sel, int d_h, int max_positions, int num_splits) {
    if (num_splits <= 0) num_splits = splitk_auto(max_positions, B * n_sel);
    return kCounterBytes + align_up((size_t)B * n_sel * num_splits * (d_h + 2) * 4, 256);
}

// The sparse MLP behind dv_sparse_mlp and its no-allocation variant: the
// arguments checked, then fc1 and fc2 with scratch carved from ws.
dv_status sparse_mlp_call(const char* who, const float* y, int B, int d, int N, const void* w1_t, const void* b1,
                          const void* w2_t, const void* b2, int wdt, const int32_t* idx, int n_idx_max,
                          const int32_t* n_idx_dev, const float* residual, float* out, float* act_out,
                          int32_t* fc2_rows, unsigned flags, void* ws, size_t ws_bytes, hipStream_t s, bool run) {
    REQ(y && w1_t && b1 && w2_t && b2 && out, DV_ERR_NULL, "%s: NULL pointer", who);
    REQ(wdt_ok(wdt), DV_ERR_DTYPE, "%s: wdt %d", who, wdt);
    REQ(B >= 1 && B <= 16 && d_ok(d) && N >= 1, DV_ERR_SHAPE, "%s: B=%d d=%d N=%d", who, B, d, N);
    REQ(n_idx_max >= 0 && n_idx_max <= N, DV_ERR_RANGE, "%s: n_idx_max=%d N=%d", who, n_idx_max, N);
    REQ(idx || n_idx_max == N, DV_ERR_SHAPE, "%s: idx NULL needs n_idx_max == N", who);
    REQ((flags & ~(unsigned)DV_SKIP_NONPOS_FC2) == 0, DV_ERR_DTYPE, "%s: flags 0x%x", who, flags);
    REQ((size_t)d * elt_bytes(wdt) % 16 == 0, DV_ERR_ALIGN, "%s: d=%d rows not 16-byte multiples", who, d);
    REQ(a16(w1_t) && a16(w2_t) && a16(y), DV_ERR_ALIGN, "%s: pointers must be 16-byte aligned", who);
    const size_t act_bytes = (size_t)B * d * 4;
    REQ(!overlap(out, act_bytes, y, act_bytes) && !overlap(out, act_bytes, residual, act_bytes), DV_ERR_RANGE,
        "%s: out overlaps y or residual", who);
    const MlpWs w = mlp_ws(ws, B, d, n_idx_max, wdt, act_out == nullptr);
    REQ(ws && ws_bytes >= w.bytes, DV_ERR_WORKSPACE, "%s: workspace %zu < %zu", who, ws_bytes, w.bytes);
    if (!run) return DV_OK;
    float* a = act_out ? act_out : w.a;
    if (w.mpart) TRY(launch_fc1_mfma(y, B, d, w1_t, b1, idx, n_idx_max, n_idx_dev, N, a, w.mpart, s));
    else TRY(launch_fc1(y, B, d, w1_t, b1, wdt, idx, n_idx_max, n_idx_dev, N, a, s));
    AxpyCall c{};
    c.w = w2_t; c.wdt = wdt; c.d = d; c.w_rows = N; c.rows = n_idx_max; c.n_rows_dev = n_idx_dev; c.idx = idx; c.blk = 1;
    c.coef = a; c.coef_stride = n_idx_max; c.skip_zero = (flags & DV_SKIP_NONPOS_FC2) != 0;
    c.B = B; c.bias = b2; c.residual = residual; c.out = out; c.rows_read = fc2_rows; c.partial = w.partial;
    return launch_axpy(c, s);
}

}  // namespace dvh

using namespace dvh;

extern "C" {

int dv_api_version(void) { return DV_API_VERSION; }

const char* dv_status_str(int s) {
    switch (s) {
        case DV_OK: return "DV_OK";
        case DV_ERR_NULL: return "DV_ERR_NULL";
        case DV_ERR_SHAPE: return "DV_ERR_SHAPE";
        case DV_ERR_DTYPE: return "DV_ERR_DTYPE";
        case DV_ERR_ALIGN: return "DV_ERR_ALIGN";
        case DV_ERR_RANGE: return "DV_ERR_RANGE";
        case DV_ERR_WORKSPACE: return "DV_ERR_WORKSPACE";
        case DV_ERR_UNSUPPORTED: return "DV_ERR_UNSUPPORTED";
        case DV_ERR_HIP: return "DV_ERR_HIP";
        default: return "DV_ERR_UNKNOWN";
    }
}

const char* dv_last_error(void) { return g_err; }

// ---------------------------------------------------------------- LayerNorm --
dv_status dv_layernorm(const float* x, int B, int d, const float* gamma, const float* beta, float eps,
                       float* y, void* stream) {
    clear_error();
    REQ(x && gamma && beta && y, DV_ERR_NULL, "dv_layernorm: NULL pointer");
    REQ(B >= 1 && d >= 1, DV_ERR_SHAPE, "dv_layernorm: B=%d d=%d", B, d);
    REQ(eps >= 0.f && isfinite(eps), DV_ERR_RANGE, "dv_layernorm: eps");
    return launch_layernorm(x, B, d, gamma, beta, eps, y, (hipStream_t)stream);
}

// ---------------------------------------------------------------- predictor --
size_t dv_predict_workspace_bytes(int B, int d, int r, int wdt) {
    if (B < 1 || d < 1 || r < 1 || !wdt_ok(wdt)) return 0;
    return predict_ws(B, d, r, wdt);
}

static dv_status check_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                               int n_out, int wdt, int act, const float* scores) {
    REQ(y && p1_t && p2_t && scores, DV_ERR_NULL, "dv_predict: NULL pointer");
    REQ(wdt_ok(wdt), DV_ERR_DTYPE, "dv_predict: wdt %d", wdt);
    REQ(act == DV_ACT_NONE || act == DV_ACT_RELU, DV_ERR_DTYPE, "dv_predict: act %d", act);
    REQ(B >= 1 && B <= 16 && d >= 1 && r >= 1 && r <= 512 && n_out >= 1, DV_ERR_SHAPE,
        "dv_predict: B=%d d=%d r=%d n_out=%d", B, d, r, n_out);
    const int eb = elt_bytes(wdt);
    REQ((size_t)d * eb % 16 == 0 && (size_t)r * eb % 16 == 0, DV_ERR_ALIGN,
        "dv_predict: rows of d=%d and r=%d elements must be multiples of 16 bytes", d, r);
    REQ(a16(p1_t) && a16(p2_t) && a16(y), DV_ERR_ALIGN, "dv_predict: pointers must be 16-byte aligned");
    return DV_OK;
}

dv_status dv_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t, int n_out, int wdt,
                     int act, float* scores, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    TRY(check_predict(y, B, d, p1_t, r, p2_t, n_out, wdt, act, scores));
    REQ(ws && ws_bytes >= predict_ws(B, d, r, wdt), DV_ERR_WORKSPACE, "dv_predict: workspace");
    return launch_predict(y, B, d, p1_t, r, p2_t, n_out, wdt, act, scores, predict_part(ws), (hipStream_t)stream);
}

// ---------------------------------------------------------------- top-k -----
size_t dv_topk_workspace_bytes(int B, int n, int k) {
    (void)B; (void)n; (void)k;
    return 0;
}

dv_status dv_topk_select(const float* scores, int B, int n, int k, int32_t* idx, int32_t* union_idx,
                         int32_t* union_count, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    (void)ws; (void)ws_bytes;
    REQ(B >= 1 && B <= 64 && n >= 0 && n <= dv::kTopkMaxN, DV_ERR_SHAPE, "dv_topk_select: B=%d n=%d", B, n);
    REQ(k >= 0 && k <= n, DV_ERR_RANGE, "dv_topk_select: k=%d outside [0, n=%d]", k, n);
    REQ(k == 0 || (scores && idx), DV_ERR_NULL, "dv_topk_select: NULL pointer");
    REQ((union_idx == nullptr) == (union_count == nullptr), DV_ERR_NULL,
        "dv_topk_select: union_idx and union_count go together");
    REQ(union_idx == nullptr || n <= dv::kUnionMaxN, DV_ERR_SHAPE, "dv_topk_select: union over n=%d > %d", n, dv::kUnionMaxN);
    hipStream_t s = (hipStream_t)stream;
    TRY(launch_topk(scores, B, n, k, idx, s));
    if (union_idx) TRY(launch_union(idx, B, k, n, union_idx, union_count, s));
    return DV_OK;
}

// ---------------------------------------------------------------- MLP -------
size_t dv_sparse_mlp_workspace_bytes(int B, int d, int n_idx_max, int wdt) {
    if (B < 1 || d < 1 || n_idx_max < 0 || !wdt_ok(wdt)) return 0;
    return mlp_ws(nullptr, B, d, n_idx_max, wdt, true).bytes;
}

dv_status dv_sparse_mlp(const float* y, int B, int d, int N, const void* w1_t, const void* b1, const void* w2_t,
                        const void* b2, int wdt, const int32_t* idx, int n_idx_max, const int32_t* n_idx_dev,
                        const float* residual, float* out, float* act_out, int32_t* fc2_rows, unsigned flags,
                        void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    return sparse_mlp_call("dv_sparse_mlp", y, B, d, N, w1_t, b1, w2_t, b2, wdt, idx, n_idx_max, n_idx_dev, residual,
                           out, act_out, fc2_rows, flags, ws, ws_bytes, (hipStream_t)stream);
}

// ---------------------------------------------------------------- projections --
size_t dv_attn_proj_workspace_bytes(int mode, int B, int d, int h, int d_h, int n_sel, int wdt) {
    (void)h;
    if ((mode != DV_PROJ_QKV && mode != DV_PROJ_OUT) || B < 1 || d < 1 || d_h < 1 || n_sel < 0 || !wdt_ok(wdt))
        return 0;
    return proj_ws(nullptr, mode, B, d, n_sel, d_h, wdt).bytes;
}

dv_status dv_sparse_attn_proj(int mode, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                              const void* w_t, const void* bias, int wdt, const float* in, const float* residual,
                              float* out, const dv_kv_state* kv, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    REQ(mode == DV_PROJ_QKV || mode == DV_PROJ_OUT, DV_ERR_DTYPE, "dv_sparse_attn_proj: mode %d", mode);
    REQ(wdt_ok(wdt), DV_ERR_DTYPE, "dv_sparse_attn_proj: wdt %d", wdt);
    REQ(w_t && in && out, DV_ERR_NULL, "dv_sparse_attn_proj: NULL pointer");
    REQ(B >= 1 && B <= 16 && d_ok(d) && h >= 1 && dh_ok(d_h), DV_ERR_SHAPE,
        "dv_sparse_attn_proj: B=%d d=%d h=%d d_h=%d", B, d, h, d_h);
    REQ(n_sel >= 0 && n_sel <= h, DV_ERR_RANGE, "dv_sparse_attn_proj: n_sel=%d h=%d", n_sel, h);
    REQ((size_t)d * elt_bytes(wdt) % 16 == 0, DV_ERR_ALIGN, "dv_sparse_attn_proj: d=%d rows", d);
    REQ(a16(w_t) && a16(in), DV_ERR_ALIGN, "dv_sparse_attn_proj: pointers must be 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const ProjWs w = proj_ws(ws, mode, B, d, n_sel, d_h, wdt);
    if (mode == DV_PROJ_QKV) {
        REQ(kv && kv->k_cache && kv->v_cache && bias, DV_ERR_NULL, "dv_sparse_attn_proj: QKV needs kv and bias");
        REQ(kv->max_len >= 1 && kv->pos >= 0 && kv->pos < kv->max_len, DV_ERR_RANGE,
            "dv_sparse_attn_proj: pos=%d max_len=%d", kv->pos, kv->max_len);
        REQ(!overlap(out, (size_t)B * n_sel * d_h * 4, in, (size_t)B * d * 4), DV_ERR_RANGE,
            "dv_sparse_attn_proj: q overlaps y");
        REQ(qkv_supported(B, d, wdt), DV_ERR_UNSUPPORTED, "dv_sparse_attn_proj: d=%d rows too long", d);
        REQ(!kv->y_buf || a16(kv->y_buf), DV_ERR_ALIGN, "dv_sparse_attn_proj: y_buf must be 16-byte aligned");
        return launch_qkv(in, B, d, h, d_h, head_idx, n_sel, w_t, bias, wdt, out, kv, true, s);
    }
    REQ(ws && ws_bytes >= w.bytes, DV_ERR_WORKSPACE, "dv_sparse_attn_proj: workspace %zu < %zu", ws_bytes, w.bytes);
    REQ(!overlap(out, (size_t)B * d * 4, in, (size_t)B * n_sel * d_h * 4) &&
            !overlap(out, (size_t)B * d * 4, residual, (size_t)B * d * 4),
        DV_ERR_RANGE, "dv_sparse_attn_proj: out overlaps o or residual");
    AxpyCall c{};
    c.w = w_t; c.wdt = wdt; c.d = d; c.w_rows = h * d_h; c.rows = n_sel * d_h; c.idx = head_idx; c.blk = d_h;
    c.coef = in; c.coef_stride = n_sel * d_h; c.B = B; c.bias = bias; c.residual = residual; c.out = out;
    c.partial = w.partial;
    return launch_axpy(c, s);
}

// ---------------------------------------------------------------- attention --
size_t dv_splitk_workspace_bytes(int B, int n_sel, int d_h, int max_positions, int num_splits) {
    if (B < 1 || n_sel < 0 || d_h < 1 || max_positions < 0 || num_splits < 0) return 0;
    return splitk_ws(B, n_sel, d_h, max_positions, num_splits);
}

static dv_status check_view(const dv_kv_view* kv, const char* who) {
    REQ(kv && kv->k_cache && kv->v_cache, DV_ERR_NULL, "%s: kv view NULL", who);
    REQ(kv->h >= 1 && kv->max_len >= 1, DV_ERR_SHAPE, "%s: h=%d max_len=%d", who, kv->h, kv->max_len);
    REQ(kv->n_ctx >= 1 && kv->n_ctx <= kv->max_len, DV_ERR_RANGE, "%s: n_ctx=%d max_len=%d", who, kv->n_ctx,
        kv->max_len);
    if (kv->sel_idx) {
        REQ(kv->sel_len, DV_ERR_NULL, "%s: sel_len NULL", who);
        REQ(kv->sel_end >= 0 && kv->sel_end <= kv->n_ctx && kv->sel_cap >= 0 && kv->sel_cap <= kv->sel_end,
            DV_ERR_RANGE, "%s: sel_cap=%d sel_end=%d n_ctx=%d", who, kv->sel_cap, kv->sel_end, kv->n_ctx);
    }
    REQ(kv->win_len >= 0 && kv->win_sink >= 0, DV_ERR_RANGE, "%s: win_sink=%d win_len=%d", who, kv->win_sink,
        kv->win_len);
    REQ(!(kv->sel_idx && kv->win_len > 0), DV_ERR_UNSUPPORTED, "%s: a KV window and retained positions together", who);
    return DV_OK;
}

dv_status dv_splitk_attn(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel, const dv_kv_view* kv,
                         float scale, int num_splits, float* o, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    REQ(q && o, DV_ERR_NULL, "dv_splitk_attn: NULL pointer");
    TRY(check_view(kv, "dv_splitk_attn"));
    REQ(B >= 1 && dh_ok(d_h), DV_ERR_SHAPE, "dv_splitk_attn: B=%d d_h=%d", B, d_h);
    REQ(n_sel >= 0 && n_sel <= kv->h, DV_ERR_RANGE, "dv_splitk_attn: n_sel=%d h=%d", n_sel, kv->h);
    REQ(isfinite(scale), DV_ERR_RANGE, "dv_splitk_attn: scale");
    REQ(num_splits >= 0 && num_splits <= 65536, DV_ERR_RANGE, "dv_splitk_attn: num_splits=%d", num_splits);
    REQ((long)B * n_sel * (num_splits > 0 ? num_splits : 1) <= (1L << 26), DV_ERR_RANGE, "dv_splitk_attn: too many splits");
    const size_t need = splitk_ws(B, n_sel, d_h, view_positions(kv), num_splits);
    REQ(ws && ws_bytes >= need, DV_ERR_WORKSPACE, "dv_splitk_attn: workspace %zu < %zu", ws_bytes, need);
    return launch_splitk(q, B, d_h, head_idx, n_sel, kv, kv->n_ctx_dev, 0, scale, num_splits, o,
                         (float*)((char*)ws + kCounterBytes), nullptr, 0, nullptr, (hipStream_t)stream);
}

// ---------------------------------------------------------------- 4-bit weights --
dv_status dv_quantize_w4(const void* w, int rows, int cols, uint8_t* q, void* scales, void* stream) {
    clear_error();
    REQ(w && q && scales, DV_ERR_NULL, "dv_quantize_w4: NULL pointer");
    REQ(rows >= 1 && cols >= 128 && cols % 128 == 0, DV_ERR_SHAPE, "dv_quantize_w4: rows=%d cols=%d", rows, cols);
    REQ(a16(w) && a16(q), DV_ERR_ALIGN, "dv_quantize_w4: pointers must be 16-byte aligned");
    return launch_quant_w4(w, rows, cols, q, scales, (hipStream_t)stream);
}

static size_t w4_ws(int d, int n_idx_max, float** a, float** partial, void* ws) {
    Carve cv(ws);
    *a = cv.take<float>((size_t)(n_idx_max > 0 ? n_idx_max : 1));
    *partial = cv.take<float>((size_t)w4_axpy_groups(n_idx_max) * d);
    return align_up(cv.off, 256);
}

size_t dv_sparse_mlp_w4_workspace_bytes(int d, int n_idx_max) {
    if (d < 128 || d % 128 || n_idx_max < 0) return 0;
    float *a, *p;
    return w4_ws(d, n_idx_max, &a, &p, nullptr);
}

dv_status dv_sparse_mlp_w4(const float* y, int d, int N, const uint8_t* q1, const void* s1, const void* b1,
                           const uint8_t* q2, const void* s2, const void* b2, const int32_t* idx, int n_idx_max,
                           const int32_t* n_idx_dev, const float* residual, float* out, float* act_out,
                           int32_t* fc2_rows, unsigned flags, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    REQ(y && q1 && s1 && b1 && q2 && s2 && b2 && out, DV_ERR_NULL, "dv_sparse_mlp_w4: NULL pointer");
    REQ(d >= 128 && d % 128 == 0 && d <= 16384 && N >= 1, DV_ERR_SHAPE, "dv_sparse_mlp_w4: d=%d N=%d", d, N);
    REQ(n_idx_max >= 0 && n_idx_max <= N, DV_ERR_RANGE, "dv_sparse_mlp_w4: n_idx_max=%d N=%d", n_idx_max, N);
    REQ(idx || n_idx_max == N, DV_ERR_SHAPE, "dv_sparse_mlp_w4: idx NULL needs n_idx_max == N");
    REQ((flags & ~(unsigned)DV_SKIP_NONPOS_FC2) == 0, DV_ERR_DTYPE, "dv_sparse_mlp_w4: flags 0x%x", flags);
    REQ(a16(y) && a16(q1) && a16(q2), DV_ERR_ALIGN, "dv_sparse_mlp_w4: pointers must be 16-byte aligned");
    const size_t act = (size_t)d * 4;
    REQ(!overlap(out, act, y, act) && !overlap(out, act, residual, act), DV_ERR_RANGE,
        "dv_sparse_mlp_w4: out overlaps y or residual");
    float *wa, *part;
    const size_t need = w4_ws(d, n_idx_max, &wa, &part, ws);
    REQ(ws && ws_bytes >= need, DV_ERR_WORKSPACE, "dv_sparse_mlp_w4: workspace %zu < %zu", ws_bytes, need);
    hipStream_t s = (hipStream_t)stream;
    float* a = act_out ? act_out : wa;
    W4RowArgs r{};
    r.y = y; r.d = d; r.q = q1; r.s = (const half_t*)s1; r.bias = (const half_t*)b1; r.idx = idx; r.n_max = n_idx_max;
    r.n_dev = n_idx_dev; r.w_rows = N; r.out = a;
    timed_begin(DV_KERNEL_FC1, s);
    TRY(launch_rowdot_w4(r, s));
    timed_end(DV_KERNEL_FC1, s);
    W4AxpyArgs x{};
    x.q = q2; x.s = (const half_t*)s2; x.d = d; x.w_rows = N; x.rows = n_idx_max; x.n_rows_dev = n_idx_dev; x.idx = idx;
    x.coef = a; x.skip_zero = (flags & DV_SKIP_NONPOS_FC2) != 0; x.partial = part; x.rows_read = fc2_rows;
    timed_begin(DV_KERNEL_FC2, s);
    TRY(launch_axpy_w4(x, s));
    timed_end(DV_KERNEL_FC2, s);
    return launch_axpy_finalize(part, w4_axpy_groups(n_idx_max), 1, d, b2, DV_F16, residual, out, s);
}

// ---------------------------------------------------------------- KV scoring --
size_t dv_kv_score_workspace_bytes(int B, int h, int n, int n_obs) {
    if (B < 1 || h < 1 || n < 1 || n_obs < 1) return 0;
    return kCounterBytes + align_up(kv_score_stats_floats(B, h, n, n_obs) * 4, 256);
}

dv_status dv_kv_score(const void* q_obs, int B, int h, int d_h, int n_obs, const dv_kv_view* kv, float scale,
                      int n_sink, int n_window, int width, float* scores, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    REQ(q_obs && scores, DV_ERR_NULL, "dv_kv_score: NULL pointer");
    TRY(check_view(kv, "dv_kv_score"));
    REQ(kv->sel_idx == nullptr, DV_ERR_UNSUPPORTED, "dv_kv_score: scores a dense view");
    REQ(B >= 1 && h == kv->h && dh_ok(d_h), DV_ERR_SHAPE, "dv_kv_score: B=%d h=%d d_h=%d", B, h, d_h);
    REQ(n_obs >= 1 && (size_t)n_obs * (d_h + 2) * 4 <= 65536 && n_obs <= kv->n_ctx, DV_ERR_RANGE, "dv_kv_score: n_obs=%d n=%d",
        n_obs, kv->n_ctx);
    REQ(width >= 1 && width <= 63 && (width & 1), DV_ERR_RANGE, "dv_kv_score: width=%d", width);
    REQ(n_sink >= 0 && n_window >= 0, DV_ERR_RANGE, "dv_kv_score: n_sink=%d n_window=%d", n_sink, n_window);
    REQ(isfinite(scale), DV_ERR_RANGE, "dv_kv_score: scale");
    REQ(a16(q_obs), DV_ERR_ALIGN, "dv_kv_score: q_obs alignment");
    const size_t need = dv_kv_score_workspace_bytes(B, h, kv->n_ctx, n_obs);
    REQ(ws && ws_bytes >= need, DV_ERR_WORKSPACE, "dv_kv_score: workspace %zu < %zu", ws_bytes, need);
    float* st = (float*)((char*)ws + kCounterBytes);
    return launch_kv_score(q_obs, B, h, d_h, n_obs, kv, scale, n_sink, n_window, width, scores, st, st,
                           (hipStream_t)stream);
}

// ---------------------------------------------------------------- the layer --
struct LayerWs {
    float *y, *hres, *y2, *hpart, *sA, *sM, *q, *o, *apart, *a, *xpart;
    float *ya, *hpartA, *hpartM, *sA2, *sM2;      // the look-ahead predictions' own scratch
    float* mpart;                                 // matrix-core row-dot partial sums (batches of 8-16), or NULL
    unsigned* khist;                              // [4096] top-12-bit histogram of the next layer's neuron scores
    uint32_t* kkeys;                              // [N] their order keys
    void* kthr;                                   // their selection threshold
    int32_t *head_idx, *nidx, *uidx, *ucnt;
    size_t bytes;
};

static int layer_nmax(const dv_decode_cfg* c) {
    if (c->flags & DV_DENSE_MLP) return c->N;
    const long m = (long)c->B * c->k_neurons;
    return (int)(m < c->N ? m : c->N);
}

static LayerWs layer_ws(void* ws, const dv_decode_cfg* c, int max_len) {
    Carve cv(ws);
    LayerWs w;
    const int B = c->B, d = c->d, h = c->h, dh = c->d_h;
    const int nsel = (c->flags & DV_DENSE_ATTN) ? h : c->k_heads;
    const int nmax = layer_nmax(c);
    w.y = cv.take<float>((size_t)B * d);
    w.hres = cv.take<float>((size_t)B * d);
    w.y2 = cv.take<float>((size_t)B * d);
    const size_t hp = pred_partials(B, d, c->r_attn > c->r_mlp ? c->r_attn : c->r_mlp, c->wdt);
    w.hpart = cv.take<float>(hp > 0 ? hp : 1);
    w.sA = cv.take<float>((size_t)B * h);
    w.sM = cv.take<float>((size_t)B * c->N);
    w.head_idx = cv.take<int32_t>(h);
    w.nidx = cv.take<int32_t>((size_t)B * (c->k_neurons > 0 ? c->k_neurons : 1));
    w.uidx = cv.take<int32_t>(c->N);
    w.ucnt = cv.take<int32_t>(1);
    w.q = cv.take<float>((size_t)B * h * dh);
    w.o = cv.take<float>((size_t)B * h * dh);
    const int splits = splitk_auto(max_len, B * nsel);
    w.apart = cv.take<float>((size_t)B * (nsel > 0 ? nsel : 1) * splits * (dh + 2));
    w.a = cv.take<float>((size_t)B * (nmax > 0 ? nmax : 1));
    const AxpyPlan po = axpy_plan(d, nsel * dh, c->wdt), pm = axpy_plan(d, nmax, c->wdt);
    const size_t xp = axpy_ws_floats(po, B, d) > axpy_ws_floats(pm, B, d) ? axpy_ws_floats(po, B, d)
                                                                           : axpy_ws_floats(pm, B, d);
    size_t xpt = xp;
    if (c->flags & DV_TEAL) {   // the input-major Q/K/V and fc1 sums are 3*h*d_h and N wide
        const size_t a1 = axpy_ws_floats(axpy_plan(3 * h * dh, d, c->wdt), B, 3 * h * dh);
        const size_t a2 = axpy_ws_floats(axpy_plan(c->N, d, c->wdt), B, c->N);
        xpt = a1 > xpt ? a1 : xpt;
        xpt = a2 > xpt ? a2 : xpt;
    }
    w.xpart = cv.take<float>(xpt);
    w.ya = cv.take<float>((size_t)d);
    w.hpartA = cv.take<float>((size_t)(c->r_attn > 0 ? c->r_attn : 1) + (c->r_mlp > 0 ? c->r_mlp : 1));   // [rA + rM]
    w.hpartM = cv.take<float>(pred_partials(1, d, c->r_mlp > 0 ? c->r_mlp : 1, c->wdt));
    w.sA2 = cv.take<float>((size_t)h);
    w.sM2 = cv.take<float>((size_t)c->N);
    w.khist = cv.take<unsigned>(4096);
    w.kkeys = cv.take<uint32_t>((size_t)c->N);
    w.kthr = cv.take<unsigned>(4);
    size_t mp = rowdot_mfma_part_floats(nmax > 3 * nsel * dh ? nmax : 3 * nsel * dh);
    const size_t pp[4] = {rowdot_mfma_rows_part_floats(c->r_attn, d), rowdot_mfma_rows_part_floats(h, c->r_attn),
                          rowdot_mfma_rows_part_floats(c->r_mlp, d), rowdot_mfma_rows_part_floats(c->N, c->r_mlp)};
    for (size_t q : pp) mp = q > mp ? q : mp;      // the predictors' layers
    w.mpart = rowdot_mfma_ok(B, d, c->wdt) ? cv.take<float>(mp) : nullptr;
    w.bytes = align_up(cv.off, 256);
    return w;
}

static dv_status check_cfg(const dv_decode_cfg* c) {
    REQ(c, DV_ERR_NULL, "dv_decode_layer: cfg NULL");
    REQ(wdt_ok(c->wdt), DV_ERR_DTYPE, "dv_decode_layer: wdt %d", c->wdt);
    REQ(c->pred_act == DV_ACT_NONE || c->pred_act == DV_ACT_RELU, DV_ERR_DTYPE, "dv_decode_layer: pred_act");
    const unsigned known = DV_SKIP_NONPOS_FC2 | DV_DENSE_ATTN | DV_DENSE_MLP | DV_HOLE_FILL | DV_KV_SELECT | DV_ADVANCE_POS |
                           DV_LOOKAHEAD | DV_KV_WINDOW | DV_TEAL;
    REQ((c->flags & ~known) == 0, DV_ERR_DTYPE, "dv_decode_layer: flags 0x%x", c->flags);
    REQ(c->B >= 1 && c->B <= 16 && d_ok(c->d) && c->h >= 1 && dh_ok(c->d_h) && c->N >= 1, DV_ERR_SHAPE,
        "dv_decode_layer: B=%d d=%d h=%d d_h=%d N=%d", c->B, c->d, c->h, c->d_h, c->N);
    const int eb = elt_bytes(c->wdt);
    REQ((size_t)c->d * eb % 16 == 0, DV_ERR_ALIGN, "dv_decode_layer: d=%d rows", c->d);
    if (!(c->flags & DV_DENSE_ATTN)) {
        REQ(c->r_attn >= 1 && c->r_attn <= 512 && (size_t)c->r_attn * eb % 16 == 0, DV_ERR_SHAPE,
            "dv_decode_layer: r_attn=%d", c->r_attn);
        REQ(c->k_heads >= 0 && c->k_heads <= c->h, DV_ERR_RANGE, "dv_decode_layer: k_heads=%d", c->k_heads);
        REQ(c->B == 1, DV_ERR_UNSUPPORTED, "dv_decode_layer: head sparsity with B=%d", c->B);
    }
    if (!(c->flags & DV_DENSE_MLP)) {
        REQ(c->r_mlp >= 1 && c->r_mlp <= 512 && (size_t)c->r_mlp * eb % 16 == 0, DV_ERR_SHAPE,
            "dv_decode_layer: r_mlp=%d", c->r_mlp);
        REQ(c->k_neurons >= 0 && c->k_neurons <= c->N && c->N <= 65536, DV_ERR_RANGE, "dv_decode_layer: k_neurons=%d",
            c->k_neurons);
    }
    REQ(isfinite(c->scale) && c->eps >= 0.f && isfinite(c->eps), DV_ERR_RANGE, "dv_decode_layer: scale/eps");
    REQ(c->n_dense_prefix >= 0, DV_ERR_RANGE, "dv_decode_layer: n_dense_prefix=%d", c->n_dense_prefix);
    REQ(!(c->flags & DV_KV_WINDOW) || (!(c->flags & DV_KV_SELECT) && c->win_len > 0 && c->win_sink >= 0),
        DV_ERR_RANGE, "dv_decode_layer: DV_KV_WINDOW win_sink=%d win_len=%d (not with DV_KV_SELECT)", c->win_sink,
        c->win_len);
    REQ(!(c->flags & DV_TEAL) || ((c->flags & DV_DENSE_ATTN) && (c->flags & DV_DENSE_MLP) &&
                                  !(c->flags & (DV_LOOKAHEAD | DV_HOLE_FILL))),
        DV_ERR_UNSUPPORTED, "dv_decode_layer: DV_TEAL needs DV_DENSE_ATTN and DV_DENSE_MLP, without DV_LOOKAHEAD "
        "or DV_HOLE_FILL (flags 0x%x)", c->flags);
    if (c->flags & DV_LOOKAHEAD) {
        REQ(c->B == 1, DV_ERR_UNSUPPORTED, "dv_decode_layer: DV_LOOKAHEAD with B=%d", c->B);
        REQ(c->r_attn >= 1 && c->r_attn <= 512 && (size_t)c->r_attn * eb % 16 == 0 && c->r_mlp >= 1 &&
                c->r_mlp <= 512 && (size_t)c->r_mlp * eb % 16 == 0,
            DV_ERR_SHAPE, "dv_decode_layer: look-ahead ranks r_attn=%d r_mlp=%d", c->r_attn, c->r_mlp);
        REQ(c->k_heads >= 0 && c->k_heads <= c->h && c->k_neurons >= 0 && c->k_neurons <= c->N &&
                c->N <= dv::kTopkMaxN,
            DV_ERR_RANGE, "dv_decode_layer: look-ahead budgets k_heads=%d k_neurons=%d", c->k_heads, c->k_neurons);
    }
    return DV_OK;
}

// DejaVu §4.3, the parallel form (batch of one): the next layer's sets are
// predicted from this layer's y = LN1(x) while this layer runs with its
// given sets, either on the auxiliary stream or riding as extra workgroups
// in this layer's launches.  LN1 is folded into the Q/K/V kernel and LN2 into
// fc1, so the layer itself runs seven kernels.
// Arguments of the look-ahead form (checked before anything is enqueued).
static dv_status check_lookahead(const dv_decode_cfg* c, const dv_layer_state* st) {
    const bool dense_a = (c->flags & DV_DENSE_ATTN) != 0, dense_m = (c->flags & DV_DENSE_MLP) != 0;
    REQ(dense_a || st->head_idx_in, DV_ERR_NULL, "dv_decode_layer: DV_LOOKAHEAD needs head_idx_in");
    REQ(dense_m || st->neuron_idx_in, DV_ERR_NULL, "dv_decode_layer: DV_LOOKAHEAD needs neuron_idx_in");
    REQ((st->next_pa1_t == nullptr) == (st->next_pa2_t == nullptr) &&
            (st->next_pm1_t == nullptr) == (st->next_pm2_t == nullptr),
        DV_ERR_NULL, "dv_decode_layer: next predictor layers go in pairs");
    REQ(!st->next_pa1_t || st->next_head_idx, DV_ERR_NULL, "dv_decode_layer: next_head_idx NULL");
    REQ(!st->next_pm1_t || st->next_neuron_idx, DV_ERR_NULL, "dv_decode_layer: next_neuron_idx NULL");
    REQ(!st->next_pa1_t || (a16(st->next_pa1_t) && a16(st->next_pa2_t)), DV_ERR_ALIGN, "dv_decode_layer: next_pa alignment");
    REQ(!st->next_pm1_t || (a16(st->next_pm1_t) && a16(st->next_pm2_t)), DV_ERR_ALIGN, "dv_decode_layer: next_pm alignment");
    REQ(!st->aux_stream || (st->ev_fork && st->ev_join), DV_ERR_NULL, "dv_decode_layer: aux_stream needs ev_fork and ev_join");
    // the next sets are written while this layer's launches still read the
    // given ones: they must be separate buffers
    {
        const size_t hb = (size_t)(c->k_heads > 0 ? c->k_heads : 1) * 4, nb = (size_t)(c->k_neurons > 0 ? c->k_neurons : 1) * 4;
        const void* hin = dense_a ? nullptr : st->head_idx_in;
        const void* nin = dense_m ? nullptr : st->neuron_idx_in;
        const void* hout = st->next_pa1_t ? st->next_head_idx : nullptr;
        const void* nout = st->next_pm1_t ? st->next_neuron_idx : nullptr;
        REQ(!overlap(hout, hb, hin, hb) && !overlap(hout, hb, nin, nb) && !overlap(nout, nb, hin, hb) &&
                !overlap(nout, nb, nin, nb) && !overlap(hout, hb, nout, nb),
            DV_ERR_RANGE, "dv_decode_layer: next_head_idx / next_neuron_idx overlap the given sets or each other");
    }
    return DV_OK;
}

// The sets of one layer predicted from LN1(x) by the given predictors, in
// launches of their own (the look-ahead form's predictions when they do not
// ride in a layer's launches, and the first layer of a stack).
static dv_status predict_sets(const dv_decode_cfg* c, const float* x, const float* g, const float* b,
                              const void* pa1, const void* pa2, int32_t* head_idx, const void* pm1, const void* pm2,
                              int32_t* neuron_idx, const LayerWs& L, hipStream_t s) {
    const int d = c->d, h = c->h, N = c->N;
    const bool pair = pa1 && pm1 && c->k_heads > 0 && c->k_neurons > 0 && row_ln_supported(d, c->wdt) &&
                      pred_topk_fusable(1, h, c->r_attn);
    if (pair) {
        TRY(launch_predict_pair_ln(x, d, g, b, c->eps, L.ya, pa1, c->r_attn, pa2, h, c->k_heads, head_idx, pm1, c->r_mlp,
                                   pm2, N, L.sA2, L.sM2, L.hpartA, c->wdt, c->pred_act, s));
        return launch_topk(L.sM2, 1, N, c->k_neurons, neuron_idx, s);
    }
    if (pa1 && c->k_heads > 0) {
        if (pred_topk_fusable(1, h, c->r_attn)) {
            TRY(launch_predict_ln_topk(x, d, g, b, c->eps, L.ya, pa1, c->r_attn, pa2, h, c->wdt, c->pred_act, L.sA2,
                                       L.hpartA, c->k_heads, head_idx, s));
        } else {
            TRY(launch_predict_ln(x, 1, d, g, b, c->eps, L.ya, pa1, c->r_attn, pa2, h, c->wdt, c->pred_act, L.sA2,
                                  L.hpartA, s));
            TRY(launch_topk(L.sA2, 1, h, c->k_heads, head_idx, s));
        }
    }
    if (pm1 && c->k_neurons > 0) {
        TRY(launch_predict_ln(x, 1, d, g, b, c->eps, L.ya, pm1, c->r_mlp, pm2, N, c->wdt, c->pred_act, L.sM2, L.hpartM, s));
        TRY(launch_topk(L.sM2, 1, N, c->k_neurons, neuron_idx, s));
    }
    return DV_OK;
}

// Whether a look-ahead layer of a stack lacks a predictor its next layer needs.
static bool next_layer_predictors_missing(const dv_layer_state& st, const dv_decode_cfg* c, bool has_next) {
    if (!has_next) return false;
    const bool dense_a = (c->flags & DV_DENSE_ATTN) != 0, dense_m = (c->flags & DV_DENSE_MLP) != 0;
    return (!dense_a && c->k_heads > 0 && !(st.next_pa1_t && st.next_pa2_t)) ||
           (!dense_m && c->k_neurons > 0 && !(st.next_pm1_t && st.next_pm2_t));
}

static dv_status decode_lookahead(const dv_layer_weights* w, const dv_decode_cfg* c, const dv_layer_state* st,
                                  const dv_kv_view& view, const LayerWs& L, const float* x_in, float* x_out, void* ws,
                                  hipStream_t s) {
    const int d = c->d, h = c->h, dh = c->d_h, N = c->N;
    const bool dense_a = (c->flags & DV_DENSE_ATTN) != 0, dense_m = (c->flags & DV_DENSE_MLP) != 0;
    const bool predict = st->next_pa1_t || st->next_pm1_t;
    hipStream_t ps = st->aux_stream ? (hipStream_t)st->aux_stream : s;
    const bool pa = st->next_pa1_t && c->k_heads > 0;      // the next layer's head set is predicted
    const bool pm = st->next_pm1_t && c->k_neurons > 0;    // the next layer's neuron set is predicted
    // Without a second stream the predictions ride in this layer's launches
    // as extra workgroups: the predictors' first layers in the Q/K/V launch
    // (same LN1(x)), their second layers (and the head selection) in the
    // attention launch, and the neuron selection split over later launches:
    // a histogram of the scores beside the output projection, the threshold
    // beside its finalize and the ordered emission beside fc2 (else a
    // launch of its own after attention).  Either predictor may be absent
    // (every head, or every neuron, is used).
    const bool ride = (pa || pm) && !st->aux_stream && ln_fusable(1, d) && row_ln_supported(d, c->wdt) &&
                      (!pa || pred_topk_fusable(1, h, c->r_attn));
    const bool ride_topk = ride && pm && topk_split_supported(N, c->k_neurons);
    const int rA = pa ? c->r_attn : 0, rM = pm ? c->r_mlp : 0;
    if (predict && st->aux_stream) {
        HIP_TRY(hipEventRecord((hipEvent_t)st->ev_fork, s));
        HIP_TRY(hipStreamWaitEvent(ps, (hipEvent_t)st->ev_fork, 0));
    }
    // ---- the next layer's sets from this layer's y (predictor layers fold LN1 in)
    if (!ride && predict)
        TRY(predict_sets(c, x_in, w->ln1_g, w->ln1_b, st->next_pa1_t, st->next_pa2_t, st->next_head_idx, st->next_pm1_t,
                         st->next_pm2_t, st->next_neuron_idx, L, ps));
    if (predict && st->aux_stream) HIP_TRY(hipEventRecord((hipEvent_t)st->ev_join, ps));

    // ---- this layer with its given sets
    const int32_t* head_idx = dense_a ? nullptr : st->head_idx_in;
    const int n_sel = dense_a ? h : c->k_heads;
    dv_kv_state kvs = st->kv;
    if (!(c->flags & DV_HOLE_FILL)) {
        kvs.y_buf = nullptr;
        kvs.valid_upto = nullptr;
    }
    const bool fill = kvs.y_buf && kvs.valid_upto;
    RowArgs p1{};
    if (ride) {   // hidden rows: the head predictor's rA, then the neuron predictor's rM
        p1.B = 1; p1.d = d;
        p1.w = pa ? st->next_pa1_t : st->next_pm1_t;
        p1.w2 = pa && pm ? st->next_pm1_t : nullptr;
        p1.split = pa && pm ? rA : rA + rM;
        p1.n_max = rA + rM; p1.w_rows = p1.n_max; p1.out = L.hpartA;
    }
    if (ln_fusable(1, d)) {
        timed_begin(DV_KERNEL_QKV, s);
        TRY(launch_qkv(x_in, 1, d, h, dh, head_idx, n_sel, w->w_qkv_t, w->b_qkv, c->wdt, L.q, &kvs, false, s, w->ln1_g,
                       w->ln1_b, c->eps, ride ? &p1 : nullptr));
        timed_end(DV_KERNEL_QKV, s);
    } else {
        TRY(launch_layernorm(x_in, 1, d, w->ln1_g, w->ln1_b, c->eps, L.y, s));
        timed_begin(DV_KERNEL_QKV, s);
        TRY(launch_qkv(L.y, 1, d, h, dh, head_idx, n_sel, w->w_qkv_t, w->b_qkv, c->wdt, L.q, &kvs, false, s));
        timed_end(DV_KERNEL_QKV, s);
    }
    int splits = 0;
    Pred2Args p2 = pred2_args(L.hpartA, rA, pa ? st->next_pa2_t : nullptr, pa ? h : 0, L.sA2, pa ? c->k_heads : 0,
                              st->next_head_idx, L.hpartA + rA, rM, pm ? st->next_pm2_t : nullptr, pm ? N : 0, L.sM2,
                              c->pred_act, c->wdt);
    p2.zero = ride_topk ? L.khist : nullptr;
    timed_begin(DV_KERNEL_ATTN, s);
    TRY(launch_splitk(L.q, 1, dh, head_idx, n_sel, &view, st->kv.pos_dev, 1, c->scale, 0, nullptr, L.apart,
                      fill ? kvs.valid_upto : nullptr, st->kv.pos, st->kv.pos_dev, s, &splits, ride ? &p2 : nullptr));
    timed_end(DV_KERNEL_ATTN, s);
    if (ride && pm && !ride_topk) TRY(launch_topk(L.sM2, 1, N, c->k_neurons, st->next_neuron_idx, s));
    const TopkSel tk{L.sM2, N, c->k_neurons, L.khist, L.kkeys, L.kthr, st->next_neuron_idx};
    {
        AxpyCall ac{};
        ac.w = w->w_o_t; ac.wdt = c->wdt; ac.d = d; ac.w_rows = h * dh; ac.rows = n_sel * dh; ac.idx = head_idx;
        ac.blk = dh; ac.apart = L.apart; ac.num_splits = splits; ac.B = 1; ac.bias = w->b_o; ac.residual = x_in;
        ac.out = L.hres; ac.partial = L.xpart;
        ac.sel = ride_topk ? &tk : nullptr;
        ac.timed = DV_KERNEL_OUT;
        TRY(launch_axpy(ac, s));
    }
    const int32_t* idx = dense_m ? nullptr : st->neuron_idx_in;
    const int n_max = dense_m ? N : c->k_neurons;
    if (row_ln_supported(d, c->wdt)) {
        timed_begin(DV_KERNEL_FC1, s);
        TRY(launch_fc1_ln(L.hres, d, w->ln2_g, w->ln2_b, c->eps, w->w1_t, w->b1, c->wdt, idx, n_max, nullptr, N, L.a, s));
        timed_end(DV_KERNEL_FC1, s);
    } else {
        TRY(launch_layernorm(L.hres, 1, d, w->ln2_g, w->ln2_b, c->eps, L.y2, s));
        timed_begin(DV_KERNEL_FC1, s);
        TRY(launch_fc1(L.y2, 1, d, w->w1_t, w->b1, c->wdt, idx, n_max, nullptr, N, L.a, s));
        timed_end(DV_KERNEL_FC1, s);
    }
    AxpyCall mc{};
    mc.w = w->w2_t; mc.wdt = c->wdt; mc.d = d; mc.w_rows = N; mc.rows = n_max; mc.idx = idx; mc.blk = 1; mc.coef = L.a;
    mc.coef_stride = n_max; mc.skip_zero = (c->flags & DV_SKIP_NONPOS_FC2) != 0; mc.B = 1; mc.bias = w->b2;
    mc.residual = L.hres; mc.out = x_out; mc.rows_read = st->fc2_rows_out; mc.partial = L.xpart;
    mc.advance = (c->flags & DV_ADVANCE_POS) ? st->kv.pos_dev : nullptr;
    mc.sel = ride_topk ? &tk : nullptr;
    mc.timed = DV_KERNEL_FC2;
    TRY(launch_axpy(mc, s));
    if (predict && st->aux_stream) HIP_TRY(hipStreamWaitEvent(s, (hipEvent_t)st->ev_join, 0));
    (void)ws;
    return DV_OK;
}

// ByteCross's projection branch (§4.1, App. A): every head and neuron, each
// projection reading only the input-major rows of the input channels above
// its threshold.  LN1, the Q/K/V gather-AXPY (its finalize scatters q and
// the token's K/V), split-K attention with its combine, the output
// projection, LN2, fc1 (finalize: bias and ReLU), fc2: each projection's
// input is thresholded where its gather resolves its rows.
static dv_status decode_teal(const dv_layer_weights* w, const dv_decode_cfg* c, const dv_layer_state* st,
                             const dv_kv_view& view, const LayerWs& L, const float* x_in, float* x_out, hipStream_t s) {
    const int B = c->B, d = c->d, h = c->h, dh = c->d_h, N = c->N, hd = h * dh;
    const dv_kv_state& kv = st->kv;
    const int R = d > hd ? (d > N ? d : N) : (hd > N ? hd : N);
    auto record = [&](int i, const float* src, int width) -> dv_status {   // the input before its threshold
        if (!st->teal_rec) return DV_OK;
        const hipError_t e = hipMemcpy2DAsync(st->teal_rec + (size_t)i * B * R, (size_t)R * 4, src, (size_t)width * 4,
                                              (size_t)width * 4, B, hipMemcpyDeviceToDevice, s);
        return e == hipSuccess ? DV_OK : fail(DV_ERR_HIP, "teal_rec copy: %s", hipGetErrorString(e));
    };
    auto rows_out = [&](int i) { return st->teal_rows_out ? st->teal_rows_out + i : nullptr; };
    auto gather = [&](const void* wt, int width, int rows, const float* coef, int i, const void* bias,
                      const float* residual, float* out, int timed) {
        AxpyCall ac{};
        ac.w = wt; ac.wdt = c->wdt; ac.d = width; ac.w_rows = rows; ac.rows = rows; ac.blk = 1; ac.coef = coef;
        ac.coef_stride = rows; ac.skip_zero = true; ac.thresh = true; ac.thr = st->teal_thr[i]; ac.B = B;
        ac.bias = bias; ac.residual = residual; ac.out = out; ac.rows_read = rows_out(i); ac.partial = L.xpart;
        ac.timed = timed;
        return ac;
    };
    TRY(launch_layernorm(x_in, B, d, w->ln1_g, w->ln1_b, c->eps, L.y, s));
    TRY(record(0, L.y, d));
    {
        AxpyCall ac = gather(w->w_qkv_in, 3 * hd, d, L.y, 0, w->b_qkv, nullptr, nullptr, DV_KERNEL_QKV);
        ac.epi.mode = FIN_QKV; ac.epi.q = L.q; ac.epi.k = (half_t*)kv.k_cache; ac.epi.v = (half_t*)kv.v_cache;
        ac.epi.h = h; ac.epi.dh = dh; ac.epi.max_len = kv.max_len; ac.epi.pos = kv.pos; ac.epi.pos_dev = kv.pos_dev;
        TRY(launch_axpy(ac, s));
    }
    timed_begin(DV_KERNEL_ATTN, s);
    TRY(launch_splitk(L.q, B, dh, nullptr, h, &view, kv.pos_dev, 1, c->scale, 0, L.o, L.apart, nullptr, kv.pos,
                      kv.pos_dev, s));
    timed_end(DV_KERNEL_ATTN, s);
    TRY(record(1, L.o, hd));
    TRY(launch_axpy(gather(w->w_o_t, d, hd, L.o, 1, w->b_o, x_in, L.hres, DV_KERNEL_OUT), s));
    TRY(launch_layernorm(L.hres, B, d, w->ln2_g, w->ln2_b, c->eps, L.y2, s));
    TRY(record(2, L.y2, d));
    {
        AxpyCall ac = gather(w->w1_in, N, d, L.y2, 2, w->b1, nullptr, L.a, DV_KERNEL_FC1);
        ac.epi.mode = FIN_RELU;
        TRY(launch_axpy(ac, s));
    }
    TRY(record(3, L.a, N));
    AxpyCall mc = gather(w->w2_t, d, N, L.a, 3, w->b2, L.hres, x_out, DV_KERNEL_FC2);
    mc.advance = (c->flags & DV_ADVANCE_POS) ? kv.pos_dev : nullptr;
    return launch_axpy(mc, s);
}

size_t dv_decode_workspace_bytes(const dv_decode_cfg* cfg, int max_len) {
    if (check_cfg(cfg) != DV_OK || max_len < 1) return 0;
    return layer_ws(nullptr, cfg, max_len).bytes;
}

static dv_status decode_one(const dv_layer_weights* w, const dv_decode_cfg* c, const dv_layer_state* st,
                            const float* x_in, float* x_out, void* ws, size_t ws_bytes, hipStream_t s, bool run = true);

dv_status dv_decode_layer(const dv_layer_weights* w, const dv_decode_cfg* c, const dv_layer_state* st,
                          const float* x_in, float* x_out, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    TRY(check_cfg(c));
    return decode_one(w, c, st, x_in, x_out, ws, ws_bytes, (hipStream_t)stream);
}

// One layer step: every argument is checked first; with run false nothing
// is launched (a stack checks all its layers before enqueueing any).
static dv_status decode_one(const dv_layer_weights* w, const dv_decode_cfg* c, const dv_layer_state* st,
                            const float* x_in, float* x_out, void* ws, size_t ws_bytes, hipStream_t s, bool run) {
    REQ(w && st && x_in && x_out, DV_ERR_NULL, "dv_decode_layer: NULL pointer");
    REQ(w->ln1_g && w->ln1_b && w->ln2_g && w->ln2_b && w->w_qkv_t && w->b_qkv && w->w_o_t && w->b_o && w->w1_t &&
            w->b1 && w->w2_t && w->b2,
        DV_ERR_NULL, "dv_decode_layer: weight pointer NULL");
    const bool ahead = (c->flags & DV_LOOKAHEAD) != 0;   // this layer's sets are given: its predictors are not read
    REQ(ahead || (c->flags & DV_DENSE_ATTN) || (w->pa1_t && w->pa2_t), DV_ERR_NULL, "dv_decode_layer: head predictor NULL");
    REQ(ahead || (c->flags & DV_DENSE_MLP) || (w->pm1_t && w->pm2_t), DV_ERR_NULL,
        "dv_decode_layer: neuron predictor NULL");
    const dv_kv_state& kv = st->kv;
    REQ(kv.k_cache && kv.v_cache, DV_ERR_NULL, "dv_decode_layer: KV cache NULL");
    REQ(kv.max_len >= 1 && kv.pos >= 0 && kv.pos < kv.max_len, DV_ERR_RANGE, "dv_decode_layer: pos=%d max_len=%d",
        kv.pos, kv.max_len);
    REQ(!(c->flags & DV_HOLE_FILL) || (kv.y_buf && kv.valid_upto), DV_ERR_NULL, "dv_decode_layer: hole fill state");
    REQ(!kv.y_buf || a16(kv.y_buf), DV_ERR_ALIGN, "dv_decode_layer: y_buf must be 16-byte aligned");
    REQ(!(c->flags & DV_ADVANCE_POS) || kv.pos_dev, DV_ERR_NULL, "dv_decode_layer: DV_ADVANCE_POS needs kv.pos_dev");
    REQ(qkv_supported(c->B, c->d, c->wdt), DV_ERR_UNSUPPORTED, "dv_decode_layer: d=%d rows too long", c->d);
    REQ(a16(w->w_qkv_t) && a16(w->w_o_t) && a16(w->w1_t) && a16(w->w2_t) && a16(x_in), DV_ERR_ALIGN,
        "dv_decode_layer: weight alignment");
    REQ(!overlap(x_out, (size_t)c->B * c->d * 4, x_in, (size_t)c->B * c->d * 4), DV_ERR_RANGE,
        "dv_decode_layer: x_out overlaps x_in");
    dv_kv_view view;
    view.k_cache = kv.k_cache; view.v_cache = kv.v_cache; view.h = c->h; view.max_len = kv.max_len;
    view.n_ctx = kv.pos + 1;
    view.sel_idx = nullptr; view.sel_len = nullptr; view.sel_cap = 0; view.sel_end = 0; view.n_ctx_dev = nullptr;
    view.win_sink = 0; view.win_len = 0;
    if (c->flags & DV_KV_WINDOW) {
        view.win_sink = c->win_sink; view.win_len = c->win_len;
    }
    if (c->flags & DV_KV_SELECT) {
        view.sel_idx = st->sel_idx; view.sel_len = st->sel_len; view.sel_cap = st->sel_cap; view.sel_end = st->sel_end;
        REQ(view.sel_idx, DV_ERR_NULL, "dv_decode_layer: DV_KV_SELECT without sel_idx");
        TRY(check_view(&view, "dv_decode_layer"));
    }
    const LayerWs L = layer_ws(ws, c, kv.max_len);
    REQ(ws && ws_bytes >= L.bytes, DV_ERR_WORKSPACE, "dv_decode_layer: workspace %zu < %zu", ws_bytes, L.bytes);
    if (ahead) TRY(check_lookahead(c, st));
    const bool teal = (c->flags & DV_TEAL) != 0;
    if (teal) {
        REQ(w->w_qkv_in && w->w1_in, DV_ERR_NULL, "dv_decode_layer: DV_TEAL needs w_qkv_in and w1_in");
        REQ(a16(w->w_qkv_in) && a16(w->w1_in), DV_ERR_ALIGN, "dv_decode_layer: input-major weight alignment");
        REQ(((size_t)3 * c->h * c->d_h * elt_bytes(c->wdt)) % 16 == 0 && ((size_t)c->N * elt_bytes(c->wdt)) % 16 == 0,
            DV_ERR_ALIGN, "dv_decode_layer: DV_TEAL rows of 3*h*d_h=%d or N=%d", 3 * c->h * c->d_h, c->N);
        for (int i = 0; i < 4; ++i)
            REQ(!isnan(st->teal_thr[i]), DV_ERR_RANGE, "dv_decode_layer: teal_thr[%d] is NaN", i);
    }
    if (!run) return DV_OK;

    if (ahead) return decode_lookahead(w, c, st, view, L, x_in, x_out, ws, s);
    if (teal) return decode_teal(w, c, st, view, L, x_in, x_out, s);
    const int B = c->B, d = c->d, h = c->h, dh = c->d_h, N = c->N;
    // attention block: LN1 folded into the head predictor when heads are selected
    const int32_t* head_idx = nullptr;
    int n_sel = h;
    if (!(c->flags & DV_DENSE_ATTN)) {
        int32_t* hi = st->head_idx_out ? st->head_idx_out : L.head_idx;
        if (pred_topk_fusable(B, h, c->r_attn)) {
            if (c->k_heads > 0)
                TRY(launch_predict_ln_topk(x_in, d, w->ln1_g, w->ln1_b, c->eps, L.y, w->pa1_t, c->r_attn, w->pa2_t, h,
                                           c->wdt, c->pred_act, L.sA, L.hpart, c->k_heads, hi, s));
            else
                TRY(launch_layernorm(x_in, B, d, w->ln1_g, w->ln1_b, c->eps, L.y, s));
        } else {
            TRY(launch_predict_ln(x_in, B, d, w->ln1_g, w->ln1_b, c->eps, L.y, w->pa1_t, c->r_attn, w->pa2_t, h,
                                  c->wdt, c->pred_act, L.sA, L.hpart, s, L.mpart));
            TRY(launch_topk(L.sA, B, h, c->k_heads, hi, s));
        }
        head_idx = hi;
        n_sel = c->k_heads;
    } else {
        TRY(launch_layernorm(x_in, B, d, w->ln1_g, w->ln1_b, c->eps, L.y, s));
    }
    dv_kv_state kvs = kv;
    if (!(c->flags & DV_HOLE_FILL)) {
        kvs.y_buf = nullptr;
        kvs.valid_upto = nullptr;
    }
    const bool fill = kvs.y_buf && kvs.valid_upto;
    timed_begin(DV_KERNEL_QKV, s);
    if (L.mpart && !fill)
        TRY(launch_qkv_mfma(L.y, B, d, h, dh, head_idx, n_sel, w->w_qkv_t, w->b_qkv, L.q, &kvs, L.mpart, s));
    else
        TRY(launch_qkv(L.y, B, d, h, dh, head_idx, n_sel, w->w_qkv_t, w->b_qkv, c->wdt, L.q, &kvs, false, s));
    timed_end(DV_KERNEL_QKV, s);
    // split-K partials go straight into the output projection, which merges
    // them per row; for the matrix cores they are merged into o first
    const bool o_first = axpy_mfma_supported(B, d, c->wdt);
    int splits = 0;
    timed_begin(DV_KERNEL_ATTN, s);
    TRY(launch_splitk(L.q, B, dh, head_idx, n_sel, &view, kv.pos_dev, 1, c->scale, 0, o_first ? L.o : nullptr,
                      L.apart, fill ? kvs.valid_upto : nullptr, kv.pos, kv.pos_dev, s, &splits));
    timed_end(DV_KERNEL_ATTN, s);
    {
        AxpyCall ac{};
        ac.w = w->w_o_t; ac.wdt = c->wdt; ac.d = d; ac.w_rows = h * dh; ac.rows = n_sel * dh; ac.idx = head_idx;
        ac.blk = dh; ac.B = B; ac.bias = w->b_o; ac.residual = x_in;
        if (o_first) {
            ac.coef = L.o; ac.coef_stride = n_sel * dh;
        } else {
            ac.apart = L.apart; ac.num_splits = splits;
        }
        ac.out = L.hres; ac.partial = L.xpart; ac.timed = DV_KERNEL_OUT;
        TRY(launch_axpy(ac, s));
    }
    // MLP block: LN2 folded into the neuron predictor
    const int32_t* idx = nullptr;
    const int32_t* n_dev = nullptr;
    int n_max = N;
    if (!(c->flags & DV_DENSE_MLP)) {
        TRY(launch_predict_ln(L.hres, B, d, w->ln2_g, w->ln2_b, c->eps, L.y2, w->pm1_t, c->r_mlp, w->pm2_t, N, c->wdt,
                              c->pred_act, L.sM, L.hpart, s, L.mpart));
        if (B == 1) {
            int32_t* ni = st->neuron_idx_out ? st->neuron_idx_out : L.nidx;
            TRY(launch_topk(L.sM, 1, N, c->k_neurons, ni, s));
            if (st->neuron_count_out) TRY(launch_set_i32(st->neuron_count_out, c->k_neurons, s));
            idx = ni;
            n_max = c->k_neurons;
        } else {
            int32_t* ui = st->neuron_idx_out ? st->neuron_idx_out : L.uidx;
            int32_t* uc = st->neuron_count_out ? st->neuron_count_out : L.ucnt;
            TRY(launch_topk(L.sM, B, N, c->k_neurons, L.nidx, s));
            TRY(launch_union(L.nidx, B, c->k_neurons, N, ui, uc, s));
            idx = ui;
            n_dev = uc;
            n_max = layer_nmax(c);
        }
    } else {
        TRY(launch_layernorm(L.hres, B, d, w->ln2_g, w->ln2_b, c->eps, L.y2, s));
    }
    timed_begin(DV_KERNEL_FC1, s);
    if (L.mpart) TRY(launch_fc1_mfma(L.y2, B, d, w->w1_t, w->b1, idx, n_max, n_dev, N, L.a, L.mpart, s));
    else TRY(launch_fc1(L.y2, B, d, w->w1_t, w->b1, c->wdt, idx, n_max, n_dev, N, L.a, s));
    timed_end(DV_KERNEL_FC1, s);
    AxpyCall mc{};
    mc.w = w->w2_t; mc.wdt = c->wdt; mc.d = d; mc.w_rows = N; mc.rows = n_max; mc.n_rows_dev = n_dev; mc.idx = idx;
    mc.blk = 1; mc.coef = L.a; mc.coef_stride = n_max; mc.skip_zero = (c->flags & DV_SKIP_NONPOS_FC2) != 0; mc.B = B;
    mc.bias = w->b2; mc.residual = L.hres; mc.out = x_out; mc.rows_read = st->fc2_rows_out; mc.partial = L.xpart;
    mc.advance = (c->flags & DV_ADVANCE_POS) ? kv.pos_dev : nullptr;
    mc.timed = DV_KERNEL_FC2;
    return launch_axpy(mc, s);
}

// ---------------------------------------------------------------- the stack --
// The configuration of one layer of a stack: the first n_dense_prefix
// layers compute every head and neuron (Explainer, "Handling the first
// layer": the first layers run dense and prediction starts after them).
static dv_decode_cfg stack_layer_cfg(const dv_decode_cfg* c, int l) {
    dv_decode_cfg cl = *c;
    if (l < c->n_dense_prefix) cl.flags |= DV_DENSE_ATTN | DV_DENSE_MLP;
    return cl;
}

static size_t stack_layer_ws_bytes(const dv_decode_cfg* c, int max_len) {
    size_t b = layer_ws(nullptr, c, max_len).bytes;
    if (c->n_dense_prefix > 0) {
        const dv_decode_cfg cd = stack_layer_cfg(c, 0);
        const size_t bd = layer_ws(nullptr, &cd, max_len).bytes;
        b = bd > b ? bd : b;
    }
    return b;
}

size_t dv_stack_workspace_bytes(const dv_decode_cfg* cfg, int max_len) {
    if (check_cfg(cfg) != DV_OK || max_len < 1) return 0;
    return stack_layer_ws_bytes(cfg, max_len) + align_up((size_t)2 * cfg->B * cfg->d * sizeof(float), 256);
}

dv_status dv_decode_stack(const dv_stack_layer* layers, int n_layers, const dv_decode_cfg* c, int32_t* head_sets,
                          int32_t* neuron_sets, int32_t* neuron_counts, int32_t* fc2_rows, const float* x_in,
                          float* x_out, float* x_trace, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    TRY(check_cfg(c));
    REQ(layers && x_in && x_out, DV_ERR_NULL, "dv_decode_stack: NULL pointer");
    REQ(n_layers >= 1 && n_layers <= 65536, DV_ERR_SHAPE, "dv_decode_stack: n_layers=%d", n_layers);
    const bool ahead = (c->flags & DV_LOOKAHEAD) != 0;
    const bool dense_a = (c->flags & DV_DENSE_ATTN) != 0, dense_m = (c->flags & DV_DENSE_MLP) != 0;
    REQ(!ahead || dense_a || head_sets, DV_ERR_NULL, "dv_decode_stack: DV_LOOKAHEAD needs head_sets");
    REQ(!ahead || dense_m || neuron_sets, DV_ERR_NULL, "dv_decode_stack: DV_LOOKAHEAD needs neuron_sets");
    const size_t act = (size_t)c->B * c->d * sizeof(float);
    REQ(!overlap(x_out, act, x_in, act), DV_ERR_RANGE, "dv_decode_stack: x_out overlaps x_in");
    REQ(!overlap(x_trace, act * (n_layers - 1), x_in, act) && !overlap(x_trace, act * (n_layers - 1), x_out, act),
        DV_ERR_RANGE, "dv_decode_stack: x_trace overlaps x_in or x_out");
    int max_len = 1;
    for (int l = 0; l < n_layers; ++l) max_len = layers[l].kv.max_len > max_len ? layers[l].kv.max_len : max_len;
    const size_t lw = stack_layer_ws_bytes(c, max_len);
    const int P = c->n_dense_prefix;
    const size_t need = lw + align_up(2 * act, 256);
    REQ(ws && ws_bytes >= need, DV_ERR_WORKSPACE, "dv_decode_stack: workspace %zu < %zu", ws_bytes, need);
    float* xb[2] = {(float*)((char*)ws + lw), (float*)((char*)ws + lw) + (size_t)c->B * c->d};
    // the output of layer l (l < n_layers - 1): x_trace row l, else a ping-pong buffer
    auto out_of = [&](int l) -> float* {
        if (l == n_layers - 1) return x_out;
        return x_trace ? x_trace + (size_t)l * c->B * c->d : xb[l & 1];
    };
    const int kA = c->k_heads, nmax = layer_nmax(c);
    hipStream_t s = (hipStream_t)stream;

    // every layer's state, checked before anything is enqueued
    auto state = [&](int l, dv_layer_state& st, dv_decode_cfg& cl) {
        const dv_stack_layer& ly = layers[l];
        st = dv_layer_state{};
        st.kv = ly.kv;
        st.sel_idx = ly.sel_idx; st.sel_len = ly.sel_len; st.sel_cap = ly.sel_cap; st.sel_end = ly.sel_end;
        st.fc2_rows_out = fc2_rows;
        for (int i = 0; i < 4; ++i) st.teal_thr[i] = ly.teal_thr[i];
        st.teal_rows_out = ly.teal_rows_out; st.teal_rec = ly.teal_rec;
        cl = stack_layer_cfg(c, l);
        // a decode position shared by several layers moves on in the last of them
        for (int m = l + 1; m < n_layers; ++m)
            if (layers[m].kv.pos_dev == ly.kv.pos_dev) cl.flags &= ~(unsigned)DV_ADVANCE_POS;
        const bool la = dense_a || l < P, lm = dense_m || l < P;            // this layer computes every head / neuron
        const bool na = dense_a || l + 1 < P, nm = dense_m || l + 1 < P;    // so does the next one
        if (ahead) {
            if (!la) st.head_idx_in = head_sets + (size_t)l * kA;
            if (!lm) st.neuron_idx_in = neuron_sets + (size_t)l * nmax;
            if (l + 1 < n_layers) {
                const dv_layer_weights& wn = layers[l + 1].w;
                if (!na && kA > 0) {
                    st.next_pa1_t = wn.pa1_t; st.next_pa2_t = wn.pa2_t;
                    st.next_head_idx = head_sets + (size_t)(l + 1) * kA;
                }
                if (!nm && c->k_neurons > 0) {
                    st.next_pm1_t = wn.pm1_t; st.next_pm2_t = wn.pm2_t;
                    st.next_neuron_idx = neuron_sets + (size_t)(l + 1) * nmax;
                }
            }
        } else {
            if (!la && head_sets) st.head_idx_out = head_sets + (size_t)l * kA;
            if (!lm && neuron_sets) st.neuron_idx_out = neuron_sets + (size_t)l * nmax;
            if (!lm && neuron_counts) st.neuron_count_out = neuron_counts + l;
        }
    };
    for (int l = 0; l < n_layers; ++l) {
        dv_layer_state st;
        dv_decode_cfg cl;
        state(l, st, cl);
        const float* xi = l == 0 ? x_in : out_of(l - 1);
        float* xo = out_of(l);
        const dv_status r = decode_one(&layers[l].w, &cl, &st, xi, xo, ws, lw, s, false);
        if (r != DV_OK) {
            char msg[512];
            snprintf(msg, sizeof msg, "%s", dv_last_error());
            return fail(r, "dv_decode_stack: layer %d: %s", l, msg);
        }
        if (ahead && l + 1 < n_layers) {
            const dv_decode_cfg cn = stack_layer_cfg(c, l + 1);
            if (next_layer_predictors_missing(st, &cn, true))
                return fail(DV_ERR_NULL, "dv_decode_stack: layer %d: predictor of the next layer NULL", l + 1);
        }
    }
    if (ahead && P == 0) {   // the first layer's sets from its own predictors on LN1(x)
        const dv_layer_weights& w0 = layers[0].w;
        REQ(dense_a || kA == 0 || (w0.pa1_t && w0.pa2_t), DV_ERR_NULL, "dv_decode_stack: layer 0 head predictor NULL");
        REQ(dense_m || c->k_neurons == 0 || (w0.pm1_t && w0.pm2_t), DV_ERR_NULL, "dv_decode_stack: layer 0 neuron predictor NULL");
        const LayerWs L0 = layer_ws(ws, c, max_len);
        TRY(predict_sets(c, x_in, w0.ln1_g, w0.ln1_b, dense_a ? nullptr : w0.pa1_t, w0.pa2_t, head_sets,
                         dense_m ? nullptr : w0.pm1_t, w0.pm2_t, neuron_sets, L0, s));
    }
    for (int l = 0; l < n_layers; ++l) {
        dv_layer_state st;
        dv_decode_cfg cl;
        state(l, st, cl);
        const float* xi = l == 0 ? x_in : out_of(l - 1);
        float* xo = out_of(l);
        TRY(decode_one(&layers[l].w, &cl, &st, xi, xo, ws, lw, s, true));
    }
    return DV_OK;
}

// ---------------------------------------------------------------- launch timing --
dv_status dv_time_launches(int kernel, void** events, int n_events) {
    clear_error();
    REQ(kernel >= 0 && kernel <= DV_KERNEL_FC2, DV_ERR_DTYPE, "dv_time_launches: kernel %d", kernel);
    REQ(kernel == 0 || (events && n_events >= 2), DV_ERR_NULL, "dv_time_launches: events");
    g_timing.kind = kernel;
    g_timing.ev = kernel ? (hipEvent_t*)events : nullptr;
    g_timing.n = kernel ? n_events : 0;
    g_timing.used = 0;
    return DV_OK;
}

int dv_launch_events_used(void) { return g_timing.used; }

// ---------------------------------------------------------------- generator --
dv_status dv_fill_normal(void* out, uint64_t n, int dtype, uint64_t seed, uint64_t stream, uint64_t offset, float mean,
                         float stdv, void* hip_stream) {
    clear_error();
    REQ(n == 0 || out, DV_ERR_NULL, "dv_fill_normal: NULL pointer");
    REQ(dtype == DV_F32 || dtype == DV_F16 || dtype == DV_U32, DV_ERR_DTYPE, "dv_fill_normal: dtype %d", dtype);
    REQ(isfinite(mean) && isfinite(stdv), DV_ERR_RANGE, "dv_fill_normal: mean/std");
    REQ(offset <= UINT64_MAX - n - 4, DV_ERR_RANGE, "dv_fill_normal: offset + n overflows");
    REQ(((uintptr_t)out & 15u) == 0, DV_ERR_ALIGN, "dv_fill_normal: out must be 16-byte aligned");
    return launch_fill_normal(out, n, dtype, seed, stream, offset, mean, stdv, (hipStream_t)hip_stream);
}

// ---------------------------------------------------------------- byte account --
dv_status dv_bytes_read(const dv_decode_cfg* c, double n_att, double fc2_rows, double holes, dv_bytes* out) {
    clear_error();
    TRY(check_cfg(c));
    REQ(out, DV_ERR_NULL, "dv_bytes_read: out NULL");
    REQ(n_att >= 0 && fc2_rows >= 0 && holes >= 0, DV_ERR_RANGE, "dv_bytes_read: negative count");
    const bool dense_a = (c->flags & DV_DENSE_ATTN) != 0, dense_m = (c->flags & DV_DENSE_MLP) != 0;
    const double B = c->B, d = c->d, h = c->h, dh = c->d_h, N = c->N, wb = elt_bytes(c->wdt);
    const double kA = dense_a ? h : c->k_heads, kM = dense_m ? N : c->k_neurons;
    const double a = 4.0 * d * B;                     // one fp32 activation vector per batch row
    dv_bytes r{};
    r.head_pred = dense_a ? 0.0 : (c->r_attn * d + h * c->r_attn) * wb;
    r.neuron_pred = dense_m ? 0.0 : (c->r_mlp * d + N * c->r_mlp) * wb;
    r.qkv = (3.0 * kA * dh * d + 3.0 * kA * dh) * wb;
    r.out_proj = (kA * dh * d + d) * wb;
    r.fc1 = (kM * d + kM) * wb;
    r.fc2 = (fc2_rows * d + d) * wb;
    r.weights = r.head_pred + r.neuron_pred + r.qkv + r.out_proj + r.fc1 + r.fc2;
    r.kv_read = 2.0 * 2.0 * kA * n_att * dh * B;
    r.kv_write = 2.0 * 2.0 * kA * dh * B + holes * 2.0 * 2.0 * dh;
    // layer input and LayerNorm vectors, the predictors' inputs, the
    // residual stream in and out of each block, the stored inputs re-read
    // for recomputed K/V
    r.act = 2.0 * a + 4.0 * 4.0 * d + (dense_a ? 0.0 : a) + (dense_m ? 0.0 : a) + 4.0 * a + holes * 4.0 * d;
    r.total = r.weights + r.kv_read + r.kv_write + r.act;
    *out = r;
    return DV_OK;
}

dv_status dv_bytes_read_teal(const dv_decode_cfg* c, double n_att, const double* kept, dv_bytes* out) {
    clear_error();
    TRY(check_cfg(c));
    REQ(out && kept, DV_ERR_NULL, "dv_bytes_read_teal: NULL pointer");
    REQ(c->flags & DV_TEAL, DV_ERR_RANGE, "dv_bytes_read_teal: cfg without DV_TEAL");
    const double B = c->B, d = c->d, h = c->h, dh = c->d_h, N = c->N, wb = elt_bytes(c->wdt);
    const double width[4] = {d, h * dh, d, N};
    for (int i = 0; i < 4; ++i)
        REQ(kept[i] >= 0 && kept[i] <= width[i], DV_ERR_RANGE, "dv_bytes_read_teal: kept[%d]=%g", i, kept[i]);
    REQ(n_att >= 0, DV_ERR_RANGE, "dv_bytes_read_teal: n_att");
    const double a = 4.0 * d * B;
    dv_bytes r{};
    r.qkv = (kept[0] * 3.0 * h * dh + 3.0 * h * dh) * wb;
    r.out_proj = (kept[1] * d + d) * wb;
    r.fc1 = (kept[2] * N + N) * wb;
    r.fc2 = (kept[3] * d + d) * wb;
    r.weights = r.qkv + r.out_proj + r.fc1 + r.fc2;
    r.kv_read = 2.0 * 2.0 * h * n_att * dh * B;
    r.kv_write = 2.0 * 2.0 * h * dh * B;
    // layer input, LayerNorm vectors, the residual stream in and out of each
    // block, and the four projection inputs read by their gathers
    r.act = 2.0 * a + 4.0 * 4.0 * d + 4.0 * a + 4.0 * B * (d + h * dh + d + N);
    r.total = r.weights + r.kv_read + r.kv_write + r.act;
    *out = r;
    return DV_OK;
}

}  // extern "C"
