// LayerNorm, the predictor's second layer, the predictor's first layer with
// LayerNorm folded in, and the valid-position update of hole fill.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).
#include "pred.h"

namespace dv {

__global__ __launch_bounds__(kLnThreads) void k_layernorm(const float* __restrict__ x, int d,
                                                          const float* __restrict__ g,
                                                          const float* __restrict__ b, float eps,
                                                          float* y) {
    __shared__ float red[16];
    const f32x4* xr = reinterpret_cast<const f32x4*>(x + (size_t)blockIdx.x * d);
    const int n4 = d / 4;
    f32x4 v[kLnVec];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        v[i] = c < n4 ? xr[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    const float mean = block_sum1024(s, red) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        if (c < n4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float t = v[i][e] - mean;
                q = fmaf(t, t, q);
            }
    }
    const float var = block_sum1024(q, red) / (float)d;
    const float rstd = 1.0f / sqrtf(var + eps);
    const f32x4* g4 = reinterpret_cast<const f32x4*>(g);
    const f32x4* b4 = reinterpret_cast<const f32x4*>(b);
    f32x4* yr = reinterpret_cast<f32x4*>(y + (size_t)blockIdx.x * d);
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) {
        const int c = threadIdx.x + i * kLnThreads;
        if (c < n4) {
            const f32x4 gg = g4[c], bb = b4[c];
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (v[i][e] - mean) * rstd * gg[e] + bb[e];
            yr[c] = o;
        }
    }
}

// The row-dot with LayerNorm folded in, one workgroup per block of 4 rows.
template <typename T, int CH, int OP, int RR, bool GB>
__global__ __launch_bounds__(kBlock) void k_rowdot_ln(RowArgs a, LnArgs ln) {
    extern __shared__ float ys[];
    rowdot_ln_block<T, CH, OP, RR, kBlock, GB>(blockIdx.x, ys, a, ln);
}

template <typename T, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_scores(const float* __restrict__ hid_in, int B, int r, int act,
                                                        const T* __restrict__ p2, int n_out, int lpr,
                                                        int rows_per_block, float* __restrict__ scores) {
    extern __shared__ float hid[];
    pred_scores_block<T, NB>(blockIdx.x, hid, hid_in, B, r, act, p2, n_out, lpr, rows_per_block, scores);
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_pred_topk_small(const float* __restrict__ hid_in, int r, int act,
                                                            const T* __restrict__ p2, int n_out,
                                                            float* __restrict__ scores, int k,
                                                            int32_t* __restrict__ idx) {
    pred_topk_small_block<T>(hid_in, r, act, p2, n_out, scores, k, idx);
}

// Both predictors' second layers in one launch: workgroup 0 scores the heads
// and selects k_h of them, the others score the neurons (their selection is
// the next launch).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_pred2_pair(Pred2Args a) {
    extern __shared__ float hid[];
    pred2_pair_block<T>(blockIdx.x, hid, a);
}

}  // namespace dv

namespace dvh {
using namespace dv;

#define DV_LAUNCH_CHECK()                                                          \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e_)); \
    } while (0)

dv_status launch_layernorm(const float* x, int B, int d, const float* g, const float* b, float eps,
                           float* y, hipStream_t s) {
    hipLaunchKernelGGL(k_layernorm, dim3(B), dim3(kLnThreads), 0, s, x, d, g, b, eps, y);
    DV_LAUNCH_CHECK();
    return DV_OK;
}

dv_status rowdot_plain(const RowArgs& a, int wdt, hipStream_t s);

size_t pred_partials(int B, int d, int r, int wdt) {
    (void)d; (void)wdt;
    return (size_t)B * r;
}

template <typename T, int NB>
static void scores_go(const float* hid, int B, int r, int act, const void* p2, int n_out, float* scores,
                      hipStream_t s) {
    constexpr int E = Vec<T>::E;
    const int rchunk = r / E;
    int lpr = 1;
    while (lpr < rchunk && lpr < kWave) lpr *= 2;
    const int rows_per_block = (kWave / lpr) * 4 * 4;
    const int r_pad = (r + 3) & ~3;
    hipLaunchKernelGGL((k_pred_scores<T, NB>), dim3(cdiv(n_out, rows_per_block)), dim3(kBlock),
                       (size_t)NB * r_pad * sizeof(float), s, hid, B, r, act, (const T*)p2, n_out, lpr,
                       rows_per_block, scores);
}

dv_status launch_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                         int n_out, int wdt, int act, float* scores, float* hid, hipStream_t s, float* mpart) {
    if (mpart && rowdot_mfma_ok(B, d, wdt) && rowdot_mfma_ok(B, r, wdt)) {
        // both layers on the matrix cores; the activation is applied to the
        // hidden layer as it is written
        dv_status st = launch_rows_mfma(y, B, d, p1_t, r, act == DV_ACT_RELU, hid, mpart, s);
        if (st != DV_OK) return st;
        return launch_rows_mfma(hid, B, r, p2_t, n_out, false, scores, mpart, s);
    }
    RowArgs a{};
    a.y = y; a.B = B; a.d = d; a.w = p1_t; a.bias = nullptr; a.idx = nullptr;
    a.n_max = r; a.n_dev = nullptr; a.w_rows = r; a.out = hid;
    dv_status st = rowdot_plain(a, wdt, s);
    if (st != DV_OK) return st;
#define DV_SC(NB)                                                                              \
    case NB:                                                                                   \
        if (wdt == DV_F16) scores_go<half_t, NB>(hid, B, r, act, p2_t, n_out, scores, s);      \
        else scores_go<float, NB>(hid, B, r, act, p2_t, n_out, scores, s);                     \
        break;
    switch (nb_bucket(B)) {
        DV_SC(1) DV_SC(2) DV_SC(4) DV_SC(8) DV_SC(16)
    }
#undef DV_SC
    DV_LAUNCH_CHECK();
    return DV_OK;
}

bool ln_fusable(int B, int d) { return B == 1 && (size_t)d * sizeof(float) <= kYLdsMax && d % 4 == 0; }

template <typename T, int OP>
static dv_status predict_ln_t(const RowArgs& a, const LnArgs& ln, int ch, hipStream_t s) {
    const int grid = cdiv(a.n_max, 4);
    // gamma and beta staged in LDS beside x when the three fit
    const bool gb = 3 * (size_t)a.d * sizeof(float) <= kYLdsMax;
    const size_t lds = (gb ? 3 : 1) * (size_t)a.d * sizeof(float);
#define DV_RL(CH)                                                                                              \
    case CH:                                                                                                   \
        if (gb) DV_LAUNCH((k_rowdot_ln<T, CH, OP, 1, true>), dim3(grid), dim3(kBlock), lds, s, a, ln);          \
        else DV_LAUNCH((k_rowdot_ln<T, CH, OP, 1, false>), dim3(grid), dim3(kBlock), lds, s, a, ln);           \
        break;
    switch (ch) {
        DV_RL(4) DV_RL(8) DV_RL(10) DV_RL(12) DV_RL(16) DV_RL(18) DV_RL(24)
        default: return fail(DV_ERR_UNSUPPORTED, "fused LayerNorm: d=%d", a.d);
    }
#undef DV_RL
    return DV_OK;
}

dv_status launch_predict_ln(const float* x, int B, int d, const float* g, const float* b, float eps, float* y_out,
                            const void* p1_t, int r, const void* p2_t, int n_out, int wdt, int act, float* scores,
                            float* hid, hipStream_t s, float* mpart) {
    if (!ln_fusable(B, d) || ch_tier(d, wdt) == 0) {
        dv_status st = launch_layernorm(x, B, d, g, b, eps, y_out, s);
        if (st != DV_OK) return st;
        return launch_predict(y_out, B, d, p1_t, r, p2_t, n_out, wdt, act, scores, hid, s, mpart);
    }
    RowArgs a{};
    a.y = nullptr; a.B = 1; a.d = d; a.w = p1_t; a.n_max = r; a.w_rows = r; a.out = hid;
    LnArgs ln{x, g, b, eps, y_out};
    dv_status st = wdt == DV_F16 ? predict_ln_t<half_t, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s)
                                 : predict_ln_t<float, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s);
    if (st != DV_OK) return st;
    DV_LAUNCH_CHECK();
#define DV_SC(NB)                                                                              \
    case NB:                                                                                   \
        if (wdt == DV_F16) scores_go<half_t, NB>(hid, B, r, act, p2_t, n_out, scores, s);      \
        else scores_go<float, NB>(hid, B, r, act, p2_t, n_out, scores, s);                     \
        break;
    switch (nb_bucket(B)) {
        DV_SC(1)
    }
#undef DV_SC
    DV_LAUNCH_CHECK();
    return DV_OK;
}

dv_status launch_fc1_ln(const float* x, int d, const float* g, const float* b, float eps, const void* w1_t,
                        const void* b1, int wdt, const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a_out,
                        hipStream_t s) {
    if (n_max == 0) return DV_OK;
    if (!ln_fusable(1, d) || ch_tier(d, wdt) == 0) return fail(DV_ERR_UNSUPPORTED, "fc1 with LayerNorm: d=%d", d);
    RowArgs a{};
    a.y = nullptr; a.B = 1; a.d = d; a.w = w1_t; a.bias = b1; a.idx = idx; a.n_max = n_max; a.n_dev = n_dev;
    a.w_rows = N; a.out = a_out;
    LnArgs ln{x, g, b, eps, nullptr};
    dv_status st = wdt == DV_F16 ? predict_ln_t<half_t, ROW_FC1>(a, ln, ch_tier(d, wdt), s)
                                 : predict_ln_t<float, ROW_FC1>(a, ln, ch_tier(d, wdt), s);
    if (st != DV_OK) return st;
    DV_LAUNCH_CHECK();
    return DV_OK;
}

// Both predictors of a layer from one normalised input: one layer-one launch
// over the head and neuron predictors' rows, one launch for both second
// layers (the heads also selected).  hid holds rA + rM floats.
dv_status launch_predict_pair_ln(const float* x, int d, const float* g, const float* b, float eps, float* y_out,
                                 const void* pa1_t, int rA, const void* pa2_t, int h, int kA, int32_t* idxA,
                                 const void* pm1_t, int rM, const void* pm2_t, int N, float* sA, float* sM, float* hid,
                                 int wdt, int act, hipStream_t s) {
    if (!row_ln_supported(d, wdt) || !pred_topk_fusable(1, h, rA))
        return fail(DV_ERR_UNSUPPORTED, "paired predictors: d=%d h=%d r=%d", d, h, rA);
    RowArgs a{};
    a.y = nullptr; a.B = 1; a.d = d; a.w = pa1_t; a.w2 = pm1_t; a.split = rA; a.n_max = rA + rM; a.w_rows = rA + rM;
    a.out = hid;
    LnArgs ln{x, g, b, eps, y_out};
    dv_status st = wdt == DV_F16 ? predict_ln_t<half_t, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s)
                                 : predict_ln_t<float, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s);
    if (st != DV_OK) return st;
    DV_LAUNCH_CHECK();
    const Pred2Args p2 = pred2_args(hid, rA, pa2_t, h, sA, kA, idxA, hid + rA, rM, pm2_t, N, sM, act, wdt);
    const size_t lds = (size_t)((rM + 3) & ~3) * sizeof(float);
    if (wdt == DV_F16) hipLaunchKernelGGL(k_pred2_pair<half_t>, dim3(pred2_blocks(p2)), dim3(kBlock), lds, s, p2);
    else hipLaunchKernelGGL(k_pred2_pair<float>, dim3(pred2_blocks(p2)), dim3(kBlock), lds, s, p2);
    DV_LAUNCH_CHECK();
    return DV_OK;
}

Pred2Args pred2_args(const float* hid_a, int r_a, const void* p2_a, int n_a, float* s_a, int k_a, int32_t* idx_a,
                     const float* hid_m, int r_m, const void* p2_m, int n_m, float* s_m, int act, int wdt) {
    Pred2Args p{};
    p.hid_a = hid_a; p.r_a = r_a; p.p2_a = p2_a; p.n_a = n_a; p.s_a = s_a; p.k_a = k_a; p.idx_a = idx_a;
    p.hid_m = hid_m; p.r_m = r_m; p.p2_m = p2_m; p.n_m = n_m; p.s_m = s_m; p.act = act; p.wdt = wdt;
    const int rchunk = r_m / (16 / elt_bytes(wdt));
    p.lpr = 1;
    while (p.lpr < rchunk && p.lpr < kWave) p.lpr *= 2;
    p.rows_per_block = (kWave / p.lpr) * 4 * 4;
    return p;
}

bool row_ln_supported(int d, int wdt) { return ln_fusable(1, d) && ch_tier(d, wdt) != 0; }

bool pred_topk_fusable(int B, int n_out, int r) { return B == 1 && n_out <= kBlock && r <= 512; }

dv_status launch_predict_ln_topk(const float* x, int d, const float* g, const float* b, float eps, float* y_out,
                                 const void* p1_t, int r, const void* p2_t, int n_out, int wdt, int act,
                                 float* scores, float* hid, int k, int32_t* idx, hipStream_t s) {
    if (ln_fusable(1, d) && ch_tier(d, wdt) != 0) {
        RowArgs a{};
        a.y = nullptr; a.B = 1; a.d = d; a.w = p1_t; a.n_max = r; a.w_rows = r; a.out = hid;
        LnArgs ln{x, g, b, eps, y_out};
        dv_status st = wdt == DV_F16 ? predict_ln_t<half_t, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s)
                                     : predict_ln_t<float, ROW_PLAIN>(a, ln, ch_tier(d, wdt), s);
        if (st != DV_OK) return st;
    } else {
        dv_status st = launch_layernorm(x, 1, d, g, b, eps, y_out, s);
        if (st != DV_OK) return st;
        RowArgs a{};
        a.y = y_out; a.B = 1; a.d = d; a.w = p1_t; a.bias = nullptr; a.idx = nullptr;
        a.n_max = r; a.n_dev = nullptr; a.w_rows = r; a.out = hid;
        st = rowdot_plain(a, wdt, s);
        if (st != DV_OK) return st;
    }
    DV_LAUNCH_CHECK();
    if (wdt == DV_F16)
        hipLaunchKernelGGL(k_pred_topk_small<half_t>, dim3(1), dim3(kBlock), 0, s, hid, r, act, (const half_t*)p2_t,
                           n_out, scores, k, idx);
    else
        hipLaunchKernelGGL(k_pred_topk_small<float>, dim3(1), dim3(kBlock), 0, s, hid, r, act, (const float*)p2_t,
                           n_out, scores, k, idx);
    DV_LAUNCH_CHECK();
    return DV_OK;
}

}  // namespace dvh
