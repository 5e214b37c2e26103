// Sparse Q/K/V projection kernel and its launch templates (instantiated per
// weight type in k_qkv.hip and k_qkv_f32.hip).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §4.2.
#pragma once

#include "rowdot.h"

namespace dv {

// ---------------------------------------------------------------- Q/K/V -----
// DejaVu §4.2: for the selected heads compute q, k, v; store k, v in the
// cache; keep y for the heads not selected; recompute a selected head's
// missing K/V from the stored inputs, reusing the weight row already held
// in registers.  Rows are ordered [which][s][e]; a workgroup's 4 rows lie
// in one head block.
struct QkvArgs {
    const float* y;
    int B, d, h, dh, n_sel;
    const int32_t* head_idx;
    const void* w;
    const void* bias;
    float* q;
    half_t* K;
    half_t* V;
    int max_len, pos;
    const int32_t* pos_dev;   // slot read at run time, or NULL for pos
    float* y_buf;
    int32_t* valid_upto;
};

// A workgroup owns rpg consecutive rows of one (which, head) block; wave wv
// takes rows wv, wv+4, ..., double-buffered.  The head's stored inputs for
// its first HB missing positions are staged in LDS next to y.
template <typename T, int NB, int CH, bool YLDS, int HB>
__global__ __launch_bounds__(kBlock) void k_qkv(QkvArgs a, int rpg) {
    constexpr int E = Vec<T>::E;
    constexpr int HV = HB > 0 ? HB : 1;
    extern __shared__ float ys[];                      // y [NB][d], then HB stored inputs [HB][d]
    const int d = a.d, dh = a.dh;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r0 = blockIdx.x * rpg;                   // rpg divides dh: one head block per workgroup
    const int which = r0 / (a.n_sel * dh);
    const int s = (r0 / dh) % a.n_sel;
    const int e0 = r0 % dh;
    const int nchunk = d / E;
    const int head = a.head_idx ? a.head_idx[s] : s;
    const bool live = (unsigned)head < (unsigned)a.h;
    const T* Wb = (const T*)a.w + ((size_t)(which * a.h + (live ? head : 0)) * dh) * d;
    const int nk = rpg > wv ? (rpg - wv + 3) / 4 : 0;
    u32x4 wa[CH], wb[CH];
    if (live && nk > 0) load_row<T, CH, true>(Wb + (size_t)(e0 + wv) * d, nchunk, wa);
    if (YLDS) stage_rows<NB, 8>(ys, a.y, a.B, d);
    const int pos = a.pos_dev ? *a.pos_dev : a.pos;
    const bool pos_ok = pos >= 0 && pos < a.max_len;   // else the call writes nothing
    const bool fill = pos_ok && live && a.y_buf != nullptr && a.valid_upto != nullptr && which > 0;
    const int lo0 = fill ? max(a.valid_upto[head] + 1, 0) : pos;
    const int staged = (HB > 0 && fill) ? min(HB, max(pos - lo0, 0)) : 0;
    if (HB > 0 && staged > 0) stage_rows<HV, 4>(ys + NB * d, a.y_buf + (size_t)lo0 * d, staged, d);
    if (blockIdx.x == 0 && a.y_buf && pos_ok) {
        for (int i = threadIdx.x; i < a.B * d; i += kBlock) {
            const int b = i / d, c = i % d;
            a.y_buf[((size_t)b * a.max_len + pos) * d + c] = a.y[i];
        }
    }
    __syncthreads();
    if (!live || !pos_ok) return;
    half_t* cache = which == 1 ? a.K : a.V;
    auto emit = [&](int k, const u32x4 (&w)[CH]) {
        const int e = e0 + wv + 4 * k;
        const float bv = to_f32(((const T*)a.bias)[(size_t)(which * a.h + head) * dh + e]);
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        if (YLDS) dot_row<T, CH, NB>(w, nchunk, ys, d, NB, acc);
        else dot_row<T, CH, NB>(w, nchunk, a.y, d, a.B, acc);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = wave_sum(acc[b]) + bv;
        if (which == 0) {
            if (lane == 0)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < a.B) a.q[((size_t)b * a.n_sel + s) * dh + e] = acc[b];
            return;
        }
        if (lane == 0)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < a.B) cache[(((size_t)b * a.h + head) * a.max_len + pos) * dh + e] = (half_t)acc[b];
        if (!fill) return;
        if (HB > 0 && staged > 0) {                    // missing positions whose inputs are in LDS
            float hacc[HV];
#pragma unroll
            for (int v = 0; v < HV; ++v) hacc[v] = 0.f;
            dot_row<T, CH, HV>(w, nchunk, ys + NB * d, d, staged, hacc);
#pragma unroll
            for (int v = 0; v < HV; ++v) {
                const float hv = wave_sum(hacc[v]) + bv;
                if (lane == 0 && v < staged) cache[((size_t)head * a.max_len + lo0 + v) * dh + e] = (half_t)hv;
            }
        }
        for (int b = 0; b < a.B; ++b) {
            const int lo = (b == 0) ? lo0 + staged : max(a.valid_upto[b * a.h + head] + 1, 0);
            for (int p = lo; p < pos; p += 2) {
                const int cnt = min(2, pos - p);
                const float* base = a.y_buf + ((size_t)b * a.max_len + p) * d;
                float hacc[2] = {0.f, 0.f};
                // two stored inputs per pass, straight from global memory (L2)
                dot_row<T, CH, 2>(w, nchunk, base, d, cnt, hacc);
#pragma unroll
                for (int v = 0; v < 2; ++v) {
                    const float hv = wave_sum(hacc[v]) + bv;
                    if (lane == 0 && v < cnt)
                        cache[(((size_t)b * a.h + head) * a.max_len + p + v) * dh + e] = (half_t)hv;
                }
            }
        }
    };
    for (int k = 0; k < nk; k += 2) {
        if (k + 1 < nk) load_row<T, CH, true>(Wb + (size_t)(e0 + wv + 4 * (k + 1)) * d, nchunk, wb);
        emit(k, wa);
        if (k + 1 < nk) {
            if (k + 2 < nk) load_row<T, CH, true>(Wb + (size_t)(e0 + wv + 4 * (k + 2)) * d, nchunk, wa);
            emit(k + 1, wb);
        }
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

#define DV_LAUNCH_CHECK()                                                          \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e_)); \
    } while (0)

template <typename T, int NB, bool YLDS, int HB>
static void qkv_go2(const QkvArgs& a, int ch, size_t lds, hipStream_t s) {
    const int rows = 3 * a.n_sel * a.dh;
    int rpg = rows_per_group(rows);
    while (a.dh % rpg) rpg -= 4;                       // a workgroup stays inside one head block
    const int grid = rows / rpg;
    switch (ch) {
        case 4: hipLaunchKernelGGL((k_qkv<T, NB, 4, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 8: hipLaunchKernelGGL((k_qkv<T, NB, 8, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 10: hipLaunchKernelGGL((k_qkv<T, NB, 10, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 12: hipLaunchKernelGGL((k_qkv<T, NB, 12, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 16: hipLaunchKernelGGL((k_qkv<T, NB, 16, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 18: hipLaunchKernelGGL((k_qkv<T, NB, 18, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        default: hipLaunchKernelGGL((k_qkv<T, NB, 24, YLDS, HB>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
    }
}

template <typename T, int NB>
static dv_status qkv_go(const QkvArgs& a, int ch, hipStream_t s) {
    if (ch == 0) return fail(DV_ERR_UNSUPPORTED, "Q/K/V projection: rows of d=%d are too long", a.d);
    const size_t row = (size_t)a.d * sizeof(float);
    const size_t lds = NB * row;
    const bool holes = a.y_buf && a.valid_upto;
    if constexpr (NB == 1) {
        if (holes && lds + 2 * row <= kYLdsMax) {
            qkv_go2<T, NB, true, 2>(a, ch, lds + 2 * row, s);
            return DV_OK;
        }
        if (holes && lds + row <= kYLdsMax) {
            qkv_go2<T, NB, true, 1>(a, ch, lds + row, s);
            return DV_OK;
        }
    }
    if (lds <= kYLdsMax) qkv_go2<T, NB, true, 0>(a, ch, lds, s);
    else qkv_go2<T, NB, false, 0>(a, ch, 0, s);
    return DV_OK;
}

template <typename T>
dv_status qkv_launch_t(const QkvArgs& a, int ch, hipStream_t s) {
    switch (nb_bucket(a.B)) {
        case 1: return qkv_go<T, 1>(a, ch, s);
        case 2: return qkv_go<T, 2>(a, ch, s);
        case 4: return qkv_go<T, 4>(a, ch, s);
        case 8: return qkv_go<T, 8>(a, ch, s);
        default: return qkv_go<T, 16>(a, ch, s);
    }
}

}  // namespace dvh
