// Row-dot kernels: sparse fc1 (DejaVu Eq. 1, first layer) and the
// predictor's first layer, one weight row per wave, double-buffered.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).
#include "rowdot.h"

namespace dv {

// A workgroup owns rows [blockIdx.x * rpg, +rpg); wave wv takes rows
// wv, wv+4, ... of them, double-buffered: the next row's loads are in
// flight while the current row is reduced.  y reaches LDS by DMA, issued
// before the first row's loads (batch rows past B are never read: their
// sums are discarded).
template <typename T, int NB, int CH, int OP>
__global__ __launch_bounds__(kBlock) void k_rowdot(RowArgs a, int rpg) {
    constexpr int E = Vec<T>::E;
    extern __shared__ float ys[];
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int u0 = blockIdx.x * rpg;
    if (u0 >= n) return;                                  // whole workgroup idle
    const int u1 = min(n, u0 + rpg);
    const int nk = u1 - u0 > wv ? (u1 - u0 - wv + 3) / 4 : 0;   // rows of this wave
    const int nchunk = a.d / E;
    // all of this wave's row indices in one load (lane k holds row k's),
    // then fc1's biases the same way, kept as bits until used (read as
    // converted values they would make the wave wait for every load before
    // them, the next row's included)
    int my_j = -1;
    if ((threadIdx.x & 63) < nk) {
        const int u = u0 + wv + 4 * (threadIdx.x & 63);
        const int j = a.idx ? a.idx[u] : u;
        my_j = (unsigned)j < (unsigned)a.w_rows ? j : -1;   // an index outside W selects nothing
    }
    const unsigned my_b = OP == ROW_FC1 ? elt_bits((const T*)a.bias + (my_j >= 0 ? my_j : 0)) : 0u;
    auto row_of = [&](int k) -> int { return __builtin_amdgcn_readlane(my_j, k); };   // k is wave-uniform
    stage_dma(ys, a.y, a.B * a.d);                        // y straight into LDS, ahead of the rows
    u32x4 wa[CH], wb[CH];
    int ja = nk > 0 ? row_of(0) : -1, jb = -1;
    if (ja >= 0) {
        // all CH loads go out (chunks past the row re-read chunk 0, never
        // used), so that a wait for CH outstanding covers y's DMA
        load_row_all<T, CH>((const T*)a.w + (size_t)ja * a.d, nchunk, wa);
        sync_after_dma<CH>();                             // y has landed; the row may still be in flight
    } else {
        sync_after_dma<0>();
    }
    auto emit = [&](int k, int j, const u32x4 (&w)[CH]) {
        const int u = u0 + wv + 4 * k;
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        if (j >= 0) dot_row<T, CH, NB>(w, nchunk, ys, a.d, NB, acc);
        const float bj = (OP == ROW_FC1 && j >= 0) ? bits_f32<T>(__builtin_amdgcn_readlane(my_b, k)) : 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float v = wave_sum(acc[b]);
            if (OP == ROW_FC1) v = j >= 0 ? fmaxf(v + bj, 0.f) : 0.f;
            if ((threadIdx.x & 63) == 0 && b < a.B) a.out[(size_t)b * a.n_max + u] = v;
        }
    };
    for (int k = 0; k < nk; k += 2) {
        if (k + 1 < nk) {
            jb = row_of(k + 1);
            if (jb >= 0) load_row<T, CH, true>((const T*)a.w + (size_t)jb * a.d, nchunk, wb);
        }
        emit(k, ja, wa);
        if (k + 1 < nk) {
            if (k + 2 < nk) {
                ja = row_of(k + 2);
                if (ja >= 0) load_row<T, CH, true>((const T*)a.w + (size_t)ja * a.d, nchunk, wa);
            }
            emit(k + 1, jb, wb);
        }
    }
}

// Generic path for rows longer than 64 * 24 chunks or batches whose inputs
// do not fit in LDS: y from global memory, the row streamed U chunks at a time.
template <typename T, int NB, int OP>
__global__ __launch_bounds__(kBlock) void k_rowdot_long(RowArgs a) {
    constexpr int E = Vec<T>::E;
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= n) return;
    const int nchunk = a.d / E;
    const int j = a.idx ? a.idx[u] : u;
    const bool live = (unsigned)j < (unsigned)a.w_rows;
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    if (live) wave_rowdot<T, NB, 8, true>((const T*)a.w + (size_t)j * a.d, nchunk, a.y, a.d, a.B, acc);
    const float bj = (OP == ROW_FC1 && live) ? to_f32(((const T*)a.bias)[j]) : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float v = wave_sum(acc[b]);
        if (OP == ROW_FC1) v = live ? fmaxf(v + bj, 0.f) : 0.f;
        if ((threadIdx.x & 63) == 0 && b < a.B) a.out[(size_t)b * a.n_max + u] = v;
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

template <typename T, int NB, int OP>
static void rowdot_go(const RowArgs& a, int ch, hipStream_t s) {
    const size_t lds = (size_t)NB * a.d * sizeof(float);
    const bool fits = ch > 0 && lds <= kYLdsMax;
    if (!fits) {
        DV_LAUNCH((k_rowdot_long<T, NB, OP>), dim3(cdiv(a.n_max, 4)), dim3(kBlock), 0, s, a);
        return;
    }
    const int rpg = rows_per_group(a.n_max);
    const int grid = cdiv(a.n_max, rpg);
    switch (ch) {
        case 4: DV_LAUNCH((k_rowdot<T, NB, 4, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 8: DV_LAUNCH((k_rowdot<T, NB, 8, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 10: DV_LAUNCH((k_rowdot<T, NB, 10, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 12: DV_LAUNCH((k_rowdot<T, NB, 12, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 16: DV_LAUNCH((k_rowdot<T, NB, 16, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        case 18: DV_LAUNCH((k_rowdot<T, NB, 18, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
        default: DV_LAUNCH((k_rowdot<T, NB, 24, OP>), dim3(grid), dim3(kBlock), lds, s, a, rpg); break;
    }
}

template <int OP>
static dv_status rowdot(const RowArgs& a, int wdt, hipStream_t s) {
    if (a.n_max == 0) return DV_OK;
    const int ch = ch_tier(a.d, wdt);
#define DV_RD(NB)                                                          \
    case NB:                                                               \
        if (wdt == DV_F16) rowdot_go<half_t, NB, OP>(a, ch, s);            \
        else rowdot_go<float, NB, OP>(a, ch, s);                           \
        break;
    switch (nb_bucket(a.B)) {
        DV_RD(1) DV_RD(2) DV_RD(4) DV_RD(8) DV_RD(16)
    }
#undef DV_RD
    DV_LAUNCH_CHECK();
    return DV_OK;
}

dv_status rowdot_plain(const RowArgs& a, int wdt, hipStream_t s) { return rowdot<ROW_PLAIN>(a, wdt, s); }

dv_status launch_fc1(const float* y, int B, int d, const void* w1_t, const void* b1, int wdt,
                     const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a_out, hipStream_t s) {
    RowArgs a{};
    a.y = y; a.B = B; a.d = d; a.w = w1_t; a.bias = b1; a.idx = idx;
    a.n_max = n_max; a.n_dev = n_dev; a.w_rows = N; a.out = a_out;
    return rowdot<ROW_FC1>(a, wdt, s);
}

}  // namespace dvh
