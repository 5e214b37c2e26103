// Row-dot kernels of the decode step: LayerNorm, the two predictor layers,
// sparse fc1 and the sparse Q/K/V projections with KV append and hole fill.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).
//
// Layout of work: one wave streams one weight row of d elements as 16-byte
// chunks (lane l takes chunks l, l+64, ...), so a 10 KB fp16 row of d=5120 is
// ten fully coalesced 1 KB wave loads.  The layer input y lives in LDS when
// it fits (loaded once per workgroup, reused by all its rows).
#include "dv_internal.h"

#include <math.h>

namespace dv {

// ---------------------------------------------------------------- LayerNorm --
// DejaVu App. B: a normalisation precedes each block of the residual stream.
__device__ __forceinline__ float block_sum256(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__global__ __launch_bounds__(kBlock) void k_layernorm(const float* __restrict__ x, int d,
                                                      const float* __restrict__ g,
                                                      const float* __restrict__ b, float eps,
                                                      float* y) {
    __shared__ float red[4];
    const float* xr = x + (size_t)blockIdx.x * d;
    float* yr = y + (size_t)blockIdx.x * d;
    float s = 0.f;
    for (int i = threadIdx.x; i < d; i += kBlock) s += xr[i];
    const float mean = block_sum256(s, red) / (float)d;
    float v = 0.f;
    for (int i = threadIdx.x; i < d; i += kBlock) {
        const float t = xr[i] - mean;
        v = fmaf(t, t, v);
    }
    const float var = block_sum256(v, red) / (float)d;
    const float rstd = 1.0f / sqrtf(var + eps);
    for (int i = threadIdx.x; i < d; i += kBlock) yr[i] = (xr[i] - mean) * rstd * g[i] + b[i];
}

// ---------------------------------------------------------------- predictor --
// DejaVu §4.1/§4.2: SP(y) = act(y P1) P2.  Layer 1 (r rows of length d) is
// split along d into S segments so that r*S waves share the read; layer 2
// sums the segment partials, applies act and scores every output row.
template <typename T, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_hidden(const float* __restrict__ y, int B, int d,
                                                        const T* __restrict__ p1, int r, int S,
                                                        int seg_chunks, float* __restrict__ part) {
    constexpr int E = Vec<T>::E;
    const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= r * S) return;
    const int k = task / S, seg = task % S;
    const int nchunk = d / E;
    const int c0 = seg * seg_chunks;
    const int c1 = min(nchunk, c0 + seg_chunks);
    float acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = 0.f;
    if (c1 > c0)
        wave_rowdot<T, NB, 4, false>(p1 + (size_t)k * d + (size_t)c0 * E, c1 - c0, y + (size_t)c0 * E, d, B, acc);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float v = wave_sum(acc[b]);
        if ((threadIdx.x & 63) == 0 && b < B) part[((size_t)b * S + seg) * r + k] = v;
    }
}

template <typename T, int NB>
__global__ __launch_bounds__(kBlock) void k_pred_scores(const float* __restrict__ part, int B, int S,
                                                        int r, int act, const T* __restrict__ p2,
                                                        int n_out, int lpr, int rows_per_block,
                                                        float* __restrict__ scores) {
    constexpr int E = Vec<T>::E;
    extern __shared__ float hid[];                       // [NB][r_pad]
    const int r_pad = (r + 3) & ~3;
    for (int i = threadIdx.x; i < NB * r_pad; i += kBlock) {
        const int b = i / r_pad, k = i % r_pad;
        float v = 0.f;
        if (b < B && k < r) {
            for (int s = 0; s < S; ++s) v += part[((size_t)b * S + s) * r + k];
            if (act == DV_ACT_RELU) v = fmaxf(v, 0.f);
        }
        hid[i] = v;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int grp = lane / lpr, t = lane % lpr;
    const int rpw = kWave / lpr;                         // rows per wave pass
    const int rchunk = r / E;                            // r*wb is a multiple of 16
    const int j0 = blockIdx.x * rows_per_block;
    const int j1 = min(n_out, j0 + rows_per_block);
    for (int jb = j0 + wv * rpw; jb < j1; jb += 4 * rpw) {
        const int j = jb + grp;
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        if (j < j1) {
            const T* row = p2 + (size_t)j * r;
            for (int c = t; c < rchunk; c += lpr) {
                float f[E];
                unpack(ld16(row + (size_t)c * E), f, T());
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[b] = fmaf(f[e], hid[b * r_pad + c * E + e], acc[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float v = group_sum_dyn(acc[b], lpr);
            if (t == 0 && j < j1 && b < B) scores[(size_t)b * n_out + j] = v;
        }
    }
}

// ---------------------------------------------------------------- fc1 -------
// DejaVu §2.3 Eq. (1), first layer: a[b][u] = relu(W1_j . y[b] + b1_j),
// j = idx[u]; only the selected rows of W1^T are read (§4.4 kernel fusion:
// index and multiply in one pass, no gathered copy).
template <typename T, int NB, bool YLDS>
__global__ __launch_bounds__(kBlock) void k_fc1(const float* __restrict__ y, int B, int d,
                                                const T* __restrict__ w1, const T* __restrict__ b1,
                                                const int32_t* __restrict__ idx, int n_max,
                                                const int32_t* __restrict__ n_dev, int N, int rw,
                                                float* __restrict__ a) {
    constexpr int E = Vec<T>::E;
    extern __shared__ float ys[];
    const int n = n_dev ? min(*n_dev, n_max) : n_max;
    const int row0 = blockIdx.x * 4 * rw;
    if (row0 >= n) return;
    const float* yv = y;
    if (YLDS) {
        for (int i = threadIdx.x; i < NB * d; i += kBlock) ys[i] = (i / d < B) ? y[i] : 0.f;
        __syncthreads();
        yv = ys;
    }
    const int nchunk = d / E;
    const int wv = threadIdx.x >> 6;
    for (int it = 0; it < rw; ++it) {
        const int u = row0 + wv + 4 * it;
        if (u >= n) break;
        const int j = idx ? idx[u] : u;
        if ((unsigned)j >= (unsigned)N) {          // an index outside the layer selects nothing
            if ((threadIdx.x & 63) == 0)
                for (int b = 0; b < B; ++b) a[(size_t)b * n_max + u] = 0.f;
            continue;
        }
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        wave_rowdot<T, NB, 8, true>(w1 + (size_t)j * d, nchunk, yv, d, YLDS ? NB : B, acc);
        const float bj = to_f32(b1[j]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float v = wave_sum(acc[b]) + bj;
            if ((threadIdx.x & 63) == 0 && b < B) a[(size_t)b * n_max + u] = fmaxf(v, 0.f);
        }
    }
}

// ---------------------------------------------------------------- Q/K/V -----
// DejaVu §4.2: for the selected heads compute q, k, v; store k, v in the
// cache; keep y for the heads not selected; recompute a selected head's
// missing K/V from the stored inputs.  Rows are ordered [which][s][e] so a
// workgroup streams contiguous memory of one head block.
struct QkvArgs {
    const float* y;
    int B, d, h, dh, n_sel, rw;
    const int32_t* head_idx;
    const void* w;
    const void* bias;
    float* q;
    half_t* K;
    half_t* V;
    int max_len, pos;
    float* y_buf;
    int32_t* valid_upto;
    unsigned* counter;
};

// Dot of a row with up to 4 vectors at independent addresses (hole inputs).
template <typename T>
__device__ __forceinline__ void wave_rowdot4p(const T* __restrict__ row, int nchunk,
                                              const float* p0, const float* p1, const float* p2,
                                              const float* p3, float (&acc)[4]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
    const float* ps[4] = {p0, p1, p2, p3};
    for (int c = lane; c < nchunk; c += kWave) {
        float f[E];
        unpack(ld16(row + (size_t)c * E), f, T());
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float* yv = ps[v] + (size_t)c * E;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[v] = fmaf(f[e], yv[e], acc[v]);
        }
    }
}

template <typename T, int NB, bool YLDS>
__global__ __launch_bounds__(kBlock) void k_qkv(QkvArgs a) {
    constexpr int E = Vec<T>::E;
    extern __shared__ float ys[];
    const T* W = (const T*)a.w;
    const T* bias = (const T*)a.bias;
    const int d = a.d, dh = a.dh;
    const int rows = 3 * a.n_sel * dh;
    const bool fill = a.y_buf != nullptr && a.valid_upto != nullptr;
    const float* yv = a.y;
    if (YLDS) {
        for (int i = threadIdx.x; i < NB * d; i += kBlock) ys[i] = (i / d < a.B) ? a.y[i] : 0.f;
        __syncthreads();
        yv = ys;
    }
    if (blockIdx.x == 0 && a.y_buf) {
        for (int i = threadIdx.x; i < a.B * d; i += kBlock) {
            const int b = i / d, c = i % d;
            a.y_buf[((size_t)b * a.max_len + a.pos) * d + c] = a.y[i];
        }
    }
    const int nchunk = d / E;
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row0 = blockIdx.x * 4 * a.rw;
    for (int it = 0; it < a.rw; ++it) {
        const int r = row0 + wv + 4 * it;
        if (r >= rows) break;
        const int which = r / (a.n_sel * dh);
        const int s = (r / dh) % a.n_sel;
        const int e = r % dh;
        const int head = a.head_idx ? a.head_idx[s] : s;
        if ((unsigned)head >= (unsigned)a.h) continue;     // not a head of this layer
        const size_t wrow = ((size_t)(which * a.h + head) * dh + e);
        const T* row = W + wrow * d;
        const float bv = to_f32(bias[wrow]);
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        wave_rowdot<T, NB, 8, true>(row, nchunk, yv, d, YLDS ? NB : a.B, acc);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = wave_sum(acc[b]) + bv;
        if (which == 0) {
            if (lane == 0)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < a.B) a.q[((size_t)b * a.n_sel + s) * dh + e] = acc[b];
            continue;
        }
        half_t* cache = which == 1 ? a.K : a.V;
        if (lane == 0)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < a.B) cache[(((size_t)b * a.h + head) * a.max_len + a.pos) * dh + e] = (half_t)acc[b];
        if (!fill) continue;
        for (int b = 0; b < a.B; ++b) {
            const int lo = a.valid_upto[b * a.h + head] + 1;
            for (int p = max(lo, 0); p < a.pos; p += 4) {
                const int cnt = min(4, a.pos - p);
                const float* base = a.y_buf + ((size_t)b * a.max_len + p) * d;
                float hacc[4] = {0.f, 0.f, 0.f, 0.f};
                wave_rowdot4p<T>(row, nchunk, base, base + (cnt > 1 ? d : 0), base + (cnt > 2 ? 2 * d : 0),
                                 base + (cnt > 3 ? 3 * d : 0), hacc);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float hv = wave_sum(hacc[v]) + bv;
                    if (lane == 0 && v < cnt)
                        cache[(((size_t)b * a.h + head) * a.max_len + p + v) * dh + e] = (half_t)hv;
                }
            }
        }
    }
    if (!fill) return;
    // The last workgroup to finish marks the selected heads as filled up to pos.
    __shared__ int last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int i = threadIdx.x; i < a.B * a.n_sel; i += kBlock) {
        const int b = i / a.n_sel, s = i % a.n_sel;
        const int head = a.head_idx ? a.head_idx[s] : s;
        if ((unsigned)head < (unsigned)a.h) a.valid_upto[b * a.h + head] = a.pos;
    }
    if (threadIdx.x == 0) *a.counter = 0u;
}

}  // namespace dv

// ============================================================== launchers ====
namespace dvh {
using namespace dv;

#define DV_LAUNCH_CHECK()                                                          \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e_)); \
    } while (0)

dv_status launch_layernorm(const float* x, int B, int d, const float* g, const float* b, float eps,
                           float* y, hipStream_t s) {
    hipLaunchKernelGGL(k_layernorm, dim3(B), dim3(kBlock), 0, s, x, d, g, b, eps, y);
    DV_LAUNCH_CHECK();
    return DV_OK;
}

static int nb_bucket(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

static void pred_split(int d, int wdt, int* S, int* seg_chunks) {
    const int E = 16 / elt_bytes(wdt);
    const int nchunk = d / E;
    *seg_chunks = 2 * kWave;                      // two chunks per lane per task
    *S = cdiv(nchunk, *seg_chunks);
}

size_t pred_partials(int B, int d, int r, int wdt) {
    int S, sc;
    pred_split(d, wdt, &S, &sc);
    return (size_t)B * S * r;
}

template <typename T, int NB>
static dv_status predict_t(const float* y, int B, int d, const void* p1, int r, const void* p2, int n_out,
                           int act, float* scores, float* part, hipStream_t s, int wdt) {
    int S, sc;
    pred_split(d, wdt, &S, &sc);
    hipLaunchKernelGGL((k_pred_hidden<T, NB>), dim3(cdiv((long)r * S, 4)), dim3(kBlock), 0, s, y, B, d,
                       (const T*)p1, r, S, sc, part);
    DV_LAUNCH_CHECK();
    constexpr int E = Vec<T>::E;
    const int rchunk = r / E;
    int lpr = 1;
    while (lpr < rchunk && lpr < kWave) lpr *= 2;
    const int rows_per_block = (kWave / lpr) * 4 * 4;
    const int r_pad = (r + 3) & ~3;
    hipLaunchKernelGGL((k_pred_scores<T, NB>), dim3(cdiv(n_out, rows_per_block)), dim3(kBlock),
                       (size_t)NB * r_pad * sizeof(float), s, part, B, S, r, act, (const T*)p2, n_out, lpr,
                       rows_per_block, scores);
    DV_LAUNCH_CHECK();
    return DV_OK;
}

dv_status launch_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                         int n_out, int wdt, int act, float* scores, float* part, hipStream_t s) {
    const int nb = nb_bucket(B);
#define DV_PRED(NB)                                                                             \
    case NB:                                                                                    \
        return wdt == DV_F16 ? predict_t<half_t, NB>(y, B, d, p1_t, r, p2_t, n_out, act, scores, part, s, wdt) \
                             : predict_t<float, NB>(y, B, d, p1_t, r, p2_t, n_out, act, scores, part, s, wdt);
    switch (nb) {
        DV_PRED(1) DV_PRED(2) DV_PRED(4) DV_PRED(8) DV_PRED(16)
    }
#undef DV_PRED
    return fail(DV_ERR_UNSUPPORTED, "batch %d", B);
}

static int rows_per_wave(long rows) {
    // enough waves to cover 256 CUs several times over before a wave takes a 2nd row
    long rw = rows / 4096;
    return (int)(rw < 1 ? 1 : rw > 8 ? 8 : rw);
}

template <typename T, int NB, bool YLDS>
static void fc1_go(const float* y, int B, int d, const void* w1, const void* b1, const int32_t* idx, int n_max,
                   const int32_t* n_dev, int N, float* a, hipStream_t s) {
    const int rw = rows_per_wave(n_max);
    const size_t lds = YLDS ? (size_t)NB * d * sizeof(float) : 0;
    hipLaunchKernelGGL((k_fc1<T, NB, YLDS>), dim3(cdiv(n_max, 4 * rw)), dim3(kBlock), lds, s, y, B, d,
                       (const T*)w1, (const T*)b1, idx, n_max, n_dev, N, rw, a);
}

dv_status launch_fc1(const float* y, int B, int d, const void* w1_t, const void* b1, int wdt,
                     const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a, hipStream_t s) {
    if (n_max == 0) return DV_OK;
    const int nb = nb_bucket(B);
    const bool lds = (size_t)nb * d * sizeof(float) <= kYLdsMax;
#define DV_FC1(NB)                                                                               \
    case NB:                                                                                     \
        if (wdt == DV_F16) {                                                                     \
            if (lds) fc1_go<half_t, NB, true>(y, B, d, w1_t, b1, idx, n_max, n_dev, N, a, s);       \
            else fc1_go<half_t, NB, false>(y, B, d, w1_t, b1, idx, n_max, n_dev, N, a, s);          \
        } else {                                                                                 \
            if (lds) fc1_go<float, NB, true>(y, B, d, w1_t, b1, idx, n_max, n_dev, N, a, s);        \
            else fc1_go<float, NB, false>(y, B, d, w1_t, b1, idx, n_max, n_dev, N, a, s);           \
        }                                                                                        \
        break;
    switch (nb) {
        DV_FC1(1) DV_FC1(2) DV_FC1(4) DV_FC1(8) DV_FC1(16)
    }
#undef DV_FC1
    DV_LAUNCH_CHECK();
    return DV_OK;
}

template <typename T, int NB, bool YLDS>
static void qkv_go(const QkvArgs& a, hipStream_t s) {
    const int rows = 3 * a.n_sel * a.dh;
    const size_t lds = YLDS ? (size_t)NB * a.d * sizeof(float) : 0;
    hipLaunchKernelGGL((k_qkv<T, NB, YLDS>), dim3(cdiv(rows, 4 * a.rw)), dim3(kBlock), lds, s, a);
}

dv_status launch_qkv(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                     const void* w, const void* bias, int wdt, float* q, const dv_kv_state* kv,
                     unsigned* counter, hipStream_t s) {
    if (n_sel == 0) return DV_OK;
    QkvArgs a;
    a.y = y; a.B = B; a.d = d; a.h = h; a.dh = d_h; a.n_sel = n_sel;
    a.rw = rows_per_wave(3L * n_sel * d_h);
    a.head_idx = head_idx; a.w = w; a.bias = bias; a.q = q;
    a.K = (half_t*)kv->k_cache; a.V = (half_t*)kv->v_cache;
    a.max_len = kv->max_len; a.pos = kv->pos;
    a.y_buf = kv->y_buf; a.valid_upto = kv->valid_upto; a.counter = counter;
    const int nb = nb_bucket(B);
    const bool lds = (size_t)nb * d * sizeof(float) <= kYLdsMax;
#define DV_QKV(NB)                                                                   \
    case NB:                                                                         \
        if (wdt == DV_F16) {                                                         \
            if (lds) qkv_go<half_t, NB, true>(a, s); else qkv_go<half_t, NB, false>(a, s); \
        } else {                                                                     \
            if (lds) qkv_go<float, NB, true>(a, s); else qkv_go<float, NB, false>(a, s);   \
        }                                                                            \
        break;
    switch (nb) {
        DV_QKV(1) DV_QKV(2) DV_QKV(4) DV_QKV(8) DV_QKV(16)
    }
#undef DV_QKV
    DV_LAUNCH_CHECK();
    return DV_OK;
}

}  // namespace dvh
