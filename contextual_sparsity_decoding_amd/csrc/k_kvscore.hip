// Attention-scored KV selection: per-position scores for one layer.
//
// Pages: ByteCross = "Where Activation Sparsity and KV-Cache Sparsity Cross in
// LLM Decoding" (arXiv 2609.33889v1), §4.1 and App. A: cached positions are
// ranked by the attention they receive from the last 64 prompt queries
// (pooled over the query heads of a KV head; one each here), smoothed by a
// width-7 average; sinks and the observation window are forced in; the top
// positions per KV head within the budget are kept (dv_topk_select).
//
// Four launches, each bandwidth- or latency-light next to a decode step:
//   stats   per (query, split): running max and sum of exp over its causal
//           range of keys                                  (like split-K)
//   combine per query: M, L over its splits
//   prob    per position: sum over queries of 2^(s - M) / L (the queries'
//           softmax rows, added up); one K row per 16-lane group, all
//           queries from LDS
//   smooth  centred moving average, forced positions set to +inf
#include "dv_internal.h"

#include <math.h>

namespace dv {

template <int DH>
__global__ __launch_bounds__(kBlock) void k_kvs_stats(const half_t* __restrict__ qobs, const half_t* __restrict__ K,
                                                      int B, int h, int n_obs, int max_len, int n, float scale_log2,
                                                      int splits, int chunk, float* __restrict__ stats) {
    constexpr int LPR = DH / 8, RPW = kWave / LPR, U = 4;
    const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= B * h * n_obs * splits) return;
    const int c = task % splits, row = task / splits;
    const int w = row % n_obs, bh = row / n_obs;
    const int lane = threadIdx.x & 63, g = lane / LPR, t = lane % LPR;
    float qv[8];
    {
        float f[8];
        unpack(ld16(qobs + (size_t)row * DH + t * 8), f, half_t());
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = f[e] * scale_log2;
    }
    const int cnt = n - n_obs + w + 1;            // causal: keys 0 .. n - n_obs + w
    const int j0 = c * chunk, j1 = min(cnt, j0 + chunk);
    const half_t* Kh = K + (size_t)bh * max_len * DH + t * 8;
    float m = -INFINITY, l = 0.f;
    for (int jb = j0; jb < j1; jb += RPW * U) {
        u32x4 kw[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jb + u * RPW + g;
            valid[u] = j < j1;
            kw[u] = valid[u] ? ld16(Kh + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u};
        }
        float sc[U], mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[8];
            unpack(kw[u], f, half_t());
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qv[e], f[e], d);
            d = group_sum<LPR>(d);
            sc[u] = valid[u] ? d : -INFINITY;
            mx = fmaxf(mx, sc[u]);
        }
        const float mn = fmaxf(m, mx);
        if (mn == -INFINITY) continue;
        l *= exp2f(m - mn);
#pragma unroll
        for (int u = 0; u < U; ++u) l += valid[u] ? exp2f(sc[u] - mn) : 0.f;
        m = mn;
    }
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(m, off, kWave), lo = __shfl_xor(l, off, kWave);
        const float M = fmaxf(m, mo);
        if (M != -INFINITY) {
            l = l * exp2f(m - M) + lo * exp2f(mo - M);
            m = M;
        }
    }
    if (lane == 0) {
        stats[(size_t)task * 2] = m;
        stats[(size_t)task * 2 + 1] = l;
    }
}

__global__ void k_kvs_combine(const float* __restrict__ stats, int rows, int splits, float* __restrict__ ml) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= rows) return;
    const float* S = stats + (size_t)row * splits * 2;
    float M = -INFINITY;
    for (int c = 0; c < splits; ++c)
        if (S[2 * c + 1] > 0.f) M = fmaxf(M, S[2 * c]);
    float L = 0.f;
    if (M != -INFINITY)
        for (int c = 0; c < splits; ++c)
            if (S[2 * c + 1] > 0.f) L = fmaf(exp2f(S[2 * c] - M), S[2 * c + 1], L);
    ml[2 * row] = M;
    ml[2 * row + 1] = L;
}

template <int DH>
__global__ __launch_bounds__(kBlock) void k_kvs_prob(const half_t* __restrict__ qobs, const half_t* __restrict__ K,
                                                     const float* __restrict__ ml, int h, int n_obs, int max_len, int n,
                                                     float scale_log2, int tile, float* __restrict__ raw) {
    constexpr int LPR = DH / 8, RPW = kWave / LPR;
    extern __shared__ float lds[];                 // q [n_obs][DH] then (M, 1/L) [n_obs][2]
    float* qs = lds;
    float* st = lds + (size_t)n_obs * DH;
    const int bh = blockIdx.y;
    for (int i = threadIdx.x; i < n_obs * DH; i += kBlock)
        qs[i] = (float)qobs[(size_t)bh * n_obs * DH + i] * scale_log2;
    for (int i = threadIdx.x; i < n_obs; i += kBlock) {
        const float M = ml[2 * ((size_t)bh * n_obs + i)], L = ml[2 * ((size_t)bh * n_obs + i) + 1];
        st[2 * i] = M;
        st[2 * i + 1] = L > 0.f ? 1.f / L : 0.f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, g = lane / LPR, t = lane % LPR;
    const half_t* Kh = K + (size_t)bh * max_len * DH + t * 8;
    const int p0 = blockIdx.x * tile, p1 = min(n, p0 + tile);
    for (int jb = p0 + wv * RPW; jb < p1; jb += 4 * RPW) {
        const int j = jb + g;
        const bool valid = j < p1;
        float f[8];
        unpack(valid ? ld16(Kh + (size_t)j * DH) : u32x4{0u, 0u, 0u, 0u}, f, half_t());
        float acc = 0.f;
        const int wfirst = j - (n - n_obs);       // query w sees key j when j <= n - n_obs + w
        for (int w = 0; w < n_obs; ++w) {
            const float* q = qs + w * DH + t * 8;
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(q[e], f[e], d);
            d = group_sum<LPR>(d);
            if (valid && w >= wfirst) acc += exp2f(d - st[2 * w]) * st[2 * w + 1];
        }
        if (valid && t == 0) raw[(size_t)bh * n + j] = acc;
    }
}

__global__ void k_kvs_smooth(const float* __restrict__ raw, int rows, int n, int width, int n_sink, int n_window,
                             float* __restrict__ scores) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)rows * n) return;
    const int j = (int)(i % n);
    const float* r = raw + (i - j);
    float v;
    if (j < n_sink || j >= n - n_window) {
        v = INFINITY;
    } else {
        const int hw = width / 2;
        float s = 0.f;
        for (int k = max(0, j - hw); k <= min(n - 1, j + hw); ++k) s += r[k];
        v = s / (float)width;
    }
    scores[i] = v;
}

}  // namespace dv

namespace dvh {
using namespace dv;

static int kvs_splits(int n) { return cdiv(n, 256); }

size_t kv_score_stats_floats(int B, int h, int n, int n_obs) {
    const size_t rows = (size_t)B * h * n_obs;
    return rows * kvs_splits(n) * 2 + rows * 2 + (size_t)B * h * n;
}

dv_status launch_kv_score(const void* q_obs, int B, int h, int d_h, int n_obs, const dv_kv_view* kv, float scale,
                          int n_sink, int n_window, int width, float* scores, float* raw, float* stats,
                          hipStream_t s) {
    (void)raw;
    const int n = kv->n_ctx;
    const int splits = kvs_splits(n);
    const int chunk = cdiv(n, splits);
    const int rows = B * h * n_obs;
    float* st = stats;
    float* ml = st + (size_t)rows * splits * 2;
    float* rw = ml + (size_t)rows * 2;
    const float sl2 = scale * 1.4426950408889634f;
    const half_t* Q = (const half_t*)q_obs;
    const half_t* K = (const half_t*)kv->k_cache;
    const int tile = 256;
    const size_t lds = ((size_t)n_obs * d_h + 2 * n_obs) * sizeof(float);
#define DV_KVS(DH)                                                                                              \
    case DH:                                                                                                    \
        hipLaunchKernelGGL((k_kvs_stats<DH>), dim3(cdiv((long)rows * splits, 4)), dim3(kBlock), 0, s, Q, K, B, h, \
                           n_obs, kv->max_len, n, sl2, splits, chunk, st);                                      \
        hipLaunchKernelGGL(k_kvs_combine, dim3(cdiv(rows, 256)), dim3(256), 0, s, st, rows, splits, ml);        \
        hipLaunchKernelGGL((k_kvs_prob<DH>), dim3(cdiv(n, tile), B * h), dim3(kBlock), lds, s, Q, K, ml, h,       \
                           n_obs, kv->max_len, n, sl2, tile, rw);                                               \
        break;
    switch (d_h) {
        DV_KVS(32) DV_KVS(64) DV_KVS(128) DV_KVS(256)
        default:
            return fail(DV_ERR_UNSUPPORTED, "d_h %d", d_h);
    }
#undef DV_KVS
    const long total = (long)B * h * n;
    hipLaunchKernelGGL(k_kvs_smooth, dim3(cdiv(total, 256)), dim3(256), 0, s, rw, B * h, n, width, n_sink, n_window,
                       scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
