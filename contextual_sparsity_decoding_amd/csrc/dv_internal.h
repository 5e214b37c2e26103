// Internal declarations of libdv: device helpers and kernel launchers.
//
// Target: gfx950 (CDNA4), wave64.  Every kernel here is bandwidth-bound at
// batch 1, so the helpers are about moving bytes: 16-byte vector loads,
// rows split across the 64 lanes of a wave, fp32 accumulation and
// fixed-order (deterministic) reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dv.h"

namespace dv {

typedef _Float16 half_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;          // 4 waves per workgroup
constexpr size_t kYLdsMax = 64 * 1024;

// ---- element traits: E elements of T per 16-byte chunk --------------------
template <typename T> struct Vec;
template <> struct Vec<half_t> { static constexpr int E = 8; };
template <> struct Vec<float> { static constexpr int E = 4; };

__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[8], half_t) {
    f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[4], float) {
    f32x4 v = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }

// ---- reductions (fixed butterfly order, so results are deterministic) ------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float group_sum_dyn(float v, int G) {
    for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Dot products of one weight row (nchunk 16-byte chunks of T) with NB fp32
// vectors, by one wave.  Lane l covers chunks l, l+64, ...; U chunk loads
// are issued before any is used.  `ys` may point to LDS or global memory
// (vector b at ys + b * ystride; vectors b >= nvalid read vector 0 and
// their sums are to be discarded).  Each lane returns its partial sums.
template <typename T, int NB, int U, bool STREAM>
__device__ __forceinline__ void wave_rowdot(const T* __restrict__ row, int nchunk,
                                            const float* __restrict__ ys, int ystride, int nvalid,
                                            float (&acc)[NB]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & (kWave - 1);
    for (int base = 0; base < nchunk; base += kWave * U) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = base + lane + kWave * u;
            if (c < nchunk)
                w[u] = STREAM ? ld16_stream(row + (size_t)c * E) : ld16(row + (size_t)c * E);
            else
                w[u] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = base + lane + kWave * u;
            if (c < nchunk) {
                float f[E];
                unpack(w[u], f, T());
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int bb = b < nvalid ? b : 0;
                    const f32x4* yv = reinterpret_cast<const f32x4*>(ys + (size_t)bb * ystride + (size_t)c * E);
#pragma unroll
                    for (int q = 0; q < E / 4; ++q) {
                        const f32x4 y4 = yv[q];
                        acc[b] = fmaf(f[4 * q + 0], y4[0], acc[b]);
                        acc[b] = fmaf(f[4 * q + 1], y4[1], acc[b]);
                        acc[b] = fmaf(f[4 * q + 2], y4[2], acc[b]);
                        acc[b] = fmaf(f[4 * q + 3], y4[3], acc[b]);
                    }
                }
            }
        }
    }
}

// Order-preserving map of fp32 to uint32 for selection: larger float ->
// larger key; -0 and +0 map to the same key; NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (f != f) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum over the block (<= 1024 threads); *total gets the sum.
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* tot /* >= 17 */, unsigned* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const unsigned incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) tot[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned run = 0;
        for (int i = 0; i < nw; ++i) {
            const unsigned t = tot[i];
            tot[i] = run;
            run += t;
        }
        tot[16] = run;
    }
    __syncthreads();
    const unsigned r = tot[w] + incl - v;
    *total = tot[16];
    __syncthreads();
    return r;
}

// Load a small vector from global memory into LDS with the whole block.
__device__ __forceinline__ void block_copy_f32(float* __restrict__ dst, const float* __restrict__ src, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

}  // namespace dv

// ---- host side --------------------------------------------------------------
namespace dvh {

dv_status fail(dv_status code, const char* fmt, ...);
void clear_error();
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
int elt_bytes(int wdt);

// Every workspace starts with a fixed block of counters (zero between calls;
// the kernels that use one reset it), so calls of any shape can share one
// workspace.  Scratch buffers are carved after it.
constexpr size_t kCounterBytes = 4096;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(unsigned));
inline unsigned* ws_counters(void* ws, int i = 0) { return ws ? (unsigned*)ws + i : nullptr; }

// Workspace carving: a bump allocator over the caller's buffer.
struct Carve {
    char* base;
    size_t off = kCounterBytes;
    explicit Carve(void* p) : base((char*)p) {}
    template <typename T> T* take(size_t n) {
        off = align_up(off, 256);
        T* p = base ? (T*)(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
};

// Kernel launchers (no validation; the entry points validate first).
dv_status launch_layernorm(const float* x, int B, int d, const float* g, const float* b, float eps,
                           float* y, hipStream_t s);
size_t pred_partials(int B, int d, int r, int wdt);
dv_status launch_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                         int n_out, int wdt, int act, float* scores, float* hid_part,
                         hipStream_t s);
dv_status launch_fc1(const float* y, int B, int d, const void* w1_t, const void* b1, int wdt,
                     const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a, hipStream_t s);
struct AxpyPlan {
    int n_slices, n_groups, rows_per_group;
};
AxpyPlan axpy_plan(int d, int rows, int wdt);
size_t axpy_ws_floats(const AxpyPlan& p, int B, int d);
dv_status launch_axpy(const void* w, int wdt, int d, int w_rows, int rows, const int32_t* n_rows_dev,
                      const int32_t* idx, int blk, const float* coef, int coef_stride, bool skip_zero,
                      int B, const void* bias, const float* residual, float* out, int32_t* rows_read,
                      float* partial, int32_t* advance, hipStream_t s);
bool qkv_supported(int B, int d, int wdt);
dv_status launch_qkv(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                     const void* w, const void* bias, int wdt, float* q, const dv_kv_state* kv, bool mark_valid,
                     hipStream_t s);
bool ln_fusable(int B, int d);
dv_status launch_predict_ln(const float* x, int B, int d, const float* g, const float* b, float eps, float* y_out,
                            const void* p1_t, int r, const void* p2_t, int n_out, int wdt, int act, float* scores,
                            float* hid, hipStream_t s);
int topk_block_threads(int n);
dv_status launch_set_i32(int32_t* p, int v, hipStream_t s);
dv_status launch_topk(const float* scores, int B, int n, int k, int32_t* idx, hipStream_t s);
dv_status launch_union(const int32_t* idx, int B, int k, int n, int32_t* union_idx,
                       int32_t* union_count, hipStream_t s);
int splitk_auto(int max_positions, int rows);
dv_status launch_splitk(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel,
                        const dv_kv_view* kv, const int32_t* n_dev, int n_add, float scale, int num_splits, float* o,
                        float* part, int32_t* mark_valid, int mark_pos, const int32_t* mark_pos_dev, hipStream_t s);
dv_status launch_kv_score(const void* q_obs, int B, int h, int d_h, int n_obs, const dv_kv_view* kv,
                          float scale, int n_sink, int n_window, int width, float* scores,
                          float* raw, float* stats, hipStream_t s);
size_t kv_score_stats_floats(int B, int h, int n, int n_obs);

}  // namespace dvh
