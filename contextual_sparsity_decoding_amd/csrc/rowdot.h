// Device helpers shared by the row-dot kernels (LayerNorm, predictor, fc1,
// Q/K/V): staging inputs in LDS, whole weight rows in registers, dot
// products of a register-resident row, and the chunk tiers.
#pragma once

#include "dv_internal.h"

#include <math.h>

namespace dv {

// ---------------------------------------------------------------- LayerNorm --
// DejaVu App. B: a normalisation precedes each block of the residual stream.
// One 1024-thread workgroup per row; the row stays in registers (float4
// loads, all issued together), two block reductions, one store.
constexpr int kLnThreads = 1024;
constexpr int kLnVec = 4;                 // float4 per thread: d <= 16384

// A workgroup barrier for LDS traffic only: this wave's LDS operations have
// completed, then s_barrier.  Unlike __syncthreads it does not wait for
// outstanding global loads, so weight rows stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));   // lgkmcnt(0), vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ float block_sum1024(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i];
    return s;
}

// Sum over a workgroup of NW waves (red: NW floats of LDS).
template <int NW>
__device__ __forceinline__ float block_sum_waves(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    lds_barrier();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += red[i];
    return s;
}

__device__ __forceinline__ float block_sum256(float v, float* red) { return block_sum_waves<4>(v, red); }

// LayerNorm of one row held in LDS, in place: population variance, then
// gamma and beta (DejaVu App. B: a norm precedes each block).  Every thread
// of the NT-thread workgroup takes part; ends with a barrier.  With `write`,
// the normalised row is also stored to ln.y_out.
struct LnArgs {
    const float* x;
    const float* g;
    const float* b;
    float eps;
    float* y_out;
};

// Mean and 1/sqrt(var + eps) of the row held in LDS (two passes, float4
// reads, four independent partial sums per thread).
template <int NT = kBlock>
__device__ __forceinline__ void ln_stats_lds(const float* __restrict__ ys, int d, float eps, float* mean_out,
                                             float* rstd_out) {
    __shared__ float red[NT / kWave];
    const f32x4* x4 = reinterpret_cast<const f32x4*>(ys);
    f32x4 s4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = threadIdx.x; c < d / 4; c += NT) s4 += x4[c];
    const float mean = block_sum_waves<NT / kWave>((s4[0] + s4[1]) + (s4[2] + s4[3]), red) / (float)d;
    f32x4 q4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = threadIdx.x; c < d / 4; c += NT) {
        const f32x4 t = x4[c] - mean;
#pragma unroll
        for (int e = 0; e < 4; ++e) q4[e] = fmaf(t[e], t[e], q4[e]);
    }
    *rstd_out = 1.0f / sqrtf(block_sum_waves<NT / kWave>((q4[0] + q4[1]) + (q4[2] + q4[3]), red) / (float)d + eps);
    *mean_out = mean;
}

template <int NT = kBlock, bool GB = false>
__device__ __forceinline__ void layernorm_lds(float* __restrict__ ys, int d, const LnArgs& ln, bool write) {
    float mean, rstd;
    ln_stats_lds<NT>(ys, d, ln.eps, &mean, &rstd);
    // gamma and beta: staged in LDS after the row (GB), else from memory
    const f32x4* g4 = reinterpret_cast<const f32x4*>(GB ? ys + d : ln.g);
    const f32x4* b4 = reinterpret_cast<const f32x4*>(GB ? ys + 2 * d : ln.b);
    f32x4* y4 = reinterpret_cast<f32x4*>(ys);
#pragma unroll 8
    for (int c = threadIdx.x; c < d / 4; c += NT) {
        const f32x4 gg = g4[c], bb = b4[c];
        f32x4 v = y4[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (v[e] - mean) * rstd * gg[e] + bb[e];
        y4[c] = v;
        if (write) reinterpret_cast<f32x4*>(ln.y_out)[c] = v;
    }
    lds_barrier();
}

// Gamma and beta for layernorm_lds_reg: float4 c = threadIdx.x + k * NT of
// each, k < GBN, loaded into registers.  Issued before a kernel's weight
// loads, they return ahead of them (vector loads retire in issue order), so
// the LayerNorm does not wait for the weights in flight.
template <int NT, int GBN>
__device__ __forceinline__ void ln_gamma_beta_regs(const LnArgs& ln, int d, f32x4 (&gr)[GBN], f32x4 (&br)[GBN]) {
    const f32x4* g4 = reinterpret_cast<const f32x4*>(ln.g);
    const f32x4* b4 = reinterpret_cast<const f32x4*>(ln.b);
#pragma unroll
    for (int k = 0; k < GBN; ++k) {
        const int c = threadIdx.x + k * NT;
        gr[k] = c < d / 4 ? g4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
        br[k] = c < d / 4 ? b4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// layernorm_lds (without the y_out copy) with gamma and beta already in
// registers; the same arithmetic per element.  d <= 4 * NT * GBN.
template <int NT, int GBN>
__device__ __forceinline__ void layernorm_lds_reg(float* __restrict__ ys, int d, float eps, const f32x4 (&gr)[GBN],
                                                  const f32x4 (&br)[GBN]) {
    float mean, rstd;
    ln_stats_lds<NT>(ys, d, eps, &mean, &rstd);
    f32x4* y4 = reinterpret_cast<f32x4*>(ys);
#pragma unroll
    for (int k = 0; k < GBN; ++k) {
        const int c = threadIdx.x + k * NT;
        if (c < d / 4) {
            const f32x4 gg = gr[k], bb = br[k];
            f32x4 v = y4[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (v[e] - mean) * rstd * gg[e] + bb[e];
            y4[c] = v;
        }
    }
    lds_barrier();
}

// Wait until at most N vector-memory operations of this wave are still
// outstanding (loads retire in issue order, so everything issued before the
// last N has completed).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Keeps the compiler from moving memory operations across this point (the
// input DMA must be issued before the weight loads that a partial vmcnt
// wait leaves in flight).
__device__ __forceinline__ void issue_order_fence() { asm volatile("" ::: "memory"); }

// After an input DMA followed by N weight loads per wave: the DMA has landed
// in every wave's share of LDS, the weights may still be in flight.
template <int N>
__device__ __forceinline__ void sync_after_dma() {
    wait_vmcnt<N>();
    lds_barrier();
}

// ---------------------------------------------------------------- staging ---
// Copy NB rows of length d (d % 4 == 0, 16-byte aligned) from global memory
// into LDS; rows b >= B are zero.  Each thread issues its first MAXV float4
// loads before the first LDS store.
template <int NB, int MAXV>
__device__ __forceinline__ void stage_rows(float* __restrict__ lds, const float* __restrict__ src, int B, int d) {
    const int n4 = NB * d / 4;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
    f32x4 v[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c = threadIdx.x + i * kBlock;
        v[i] = (c < n4 && (c * 4) / d < B) ? s4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    f32x4* l4 = reinterpret_cast<f32x4*>(lds);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
        const int c = threadIdx.x + i * kBlock;
        if (c < n4) l4[c] = v[i];
    }
    for (int c = threadIdx.x + MAXV * kBlock; c < n4; c += kBlock)   // inputs longer than MAXV*1024 floats
        l4[c] = (c * 4) / d < B ? s4[c] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Copy n floats (n % 4 == 0, 16-byte aligned source) from global memory
// straight into LDS (gfx950 LDS DMA: lane l of a wave fills bytes
// [16 l, 16 l + 16) of the wave's 1 KB block), with no registers in
// between.  The data is there once the issuing wave's vmcnt has drained;
// callers wait for vmcnt(0) and then synchronise the workgroup.
typedef __attribute__((address_space(3))) void lds_void_t;
template <int NT = kBlock>
__device__ __forceinline__ void stage_dma(float* lds, const float* __restrict__ src, int n) {
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nkb = (n + 255) / 256;
    for (int c = wv; c < nkb; c += NT / kWave) {
        const int i = c * 256 + lane * 4;
        if (i < n) __builtin_amdgcn_global_load_lds(src + i, (lds_void_t*)(lds + c * 256), 16, 0, 0);
    }
}
__device__ __forceinline__ void wait_dma_and_sync() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

// One wave's whole weight row in registers: chunks lane, lane+64, ... of
// nchunk (at most CH per lane).
template <typename T, int CH, bool STREAM>
__device__ __forceinline__ void load_row(const T* __restrict__ row, int nchunk, u32x4 (&w)[CH]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk)
            w[i] = STREAM ? ld16_stream(row + (size_t)c * E) : ld16(row + (size_t)c * E);
        else
            w[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

// As load_row, but every one of the CH loads is issued (chunks past the row
// re-read chunk 0; dot_row never uses them), so a wave has exactly CH loads
// in flight.
template <typename T, int CH>
__device__ __forceinline__ void load_row_all(const T* __restrict__ row, int nchunk, u32x4 (&w)[CH]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        w[i] = ld16_stream(row + (size_t)(c < nchunk ? c : 0) * E);
    }
}

// Lane-partial dots of a register-resident row with NB vectors (LDS or
// global, vector b at ys + b * ystride).
template <typename T, int CH, int NB>
__device__ __forceinline__ void dot_row(const u32x4 (&w)[CH], int nchunk, const float* __restrict__ ys, int ystride,
                                        int nvalid, float (&acc)[NB]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            float f[E];
            unpack(w[i], f, T());
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int bb = b < nvalid ? b : 0;     // vectors past the batch are discarded
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

// ---------------------------------------------------------------- row-dot ---
// out[b][u] = epilogue(W[row(u)] . y[b]) for u in [0, n): the predictor's
// first layer (its activation is applied by the next kernel) and sparse fc1
// (bias + ReLU).
enum RowOp { ROW_PLAIN = 0, ROW_FC1 = 1 };

struct RowArgs {
    const float* y;
    int B, d;
    const void* w;
    const void* bias;       // per row (FC1)
    const int32_t* idx;     // row(u) = idx[u], or u
    int n_max;
    const int32_t* n_dev;   // count used, <= n_max, or NULL
    int w_rows;             // rows of W (bounds of idx)
    float* out;             // [B][n_max]
    const void* w2;         // rows j >= split come from w2 (row j - split), or NULL
    int split;
};


// The layer input normalised in LDS (used by the predictor with LN folded in).
}  // namespace dv

namespace dvh {
using namespace dv;

inline int nb_bucket(int B) { return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16; }

// Chunks per lane held in registers: the smallest tier covering a row.
inline int ch_tier(int d, int wdt) {
    const int E = 16 / elt_bytes(wdt);
    const int per_lane = cdiv(d / E, kWave);
    if (per_lane <= 4) return 4;
    if (per_lane <= 8) return 8;
    if (per_lane <= 10) return 10;            // d = 5120 in fp16
    if (per_lane <= 12) return 12;
    if (per_lane <= 16) return 16;
    if (per_lane <= 18) return 18;            // d = 9216 in fp16
    if (per_lane <= 24) return 24;
    return 0;                                 // too long: generic path
}

// Rows per workgroup for the streaming kernels: a multiple of 4, about
// two workgroups per CU (256 CUs) when there are enough rows, at most 32.
inline int rows_per_group(long rows) {
    long r = (rows + 2047) / 2048;              // 512 workgroups of 4 * r rows
    r = r < 1 ? 1 : r > 8 ? 8 : r;
    return (int)(4 * r);
}


}  // namespace dvh
