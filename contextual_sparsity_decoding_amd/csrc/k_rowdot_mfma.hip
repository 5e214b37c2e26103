// Batched row-dot products on the matrix cores: for a batch of 8-16 decode
// rows (or 4-7 whose inputs are too wide for LDS) every fp16 weight row meets
// 4-16 inputs, so sparse fc1 over the
// batch's union of neurons (DejaVu §5.2 / App. C.1) and the Q/K/V
// projections become a skinny dense contraction
//     out[b][u] = sum_k y[b][k] * W[row(u)][k]        (b < B <= 16)
// that the vector ALUs cannot keep up with at HBM speed (16 FMAs per weight
// element; rocprof shows the VALU paths reading y again for every row).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §2.3 Eq. 1-2 (the products), §5.2
// and App. C.1 (the batch runs over the union of its sets).
//
// v_mfma_f32_16x16x32_f16: A = 16 x 32 (batch x k), B = 32 x 16 (k x rows),
// fp32 accumulate.  Lane l supplies A row l % 16 and B column l % 16, both
// at k = 8 (l / 16) .. +7, so its B operand is 16 contiguous bytes of one
// weight row: a wave's load covers 64 bytes of each of 16 rows.  The fp32
// inputs are split into fp16 hi + lo (hi = fp16(y), lo = fp16(y - hi)) and
// both go through the matrix core, so the inputs keep about 22 bits.
//
// A wave owns RT tiles of 16 rows over one of KS ranges of k; its partial
// sums go to a [KS][16][n_max] buffer and a second launch adds the ranges in
// order and applies the epilogue (fc1: bias and ReLU; Q/K/V: bias, q in
// fp32 and K/V into the cache in fp16).
#include "rowdot.h"

namespace dv {

typedef _Float16 f16x8m __attribute__((ext_vector_type(8)));

constexpr int kMfmaRT = 4;          // 16-row tiles per wave
constexpr int kMfmaPF = 4;          // k-steps of weight loads in flight
constexpr int kMfmaMaxKS = 16;

struct MfmaArgs {
    const float* y;           // [B][d]
    int B, d;
    const half_t* w;          // rows of d
    int w_rows;
    // fc1: row(u) = idx[u] (or u); Q/K/V: u = (which * n_sel + s) * dh + e,
    // row = (which * h + head(s)) * dh + e
    const int32_t* idx;
    int qkv, n_sel, dh, h;
    const int32_t* head_idx;
    int n_max;
    const int32_t* n_dev;
    int ks, steps_per_split;  // k ranges and their length in 32-element steps
    int short_ranges;         // few rows: k ranges of kMfmaSPSShort steps (up to kMfmaMaxKSShort of them)
    float* part;              // [ks][16][n_max]
};

__device__ __forceinline__ int mfma_row(const MfmaArgs& a, int u, int n) {
    if (u >= n) return -1;
    int j;
    if (a.qkv) {
        const int which = u / (a.n_sel * a.dh), s = (u / a.dh) % a.n_sel, e = u % a.dh;
        const int head = a.head_idx ? a.head_idx[s] : s;
        if ((unsigned)head >= (unsigned)a.h) return -1;
        j = (which * a.h + head) * a.dh + e;
    } else {
        j = a.idx ? a.idx[u] : u;
    }
    return (unsigned)j < (unsigned)a.w_rows ? j : -1;
}

__global__ __launch_bounds__(kBlock) void k_rowdot_mfma(MfmaArgs a) {
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    const int tile = wid / a.ks, ksi = wid % a.ks;
    const int u0 = tile * 16 * kMfmaRT;
    if (u0 >= n) return;                                   // whole wave idle
    const int nsteps = a.d / 32;
    const int st0 = ksi * a.steps_per_split, st1 = min(nsteps, st0 + a.steps_per_split);
    const int col = lane & 15, kq = lane >> 4;             // B column / A row, k block of 8
    const half_t* rowp[kMfmaRT];
    bool rv[kMfmaRT];
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) {
        const int j = mfma_row(a, u0 + 16 * t + col, n);
        rv[t] = j >= 0;
        rowp[t] = a.w + (size_t)(j >= 0 ? j : 0) * a.d + 8 * kq;
    }
    const bool yrow = col < a.B;                           // A row = batch row
    const float* yp = a.y + (size_t)(yrow ? col : 0) * a.d + 8 * kq;
    f32x4 acc[kMfmaRT];
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 wr[kMfmaPF][kMfmaRT];
    auto load_w = [&](int st, int slot) {
#pragma unroll
        for (int t = 0; t < kMfmaRT; ++t)
            wr[slot][t] = (st < st1 && rv[t]) ? ld16_stream(rowp[t] + (size_t)st * 32) : u32x4{0u, 0u, 0u, 0u};
    };
#pragma unroll
    for (int p = 0; p < kMfmaPF; ++p) load_w(st0 + p, p);
    for (int st = st0; st < st1; st += kMfmaPF) {
#pragma unroll
        for (int p = 0; p < kMfmaPF; ++p) {
            const int s = st + p;
            if (s < st1) {                                 // uniform over the wave
                f32x4 y0 = f32x4{0.f, 0.f, 0.f, 0.f}, y1 = y0;
                if (yrow) {
                    y0 = *reinterpret_cast<const f32x4*>(yp + (size_t)s * 32);
                    y1 = *reinterpret_cast<const f32x4*>(yp + (size_t)s * 32 + 4);
                }
                f16x8m hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hi[e] = (half_t)y0[e];
                    hi[4 + e] = (half_t)y1[e];
                    lo[e] = (half_t)(y0[e] - (float)hi[e]);
                    lo[4 + e] = (half_t)(y1[e] - (float)hi[4 + e]);
                }
#pragma unroll
                for (int t = 0; t < kMfmaRT; ++t) {
                    const f16x8m wb = __builtin_bit_cast(f16x8m, wr[p][t]);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, wb, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, wb, acc[t], 0, 0, 0);
                }
                load_w(s + kMfmaPF, p);                    // the slot just consumed takes step s + PF
            }
        }
    }
    // D: lane l, register i = row (batch) 4 (l / 16) + i, column (tile row) l % 16
    float* P = a.part + (size_t)ksi * 16 * a.n_max;
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) {
        const int u = u0 + 16 * t + col;
        if (u < a.n_max) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = 4 * kq + i;
                if (b < a.B) P[(size_t)b * a.n_max + u] = acc[t][i];
            }
        }
    }
}

// The same contraction by workgroups whose 4 waves share one k range of SPS
// steps (the last range of a row may be shorter), each wave taking 4 tiles,
// so that a workgroup covers 256 rows.  The range's inputs go into LDS once
// per workgroup by DMA, ahead of the weight loads (at a batch of 16 the
// per-wave input loads from L2 cost as much time as a third of the weight
// loads); a row of them is padded by 16 bytes so that the 16 batch rows'
// reads of one step fall on different banks.  The loop is unrolled in full:
// with no loop the compiler's waits count the loads of each slot exactly.
// The weight loads are unmasked and unconditional (a masked load, or a
// value merged with a default, makes the next use wait for every load): a
// row not selected reads row 0, masked where used; a step past the range
// reads the range's last step again, never used.  They are plain loads:
// with the streaming hint the two 64-byte halves of a line, read a few
// instructions apart, were each fetched from HBM as a whole line (1.7x the
// bytes).
template <int SPS>
__global__ __launch_bounds__(kBlock) void k_rowdot_mfma_u(MfmaArgs a) {
    constexpr int YS = SPS * 32 + 4;                      // floats per staged input row
    __shared__ __align__(16) float yl[16 * YS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ksi = blockIdx.x % a.ks, rb = blockIdx.x / a.ks;
    const int u0 = (rb * (kBlock / kWave) + wv) * 16 * kMfmaRT;
    const int nsteps = a.d / 32;
    const int st0 = ksi * SPS, st1 = min(nsteps, st0 + SPS);
    const int col = lane & 15, kq = lane >> 4;             // B column / A row, k block of 8
    // a tile's weights are loaded 4 lanes to a row (lane l: row l / 4, k
    // block l % 4), so that consecutive lanes read consecutive bytes, and
    // moved into the operand layout (row l % 16, k block l / 16) by a lane
    // permute at use; loading in the operand layout measured 3% slower
    const int lrow = lane >> 2, lkb = lane & 3;
    int key[kMfmaRT], raw[kMfmaRT];
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) {
        const int u = u0 + 16 * t + lrow, uc = u < a.n_max ? u : a.n_max - 1;
        key[t] = a.qkv ? (uc / a.dh) % a.n_sel : uc;
    }
    const int32_t* src = a.qkv ? a.head_idx : a.idx;
    if (src) {
#pragma unroll
        for (int t = 0; t < kMfmaRT; ++t) raw[t] = src[key[t]];
    } else {
#pragma unroll
        for (int t = 0; t < kMfmaRT; ++t) raw[t] = key[t];
    }
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    if (rb * (kBlock / kWave) * 16 * kMfmaRT >= n) return;   // the whole workgroup idle
    const half_t* rowp[kMfmaRT];
    bool rv[kMfmaRT];
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) {
        const int u = u0 + 16 * t + lrow;
        int j = -1;
        if (u < n) {
            if (a.qkv) {
                const int which = u / (a.n_sel * a.dh), e = u % a.dh, head = raw[t];
                if ((unsigned)head < (unsigned)a.h) j = (which * a.h + head) * a.dh + e;
            } else {
                j = raw[t];
            }
            if ((unsigned)j >= (unsigned)a.w_rows) j = -1;   // an index outside W selects nothing
        }
        rv[t] = j >= 0;
        rowp[t] = a.w + (size_t)(j >= 0 ? j : 0) * a.d + 8 * lkb;
    }
    // the rows are resolved (their index loads waited for); then the inputs
    // and the weights go out back to back
    {   // the range's inputs, 1 KB a wave-instruction, a fixed count per wave
        // and unconditional (a branch around one makes the compiler wait for
        // every load): a row past the batch copies row 0 and k past a short
        // range the range's last 4 inputs, neither ever used
        constexpr int NKB = SPS * 32 / 256;
        static_assert(SPS * 32 % 256 == 0 && 16 * NKB % (kBlock / kWave) == 0, "whole chunks per wave");
        const int nk = (st1 - st0) * 32;
        const int wu = __builtin_amdgcn_readfirstlane(wv);
#pragma unroll
        for (int r = 0; r < 16 * NKB / (kBlock / kWave); ++r) {
            const int c = r * (kBlock / kWave) + wu, b = c / NKB, kc = c % NKB, e = min(kc * 256 + lane * 4, nk - 4);
            __builtin_amdgcn_global_load_lds(a.y + (size_t)(b < a.B ? b : 0) * a.d + st0 * 32 + e,
                                             (lds_void_t*)(yl + b * YS + kc * 256), 16, 0, 0);
        }
    }
    asm volatile("" ::: "memory");
    f32x4 acc[kMfmaRT];
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 wr[kMfmaPF][kMfmaRT];
    auto load_w = [&](int st, int slot) {
        const size_t sc = (size_t)(st < st1 ? st : st1 - 1) * 32;
#pragma unroll
        for (int t = 0; t < kMfmaRT; ++t) wr[slot][t] = ld16(rowp[t] + sc);
    };
#pragma unroll
    for (int p = 0; p < kMfmaPF; ++p) {                   // in slot order (the first slot's loads first)
        load_w(st0 + p, p);
        asm volatile("" ::: "memory");
    }
    sync_after_dma<kMfmaPF * kMfmaRT>();                   // the inputs have landed; the weights may be in flight
    if (u0 >= n) return;                                   // this wave idle (uniform)
    const bool yrow = col < a.B;                           // A row = batch row
    const float* yrw = yl + col * YS + 8 * kq;
#pragma unroll
    for (int i = 0; i < SPS; ++i) {
        constexpr int PFc = kMfmaPF;
        const int p = i % PFc;
        if (st0 + i < st1) {                               // uniform over the wave
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
            const f32x4 y0 = yrow ? *reinterpret_cast<const f32x4*>(yrw + i * 32) : zero;
            const f32x4 y1 = yrow ? *reinterpret_cast<const f32x4*>(yrw + i * 32 + 4) : zero;
            f16x8m hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hi[e] = (half_t)y0[e];
                hi[4 + e] = (half_t)y1[e];
                lo[e] = (half_t)(y0[e] - (float)hi[e]);
                lo[4 + e] = (half_t)(y1[e] - (float)hi[4 + e]);
            }
#pragma unroll
            for (int t = 0; t < kMfmaRT; ++t) {
                u32x4 wq = rv[t] ? wr[p][t] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) wq[e] = (unsigned)__builtin_amdgcn_ds_bpermute((4 * col + kq) * 4, (int)wq[e]);
                const f16x8m wb = __builtin_bit_cast(f16x8m, wq);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, wb, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo, wb, acc[t], 0, 0, 0);
            }
        }
        if (i + PFc < SPS) {                               // the slot just consumed takes step i + PF
            asm volatile("" ::: "memory");
            load_w(st0 + i + PFc, p);
            asm volatile("" ::: "memory");
        }
    }
    float* P = a.part + (size_t)ksi * 16 * a.n_max;
#pragma unroll
    for (int t = 0; t < kMfmaRT; ++t) {
        const int u = u0 + 16 * t + col;
        if (u < a.n_max) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = 4 * kq + i;
                if (b < a.B) P[(size_t)b * a.n_max + u] = acc[t][i];
            }
        }
    }
}

struct MfmaEpi {
    const float* part;
    int ks, B, n_max;
    const int32_t* n_dev;
    const void* bias;         // or NULL
    int relu;
    // fc1 and plain rows: out[b][n_max] = sum + bias[row], its ReLU when
    // asked; Q/K/V: q and the cache
    float* out;
    half_t* K;
    half_t* V;
    int max_len, pos;
    const int32_t* pos_dev;
};

__global__ __launch_bounds__(kBlock) void k_rowdot_mfma_epi(MfmaArgs a, MfmaEpi e) {
    const int n = e.n_dev ? min(*e.n_dev, e.n_max) : e.n_max;
    const int i = blockIdx.x * kBlock + threadIdx.x;       // (b, u)
    if (i >= e.B * e.n_max) return;
    const int b = i / e.n_max, u = i % e.n_max;
    if (u >= n) return;
    // up to 16 ranges' loads in flight, then their sum in order
    auto add16 = [&](int k0, float v) {
        float pv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            pv[k] = k0 + k < e.ks ? e.part[((size_t)(k0 + k) * 16 + b) * e.n_max + u] : 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) v += pv[k];
        return v;
    };
    float v = add16(0, 0.f);
    for (int k0 = 16; k0 < e.ks; k0 += 16) v = add16(k0, v);   // short ranges of few rows
    const int j = mfma_row(a, u, n);
    const half_t* bias = (const half_t*)e.bias;
    if (!a.qkv) {
        if (j >= 0 && bias) v += (float)bias[j];
        e.out[(size_t)b * e.n_max + u] = j < 0 ? 0.f : e.relu ? fmaxf(v, 0.f) : v;
        return;
    }
    if (j < 0) return;
    v += (float)bias[j];
    const int which = u / (a.n_sel * a.dh), s = (u / a.dh) % a.n_sel, el = u % a.dh;
    if (which == 0) {
        e.out[((size_t)b * a.n_sel + s) * a.dh + el] = v;
        return;
    }
    const int pos = e.pos_dev ? *e.pos_dev : e.pos;
    if (pos < 0 || pos >= e.max_len) return;
    const int head = a.head_idx ? a.head_idx[s] : s;
    (which == 1 ? e.K : e.V)[(((size_t)b * a.h + head) * e.max_len + pos) * a.dh + el] = (half_t)v;
}

}  // namespace dv

namespace dvh {
using namespace dv;

// Batches of 8-16, and batches of 2-7 whose inputs do not fit in LDS (the
// vector paths would read them from global memory for every row; the
// matrix cores take them as a padded 16-row operand).  OPT-175B width, 8
// layers over a union of neurons: batch 2 3.66 -> 3.27 ms per step with
// this and the matrix-core gather-AXPY, batch 4 4.25 -> 3.91.
bool rowdot_mfma_ok(int B, int d, int wdt) {
    const bool wide = B >= 2 && (size_t)B * d * sizeof(float) > kYLdsMax;
    return (B >= 8 || wide) && B <= 16 && wdt == DV_F16 && d % 32 == 0;
}

size_t rowdot_mfma_part_floats(int n_max) { return (size_t)kMfmaMaxKS * 16 * (n_max > 0 ? n_max : 1); }

constexpr int kMfmaSPS = 24;       // k steps per workgroup in the unrolled kernel (d <= 32 * 24 * kMfmaMaxKS)

constexpr int kMfmaSPSShort = 8;   // rows of at most 256 (a predictor's second layer), or few rows

static bool mfma_unrolled(const MfmaArgs& a) { return a.d / 32 <= kMfmaSPS * kMfmaMaxKS; }
static int mfma_sps(int d) { return d / 32 <= kMfmaSPSShort ? kMfmaSPSShort : kMfmaSPS; }

constexpr int kMfmaMaxKSShort = 64;

static void mfma_split(MfmaArgs& a) {
    const int nsteps = a.d / 32;
    if (mfma_unrolled(a)) {
        a.steps_per_split = mfma_sps(a.d);
        a.ks = cdiv(nsteps, a.steps_per_split);
        // a launch of fewer than 128 workgroups (a predictor's 128 rows) takes
        // short k ranges instead: each wave's chain of loads is a third as long
        const int wgs = cdiv(a.n_max > 0 ? a.n_max : 1, 16 * kMfmaRT * (kBlock / kWave)) * a.ks;
        if (a.short_ranges && wgs < 128 && cdiv(nsteps, kMfmaSPSShort) <= kMfmaMaxKSShort) {
            a.steps_per_split = kMfmaSPSShort;
            a.ks = cdiv(nsteps, kMfmaSPSShort);
        }
        return;
    }
    const int tiles = cdiv(a.n_max > 0 ? a.n_max : 1, 16 * kMfmaRT);
    int ks = cdiv(4096, tiles);                            // about 4096 waves in all
    ks = ks < 1 ? 1 : ks > kMfmaMaxKS ? kMfmaMaxKS : ks;
    if (ks > nsteps) ks = nsteps;
    a.steps_per_split = cdiv(nsteps, ks);
    a.ks = cdiv(nsteps, a.steps_per_split);
}

static dv_status mfma_go(MfmaArgs& a, MfmaEpi& e, hipStream_t s) {
    if (a.n_max == 0) return DV_OK;
    mfma_split(a);
    e.part = a.part; e.ks = a.ks; e.B = a.B; e.n_max = a.n_max; e.n_dev = a.n_dev;
    const int waves = cdiv(a.n_max, 16 * kMfmaRT) * a.ks;
    const dim3 ug(cdiv(a.n_max, 16 * kMfmaRT * (kBlock / kWave)) * a.ks);   // 256 rows x one k range a workgroup
    if (mfma_unrolled(a) && a.steps_per_split == kMfmaSPSShort)
        hipLaunchKernelGGL(k_rowdot_mfma_u<kMfmaSPSShort>, ug, dim3(kBlock), 0, s, a);
    else if (mfma_unrolled(a))
        hipLaunchKernelGGL(k_rowdot_mfma_u<kMfmaSPS>, ug, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL(k_rowdot_mfma, dim3(cdiv(waves, kBlock / kWave)), dim3(kBlock), 0, s, a);
    hipLaunchKernelGGL(k_rowdot_mfma_epi, dim3(cdiv((long)a.B * a.n_max, kBlock)), dim3(kBlock), 0, s, a, e);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(err));
    return DV_OK;
}

dv_status launch_fc1_mfma(const float* y, int B, int d, const void* w1_t, const void* b1, const int32_t* idx,
                          int n_max, const int32_t* n_dev, int N, float* a_out, float* part, hipStream_t s) {
    MfmaArgs a{};
    a.y = y; a.B = B; a.d = d; a.w = (const half_t*)w1_t; a.w_rows = N; a.idx = idx; a.qkv = 0;
    a.n_max = n_max; a.n_dev = n_dev; a.part = part;
    MfmaEpi e{};
    e.bias = b1; e.relu = 1; e.out = a_out;
    return mfma_go(a, e, s);
}

dv_status launch_qkv_mfma(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                          const void* w, const void* bias, float* q, const dv_kv_state* kv, float* part,
                          hipStream_t s) {
    MfmaArgs a{};
    a.y = y; a.B = B; a.d = d; a.w = (const half_t*)w; a.w_rows = 3 * h * d_h; a.qkv = 1; a.n_sel = n_sel;
    a.dh = d_h; a.h = h; a.head_idx = head_idx; a.n_max = 3 * n_sel * d_h; a.n_dev = nullptr; a.part = part;
    MfmaEpi e{};
    e.bias = bias; e.out = q; e.K = (half_t*)kv->k_cache; e.V = (half_t*)kv->v_cache; e.max_len = kv->max_len;
    e.pos = kv->pos; e.pos_dev = kv->pos_dev;
    return mfma_go(a, e, s);
}

size_t rowdot_mfma_rows_part_floats(int n_rows, int d) {
    MfmaArgs a{};
    a.d = d; a.n_max = n_rows > 0 ? n_rows : 1; a.short_ranges = 1;
    mfma_split(a);
    return (size_t)a.ks * 16 * a.n_max;
}

dv_status launch_rows_mfma(const float* y, int B, int d, const void* w, int n_rows, bool relu, float* out, float* part,
                           hipStream_t s) {
    MfmaArgs a{};
    a.y = y; a.B = B; a.d = d; a.w = (const half_t*)w; a.w_rows = n_rows; a.qkv = 0; a.n_max = n_rows; a.part = part;
    a.short_ranges = 1;
    MfmaEpi e{};
    e.relu = relu ? 1 : 0; e.out = out;
    return mfma_go(a, e, s);
}

}  // namespace dvh
