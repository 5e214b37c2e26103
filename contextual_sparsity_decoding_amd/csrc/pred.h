// Device bodies shared by the predictor kernels and by the launches that
// carry predictor work as extra workgroups (the look-ahead schedule without a
// second stream): the LayerNorm-folded row-dot and the second layers.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §4.1-4.3.
#pragma once

#include "rowdot.h"

namespace dv {

// A row-dot with the block's LayerNorm folded in (batch row 0): the
// predictor's first layer (OP = ROW_PLAIN, rows 0..n_max-1, optionally the
// rows of two predictors, the second's from a.w2) or fc1 over the selected
// rows (OP = ROW_FC1: bias, ReLU).  RR rows per wave, NT/64*RR per
// workgroup of NT threads.
// Every workgroup normalises x in LDS itself while its rows are still in
// flight (the statistics of a 5120-float row cost far less than a launch);
// workgroup 0 also writes y when ln.y_out is set.
template <typename T, int CH, int OP, int RR = 1, int NT = kBlock, bool GB = false>
__device__ __forceinline__ void rowdot_ln_block(int blk, float* ys, const RowArgs& a, const LnArgs& ln) {
    constexpr int E = Vec<T>::E;
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    const int u0 = (blk * (NT / kWave) + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))) * RR;
    const int nchunk = a.d / E;
    // The row indices first: the rows wait for them, and loads retire in
    // issue order, so behind x's DMA they would make the rows wait for x.
    int j[RR];
    int jany = -1;                                   // a valid row of this wave, re-read in place of invalid ones
#pragma unroll
    for (int r = RR - 1; r >= 0; --r) {
        const int u = u0 + r;
        int jj = -1;
        if (u < n) {
            jj = a.idx ? a.idx[u] : u;
            jj = (unsigned)jj < (unsigned)a.w_rows ? jj : -1;   // an index outside W selects nothing
        }
        j[r] = __builtin_amdgcn_readfirstlane(jj);
        if (j[r] >= 0) jany = j[r];
    }
    // x straight into LDS, ahead of the rows
    stage_dma<NT>(ys, ln.x, a.d);
    if constexpr (GB) {
        // gamma and beta too: fetched after the rows they would hold the
        // LayerNorm until the rows arrive
        stage_dma<NT>(ys + a.d, ln.g, a.d);
        stage_dma<NT>(ys + 2 * a.d, ln.b, a.d);
    }
    // fc1's bias as stored, also ahead of the rows; converted where it is
    // added (a conversion next to its load would wait for x's DMA)
    T braw[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) braw[r] = OP == ROW_FC1 ? ((const T*)a.bias)[j[r] >= 0 ? j[r] : 0] : T(0);
    issue_order_fence();
    // With several rows per wave, the first PF chunks of every row now and
    // the rest one chunk ahead of the dot products (a wave's loads go out
    // only as fast as HBM drains them; issuing them all first would leave
    // the arithmetic as a tail).  With one row per wave (10 KB at d = 5120)
    // every load goes out first: deferring any of them past the LayerNorm
    // measured slower.
    constexpr int PF = RR >= 2 && (8 / RR) < CH ? 8 / RR : CH;
    const int lane = threadIdx.x & 63;
    const T* rowp[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const int jl = j[r] >= 0 ? j[r] : (jany >= 0 ? jany : 0);
        rowp[r] = (a.w2 && jl >= a.split) ? (const T*)a.w2 + (size_t)(jl - a.split) * a.d : (const T*)a.w + (size_t)jl * a.d;
    }
    u32x4 w[RR][CH];
    auto load_chunk = [&](int i) {
        const int c = lane + i * kWave;
#pragma unroll
        for (int r = 0; r < RR; ++r) w[r][i] = ld16_stream(rowp[r] + (size_t)(c < nchunk ? c : 0) * E);
    };
    if (jany >= 0) {
#pragma unroll
        for (int i = 0; i < PF; ++i) load_chunk(i);
        sync_after_dma<RR * PF>();                   // x has landed; the rows may still be in flight
    } else {
        sync_after_dma<0>();
    }
    layernorm_lds<NT, GB>(ys, a.d, ln, blk == 0 && ln.y_out != nullptr);
    float acc[RR];
#pragma unroll
    for (int r = 0; r < RR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            float yv[E];
            const f32x4* y4 = reinterpret_cast<const f32x4*>(ys + (size_t)c * E);
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const f32x4 t = y4[q];
                yv[4 * q] = t[0]; yv[4 * q + 1] = t[1]; yv[4 * q + 2] = t[2]; yv[4 * q + 3] = t[3];
            }
#pragma unroll
            for (int r = 0; r < RR; ++r) {
                float f[E];
                unpack(w[r][i], f, T());
#pragma unroll
                for (int e = 0; e < E; ++e) acc[r] = fmaf(f[e], yv[e], acc[r]);
            }
        }
        if (i + PF < CH) {
            issue_order_fence();
            if (jany >= 0) load_chunk(i + PF);
            issue_order_fence();
        }
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
        const int u = u0 + r;
        if (u >= a.n_max) break;
        float v = wave_sum(j[r] >= 0 ? acc[r] : 0.f);
        if (OP == ROW_FC1) v = j[r] >= 0 ? fmaxf(v + to_f32(braw[r]), 0.f) : 0.f;
        if ((threadIdx.x & 63) == 0) a.out[u] = v;
    }
}

// ---------------------------------------------------------------- predictor --
// DejaVu §4.1/§4.2: SP(y) = act(y P1) P2.  Layer 1 is k_rowdot (r rows);
// layer 2 applies act to the r hidden values and scores every output row,
// lpr lanes per row of r elements.
template <typename T, int NB>
__device__ __forceinline__ void pred_scores_block(int blk, float* hid /* LDS [NB][r_pad] */,
                                                  const float* __restrict__ hid_in, int B, int r, int act,
                                                  const T* __restrict__ p2, int n_out, int lpr, int rows_per_block,
                                                  float* __restrict__ scores) {
    constexpr int E = Vec<T>::E;
    const int r_pad = (r + 3) & ~3;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int grp = lane / lpr, t = lane % lpr;
    const int rpw = kWave / lpr;                         // rows per wave pass
    const int rchunk = r / E;                            // r*wb is a multiple of 16
    const int j0 = blk * rows_per_block;
    const int j1 = min(n_out, j0 + rows_per_block);
    // the first chunk of this wave's rows in its first MAXP passes, all
    // loaded before the hidden vector is staged (one round trip, not one per
    // pass)
    constexpr int MAXP = 4;
    u32x4 pre[MAXP];
#pragma unroll
    for (int pi = 0; pi < MAXP; ++pi) {
        const int jp = j0 + wv * rpw + pi * 4 * rpw + grp;
        pre[pi] = (jp < j1 && t < rchunk) ? ld16(p2 + (size_t)jp * r + (size_t)t * E) : u32x4{0u, 0u, 0u, 0u};
    }
    for (int i = threadIdx.x; i < NB * r_pad; i += kBlock) {
        const int b = i / r_pad, k = i % r_pad;
        float v = (b < B && k < r) ? hid_in[(size_t)b * r + k] : 0.f;
        if (act == DV_ACT_RELU) v = fmaxf(v, 0.f);
        hid[i] = v;
    }
    __syncthreads();
    int pi = 0;
    for (int jb = j0 + wv * rpw; jb < j1; jb += 4 * rpw, ++pi) {
        const int j = jb + grp;
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.f;
        u32x4 w0 = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
            if (q == pi) w0 = pre[q];
        if (j < j1) {
            const T* row = p2 + (size_t)j * r;
            for (int c = t; c < rchunk; c += lpr) {
                float f[E];
                unpack((pi < MAXP && c == t) ? w0 : ld16(row + (size_t)c * E), f, T());
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

// The predictor's second layer fused with the selection for a short score
// row (n_out <= 256, e.g. heads; batch row 0): thread j scores row j of P2
// (all its r-element loads in flight at once), then ranks its key against
// the others in LDS; rank < k selects it, and a block scan writes the set
// ascending.  Same order as k_topk: score descending, ties to the lower
// index, NaN last.
template <typename T>
__device__ __forceinline__ void pred_topk_small_block(const float* __restrict__ hid_in, int r, int act,
                                                      const T* __restrict__ p2, int n_out, float* __restrict__ scores,
                                                      int k, int32_t* __restrict__ idx) {
    constexpr int E = Vec<T>::E;
    constexpr int CB = 16;                               // chunk loads in flight per batch
    __shared__ float hid[512];
    __shared__ uint32_t keys[kBlock];
    __shared__ unsigned tot[17];
    const int j = threadIdx.x;
    const int rchunk = r / E;
    for (int i = threadIdx.x; i < r; i += kBlock) {
        const float v = hid_in[i];
        hid[i] = act == DV_ACT_RELU ? fmaxf(v, 0.f) : v;
    }
    const T* row = p2 + (size_t)(j < n_out ? j : 0) * r;
    float acc = 0.f;
    for (int c0 = 0; c0 < rchunk; c0 += CB) {
        u32x4 w[CB];
#pragma unroll
        for (int c = 0; c < CB; ++c)
            w[c] = (j < n_out && c0 + c < rchunk) ? ld16(row + (size_t)(c0 + c) * E) : u32x4{0u, 0u, 0u, 0u};
        if (c0 == 0) __syncthreads();                    // hid staged
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            if (c0 + c < rchunk) {
                float f[E];
                unpack(w[c], f, T());
#pragma unroll
                for (int e = 0; e < E; ++e) acc = fmaf(f[e], hid[(c0 + c) * E + e], acc);
            }
        }
    }
    if (rchunk == 0) __syncthreads();
    const uint32_t kj = j < n_out ? order_key(acc) : 0u;
    if (j < n_out) scores[j] = acc;
    keys[j] = kj;
    __syncthreads();
    unsigned rank = 0;
    for (int i = 0; i < n_out; ++i) {
        const uint32_t ki = keys[i];
        rank += (ki > kj) || (ki == kj && i < j);
    }
    const bool sel = j < n_out && rank < (unsigned)k;
    unsigned total;
    const unsigned pos = block_excl_scan(sel ? 1u : 0u, tot, &total);
    if (sel && pos < (unsigned)k) idx[pos] = j;
}

// Both predictors' second layers as one role (batch row 0): block 0 scores
// the heads and selects k_a of them, blocks 1.. score the neuron rows.  The
// neuron selection is left to the top-k kernel.
struct Pred2Args {
    const float* hid_a;     // head predictor hidden values [r_a]
    int r_a;
    const void* p2_a;       // [h][r_a]
    int n_a;
    float* s_a;             // head scores [n_a]
    int k_a;
    int32_t* idx_a;         // selected heads [k_a], ascending
    const float* hid_m;     // neuron predictor hidden values [r_m]
    int r_m;
    const void* p2_m;       // [N][r_m]
    int n_m;
    int lpr, rows_per_block;
    float* s_m;             // neuron scores [n_m]
    unsigned* zero;         // block 0 also clears zero[0, 4096), or NULL
    int act;
    int wdt;
};

inline __host__ __device__ int pred2_blocks(const Pred2Args& a) {
    return 1 + (a.n_m + a.rows_per_block - 1) / a.rows_per_block;
}

template <typename T>
__device__ __forceinline__ void pred2_pair_block(int blk, float* hid /* LDS [r_m] */, const Pred2Args& a) {
    if (blk == 0) {
        if (a.zero)
            for (int i = threadIdx.x; i < 4096; i += kBlock) a.zero[i] = 0u;
        if (a.n_a > 0)                                  // the head predictor, when it rides
            pred_topk_small_block<T>(a.hid_a, a.r_a, a.act, (const T*)a.p2_a, a.n_a, a.s_a, a.k_a, a.idx_a);
    }
    else
        pred_scores_block<T, 1>(blk - 1, hid, a.hid_m, 1, a.r_m, a.act, (const T*)a.p2_m, a.n_m, a.lpr,
                                a.rows_per_block, a.s_m);
}

}  // namespace dv
