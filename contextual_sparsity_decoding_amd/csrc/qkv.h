// Sparse Q/K/V projection kernel and its launch templates (instantiated per
// weight type and batch bucket in k_qkv_*.hip).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §4.2.
#pragma once

#include "pred.h"

#include <type_traits>

namespace dv {

// ---------------------------------------------------------------- Q/K/V -----
// DejaVu §4.2: for the selected heads compute q, k, v; store k, v in the
// cache; keep y for the heads not selected; recompute a selected head's
// missing K/V from the stored inputs, reusing the weight rows already held
// in registers.  Rows are ordered [which][s][e]; workgroups take the K and
// V blocks before the Q blocks.
#ifndef DV_QKV_FLIGHT_KB
#define DV_QKV_FLIGHT_KB 8
#endif
constexpr int kQkvFlightKB = DV_QKV_FLIGHT_KB;   // weight bytes a wave keeps in flight (KB; 1 KB per row chunk)

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
    const float* ln_g;        // LNF: y = LayerNorm(input) computed in the kernel
    const float* ln_b;
    float eps;
    int qkv_blocks;           // the projection's workgroups
    int hole_blocks;          // NB == 1, HB > 0: hole helpers after them (qkv_hole_items), or 0
    int pred_blocks;          // LNF: workgroups placed first that compute `pred` rows (4*R per workgroup)
    RowArgs pred;             // the next layer's predictor layer one (look-ahead) on LN(input), or w == NULL
};

// Lane-partial dots of a wave's R register-resident rows with NV inputs at
// `in` (LDS, stride d): per accumulator the same sequence of fmaf over the
// chunks and their elements as the on-time dot products.  Within a chunk the
// R * NV accumulators advance together, element by element, so a lone wave
// has independent FMAs to issue instead of one dependent chain per
// accumulator.
template <typename T, int CH, int R, int NV>
__device__ __forceinline__ void qkv_dots(const u32x4 (&w)[R][CH], const float* in, int d, int nchunk,
                                         float (&acc)[R][NV]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[j][v] = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            float yv[NV][E];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const f32x4* y4 = reinterpret_cast<const f32x4*>(in + (size_t)v * d + (size_t)c * E);
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    const f32x4 t = y4[q];
                    yv[v][4 * q] = t[0]; yv[v][4 * q + 1] = t[1]; yv[v][4 * q + 2] = t[2]; yv[v][4 * q + 3] = t[3];
                }
            }
            float f[R][E];
#pragma unroll
            for (int j = 0; j < R; ++j) unpack(w[j][i], f[j], T());
#pragma unroll
            for (int e = 0; e < E; ++e)
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int v = 0; v < NV; ++v) acc[j][v] = fmaf(f[j][e], yv[v][e], acc[j][v]);
        }
    }
}

// Hole helpers (batch of one, n_sel <= 64): the missing positions of each
// selected head past the first FIRST (which its owner workgroups compute
// beside their on-time dot products) are cut into items of 4*R rows of one K or V
// block (R rows per wave; a row's sums do not depend on how many rows a wave
// holds) and up to NV positions.  Helper `hid` takes items hid, hid + hole_blocks,
// ...: it loads the item's weight rows again (read moments before by their
// owner) and its stored inputs, and runs the owner's instructions on the
// same values, so the entries are bit-identical to on-time ones.  The
// helpers come after every owner in the grid, so they take the CUs the
// owners leave, and the rounds run side by side instead of one after
// another in the owner.
template <typename T, int CH, int R, int FIRST, int NV>
__device__ __forceinline__ void qkv_hole_items(const QkvArgs& a, int hid, float* ys) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int pos = a.pos_dev ? *a.pos_dev : a.pos;
    if (pos < 0 || pos >= a.max_len || !a.y_buf || !a.valid_upto) return;
    const int d = a.d, dh = a.dh, nchunk = d / E;
    const int nrb = dh / (4 * R);                      // row blocks per K or V block
    // lane s: selected head s, its first missing position, its rounds of NV.
    // With at most 64 heads every head's valid position is loaded beside the
    // head list and picked by lane (one memory round trip, not two).
    int head = 0, lo0 = pos, nr = 0;
    const int vu_all = a.h <= kWave && lane < a.h ? a.valid_upto[lane] : 0;
    if (lane < a.n_sel) head = a.head_idx ? a.head_idx[lane] : lane;
    const bool hv = lane < a.n_sel && (unsigned)head < (unsigned)a.h;
    const int vu = a.h <= kWave ? __shfl(vu_all, hv ? head : 0, kWave) : (hv ? a.valid_upto[head] : 0);
    if (hv) {
        lo0 = min(max(vu + 1, 0), pos);
        const int m = pos - lo0 - FIRST;
        nr = m > 0 ? (m + NV - 1) / NV : 0;
    }
    const unsigned cnt = 2u * (unsigned)(nrb * nr);    // items of head s
    const unsigned incl = wave_incl_scan(cnt);
    const unsigned total = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
    for (unsigned it = (unsigned)hid; it < total; it += (unsigned)a.hole_blocks) {
        const int s = (int)__builtin_ctzll(__ballot(incl > it));    // the first head whose items reach past it
        const unsigned l = it - ((unsigned)__builtin_amdgcn_readlane((int)incl, s) -
                                 (unsigned)__builtin_amdgcn_readlane((int)cnt, s));
        const int hd = __builtin_amdgcn_readlane(head, s);
        const int lo = __builtin_amdgcn_readlane(lo0, s);
        const int nrs = __builtin_amdgcn_readlane(nr, s);
        const int per = nrb * nrs;                     // items of one of K, V
        const int which = 1 + (int)l / per;
        const int rb = ((int)l % per) / nrs, rnd = ((int)l % per) % nrs;
        const int p0 = lo + FIRST + rnd * NV;
        const int np = min(NV, pos - p0);
        const int e0 = rb * 4 * R + wv * R;
        const T* Wb = (const T*)a.w + ((size_t)(which * a.h + hd) * dh + e0) * d;
        __syncthreads();                               // the previous item's inputs are consumed
        stage_dma(ys, a.y_buf + (size_t)p0 * d, np * d);
        T braw[R];                                     // the bias ahead of the rows (loads retire in issue order)
#pragma unroll
        for (int j = 0; j < R; ++j) braw[j] = ((const T*)a.bias)[(size_t)(which * a.h + hd) * dh + e0 + j];
        issue_order_fence();
        u32x4 w[R][CH];
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int c = lane + i * kWave;
                w[j][i] = ld16_stream(Wb + (size_t)j * d + (size_t)(c < nchunk ? c : 0) * E);
            }
        sync_after_dma<R * CH>();                      // the inputs have landed; the rows may still be in flight
        float bv[R];
#pragma unroll
        for (int j = 0; j < R; ++j) bv[j] = to_f32(braw[j]);
        float acc[R][NV];
        qkv_dots<T, CH, R, NV>(w, ys, d, nchunk, acc);
        half_t* cache = which == 1 ? a.K : a.V;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float hv = wave_sum(acc[j][v]) + bv[j];
                if (lane == 0 && v < np) cache[((size_t)hd * a.max_len + p0 + v) * dh + e0 + j] = (half_t)hv;
            }
    }
}

// Rows per wave of a hole helper's item: half the owner's, so an item
// reloads and computes half as much and twice as many run side by side.
constexpr int qkv_hole_rows(int r) { return r >= 2 ? r / 2 : 1; }

// Rows per wave of the predictor workgroups riding in the launch: one with
// split rows, so that they need no more registers than the projection's.
constexpr int qkv_pred_rows(int r, int split) { return split == 2 ? 1 : r; }

// A workgroup owns 4*R consecutive rows of one (which, head) block; wave wv
// holds rows wv*R .. wv*R+R-1 in registers (lane l: chunks l, l+64, ...), so
// every input chunk read from LDS serves R rows.  The inputs are y (NB
// batch rows) and, for K and V of batch row 0, the stored inputs of the
// head's missing positions, staged HB at a time by the whole workgroup.
// Inputs reach LDS by DMA (no registers), issued before the weight loads.
// Recomputed entries take the same instructions on the same input values as
// the entries computed on time, so they are bit-identical to them.  When y
// does not fit in LDS (YL false: wide batches) it is read from global memory.
// With LNF (batch of one) the input is the residual stream x and every
// workgroup applies the block's LayerNorm in LDS while its weight rows are
// still in flight.
//
// SPLIT = 2 (no LDS staging of stored inputs, HB = 0): a row's chunks are
// shared by a pair of waves, each holding CH/2 of them for its R rows, so a
// workgroup owns 2*R rows and a wave half the registers.  Each wave's dot
// products cover its half; the pair adds the halves in a fixed order
// (first + second) through LDS, on time and for recomputed positions alike.
template <typename T, int NB, int CH, int R, int HB, bool YL, bool LNF, int SPLIT = 1>
__global__ __launch_bounds__(kBlock) void k_qkv(QkvArgs a) {
    static_assert(SPLIT == 1 || (SPLIT == 2 && HB == 0 && CH % 2 == 0), "split rows: even chunk count, no staged holes");
    constexpr int E = Vec<T>::E;
    constexpr int HV = HB > 0 ? HB : 1;
    constexpr int CHW = CH / SPLIT;                    // chunks of a row held by one wave
    constexpr int RG = 4 / SPLIT;                      // row groups (of R rows) per workgroup
    extern __shared__ float ys[];                      // y [NB][d], then [HB][d] stored inputs
    __shared__ float pair_part[SPLIT == 2 ? RG * R * NB : 1];   // the second halves' sums
    int qb = blockIdx.x;                               // this workgroup among the projection's
    if constexpr (LNF) {
        if (qb < a.pred_blocks) {                      // look-ahead: the next layer's predictor rows, same LN1(x)
            const LnArgs ln{a.y, a.ln_g, a.ln_b, a.eps, nullptr};
            rowdot_ln_block<T, CH, ROW_PLAIN, qkv_pred_rows(R, SPLIT)>(qb, ys, a.pred, ln);
            return;
        }
        qb -= a.pred_blocks;
    }
    if constexpr (NB == 1 && HB > 0 && YL) {
        if (qb >= a.qkv_blocks) {                      // a hole helper
            // the owner computes the first HB missing positions; items of HB
            // positions measured best of 1, 2 and 3
            qkv_hole_items<T, CH, qkv_hole_rows(R), HB, HB>(a, qb - a.qkv_blocks, ys);
            return;
        }
    }
    const int d = a.d, dh = a.dh;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int grp = SPLIT == 2 ? wv >> 1 : wv;        // this wave's row group
    const int half = SPLIT == 2 ? wv & 1 : 0;         // and its share of the chunks
    const int cbase = half * CHW;                      // first chunk index of the share
    const int r0 = qb * RG * R;                        // RG*R divides dh: one head block per workgroup
    // the K and V blocks (which may carry missing positions) are dispatched
    // first and the Q blocks last, so cheap uniform blocks fill the tail
    const int which = (r0 / (a.n_sel * dh) + 1) % 3;
    const int s = (r0 / dh) % a.n_sel;
    const int e0 = r0 % dh + grp * R;                  // this wave's first row in the block
    const int nchunk = d / E;
    const int head = a.head_idx ? a.head_idx[s] : s;
    const bool live = (unsigned)head < (unsigned)a.h;
    const int pos = a.pos_dev ? *a.pos_dev : a.pos;
    const bool pos_ok = pos >= 0 && pos < a.max_len;   // else the call writes nothing
    const bool fill = pos_ok && live && a.y_buf != nullptr && a.valid_upto != nullptr && which > 0;
    const int lo0 = fill ? min(max(a.valid_upto[head] + 1, 0), pos) : pos;
    float* hin = ys + (YL ? NB : 0) * d;               // stored inputs of missing positions
    // inputs straight into LDS first (y, then the first round of stored
    // inputs), then the weight rows, all in flight together
    if (YL) stage_dma(ys, a.y, a.B * d);
    if (HB > 0 && fill && pos > lo0) stage_dma(hin, a.y_buf + (size_t)lo0 * d, min(HB, pos - lo0) * d);
    // LNF: the LayerNorm's gamma and beta into registers behind the inputs
    // and ahead of the weight rows, so the LayerNorm waits for the inputs
    // only (their registers are free again before most rows are loaded)
    constexpr int GBN = LNF ? (CH * kWave * E / 4 + kBlock - 1) / kBlock : 1;
    f32x4 gr[GBN], br[GBN];
    if constexpr (LNF) ln_gamma_beta_regs<kBlock, GBN>(LnArgs{a.y, a.ln_g, a.ln_b, a.eps, nullptr}, d, gr, br);
    // the bias as stored, also ahead of the rows; converted where it is
    // added (a conversion next to its load would wait for every load
    // issued before it, the rows included)
    T braw[R];
#pragma unroll
    for (int j = 0; j < R; ++j) braw[j] = ((const T*)a.bias)[(size_t)(which * a.h + (live ? head : 0)) * dh + e0 + j];
    const T* Wb = (const T*)a.w + ((size_t)(which * a.h + (live ? head : 0)) * dh + e0) * d;
    issue_order_fence();
    // Chunk-major, the order the dot products consume them in.  Only the
    // first PF chunks are issued here; the on-time dot products issue chunk
    // i + PF after consuming chunk i.  A wave cannot issue loads faster than
    // HBM drains them, so issuing all of them first would leave every dot
    // product for after the last byte arrives.  Every workgroup issues all
    // R * CH loads (chunks past the row re-read chunk 0 and are never used:
    // the dot products stop at the row's end).
    constexpr int PF = (kQkvFlightKB / R) < CHW ? kQkvFlightKB / R : CHW;   // kQkvFlightKB of rows in flight per wave
    u32x4 w[R][CHW];
    auto load_chunk = [&](int i) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int c = lane + (cbase + i) * kWave;
            w[j][i] = ld16_stream(Wb + (size_t)j * d + (size_t)(c < nchunk ? c : 0) * E);
        }
    };
    // Every workgroup loads its rows, one whose head is outside W those of
    // head 0 (it stores nothing): with a single path the compiler's wait
    // for gamma, beta and the bias leaves these rows in flight (merged with
    // a path without them it would wait for every load).
#pragma unroll
    for (int i = 0; i < PF; ++i) load_chunk(i);
    sync_after_dma<R * PF>();                          // the inputs have landed; the rows may still be in flight
    float bv[R];                                       // loaded before the rows: here they have landed
#pragma unroll
    for (int j = 0; j < R; ++j) bv[j] = live ? to_f32(braw[j]) : 0.f;
    if constexpr (LNF) layernorm_lds_reg<kBlock, GBN>(ys, d, a.eps, gr, br);
    // this step's input joins the stored inputs: float4 c of [B][d] goes
    // with thread c of the grid (a handful of workgroups), from LDS when staged
    if (a.y_buf && pos_ok) {
        for (int c = qb * kBlock + threadIdx.x; c < a.B * d / 4; c += a.qkv_blocks * kBlock) {
            const int b = (c * 4) / d, col = (c * 4) % d;
            const f32x4 v = (YL || LNF) ? reinterpret_cast<const f32x4*>(ys)[c] : reinterpret_cast<const f32x4*>(a.y)[c];
            *reinterpret_cast<f32x4*>(a.y_buf + ((size_t)b * a.max_len + pos) * d + col) = v;
        }
    }

    // lane-partial dots of the R rows with NV inputs at `in` (stride d),
    // over this wave's share of the chunks
    auto dots = [&](const float* in, auto nv_tag, float (&acc)[R][decltype(nv_tag)::value]) {
        qkv_dots<T, CHW, R, decltype(nv_tag)::value>(w, in + (size_t)cbase * kWave * E, d, nchunk - cbase * kWave, acc);
    };

    // Whole-row sums of R * NV wave-reduced values: with split rows the
    // second wave of each pair hands its sums to the first, which adds them
    // after its own; the result is valid in the first wave of the pair.
    auto pair_add = [&](auto nv_tag, float (&v)[R][decltype(nv_tag)::value]) {
        constexpr int NV = decltype(nv_tag)::value;
        if constexpr (SPLIT == 2) {
            static_assert(NV <= NB, "pair buffer holds NB values per row");
            if (half == 1 && lane == 0) {
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int u = 0; u < NV; ++u) pair_part[(grp * R + j) * NB + u] = v[j][u];
            }
            __syncthreads();
            if (half == 0) {
#pragma unroll
                for (int j = 0; j < R; ++j)
#pragma unroll
                    for (int u = 0; u < NV; ++u) v[j][u] = v[j][u] + pair_part[(grp * R + j) * NB + u];
            }
            __syncthreads();                           // read before the next round's writes
        }
    };

    // The weight registers are marked as rewritten after each use, so the
    // compiler converts fp16 to fp32 again for every input instead of
    // keeping all converted rows live (which would cost occupancy).
    auto fence_w = [&]() {
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int i = 0; i < CHW; ++i) asm volatile("" : "+v"(w[j][i]));
    };

    // ---- on-time q, k, v (same instructions per input as `dots`, so the
    // recomputed entries below stay bit-identical).  The first round of
    // missing positions rides along: its stored inputs were staged with y,
    // and the VALU would otherwise wait on the rows.
    const bool hole1 = HB > 0 && fill && pos > lo0;    // uniform over the workgroup
    float hacc1[R][HV];
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
        for (int v = 0; v < HV; ++v) hacc1[j][v] = 0.f;
    {
        float acc[R][NB];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[j][b] = 0.f;
        const float* yin = YL ? ys : a.y;
#pragma unroll
        for (int i = 0; i < CHW; ++i) {
            const int c = lane + (cbase + i) * kWave;
            if (c < nchunk) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float yv[E];
                    const f32x4* y4 = reinterpret_cast<const f32x4*>(yin + (size_t)b * d + (size_t)c * E);
#pragma unroll
                    for (int q = 0; q < E / 4; ++q) {
                        const f32x4 t = y4[q];
                        yv[4 * q] = t[0]; yv[4 * q + 1] = t[1]; yv[4 * q + 2] = t[2]; yv[4 * q + 3] = t[3];
                    }
#pragma unroll
                    for (int j = 0; j < R; ++j) {
                        float f[E];
                        unpack(w[j][i], f, T());
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[j][b] = fmaf(f[e], yv[e], acc[j][b]);
                    }
                }
                if constexpr (HB > 0) {
                    if (hole1) {
#pragma unroll
                        for (int v = 0; v < HV; ++v) {
                            float yv[E];
                            const f32x4* y4 = reinterpret_cast<const f32x4*>(hin + (size_t)v * d + (size_t)c * E);
#pragma unroll
                            for (int q = 0; q < E / 4; ++q) {
                                const f32x4 t = y4[q];
                                yv[4 * q] = t[0]; yv[4 * q + 1] = t[1]; yv[4 * q + 2] = t[2]; yv[4 * q + 3] = t[3];
                            }
#pragma unroll
                            for (int j = 0; j < R; ++j) {
                                float f[E];
                                unpack(w[j][i], f, T());
#pragma unroll
                                for (int e = 0; e < E; ++e) hacc1[j][v] = fmaf(f[e], yv[e], hacc1[j][v]);
                            }
                        }
                    }
                }
            }
            if (i + PF < CHW) {
                issue_order_fence();                     // the next loads go out after this chunk's work
                load_chunk(i + PF);
                issue_order_fence();
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[j][b] = wave_sum(acc[j][b]);
        pair_add(std::integral_constant<int, NB>(), acc);
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[j][b] += bv[j];
        if (live && pos_ok && lane == 0 && half == 0) {
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b >= a.B) continue;
                    if (which == 0) a.q[((size_t)b * a.n_sel + s) * dh + e0 + j] = acc[j][b];
                    else (which == 1 ? a.K : a.V)[(((size_t)b * a.h + head) * a.max_len + pos) * dh + e0 + j] =
                        (half_t)acc[j][b];
                }
        }
    }
    if (which == 0 || !fill) return;                   // uniform over the workgroup
    fence_w();

    // ---- missing positions of batch row 0: the first HB were staged up
    // front beside y; later rounds take HB2 at a time, y's slots included
    half_t* cache = which == 1 ? a.K : a.V;
    if constexpr (HB > 0) {
        constexpr int HB2 = HB + (YL ? NB : 0);
        auto round = [&](const float* in, int p0, int cnt, auto nv_tag) {
            constexpr int NV = decltype(nv_tag)::value;
            float hacc[R][NV];
            dots(in, nv_tag, hacc);
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const float hv = wave_sum(hacc[j][v]) + bv[j];
                    if (lane == 0 && v < cnt) cache[((size_t)head * a.max_len + p0 + v) * dh + e0 + j] = (half_t)hv;
                }
            fence_w();
        };
        {   // the first round, computed beside the on-time dot products
            const int cnt = min(HB, pos - lo0);
#pragma unroll
            for (int j = 0; j < R; ++j)
#pragma unroll
                for (int v = 0; v < HV; ++v) {
                    const float hv = wave_sum(hacc1[j][v]) + bv[j];
                    if (lane == 0 && v < cnt) cache[((size_t)head * a.max_len + lo0 + v) * dh + e0 + j] = (half_t)hv;
                }
        }
        const int p_end = a.hole_blocks > 0 ? lo0 + HB : pos;   // else the hole helpers take the rest
        for (int p0 = lo0 + HB; p0 < p_end; p0 += HB2) {
            const int cnt = min(HB2, p_end - p0);
            __syncthreads();                           // the previous round's inputs (and y) are consumed
            stage_dma(ys, a.y_buf + (size_t)p0 * d, cnt * d);
            wait_dma_and_sync();
            round(ys, p0, cnt, std::integral_constant<int, HB2>());
        }
    } else {
        // one stored input at a time: with y in LDS (batch of one) it is
        // staged there by DMA, y being consumed (one round trip, no
        // registers), else read from global memory
        for (int p = lo0; p < pos; ++p) {
            const float* in = a.y_buf + (size_t)p * d;
            if constexpr (YL && NB == 1) {
                __syncthreads();                       // every wave has consumed y (or the previous input)
                stage_dma(ys, in, d);
                wait_dma_and_sync();
                in = ys;
            }
            float hacc[R][1];
            dots(in, std::integral_constant<int, 1>(), hacc);
#pragma unroll
            for (int j = 0; j < R; ++j) hacc[j][0] = wave_sum(hacc[j][0]);
            pair_add(std::integral_constant<int, 1>(), hacc);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float hv = hacc[j][0] + bv[j];
                if (lane == 0 && half == 0) cache[((size_t)head * a.max_len + p) * dh + e0 + j] = (half_t)hv;
            }
            fence_w();
        }
    }
    // batch rows past the first keep their own valid positions (read from global memory)
    for (int b = 1; b < a.B; ++b) {
        const int lo = min(max(a.valid_upto[b * a.h + head] + 1, 0), pos);
        for (int p = lo; p < pos; ++p) {
            float hacc[R][1];
            dots(a.y_buf + ((size_t)b * a.max_len + p) * d, std::integral_constant<int, 1>(), hacc);
#pragma unroll
            for (int j = 0; j < R; ++j) hacc[j][0] = wave_sum(hacc[j][0]);
            pair_add(std::integral_constant<int, 1>(), hacc);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float hv = hacc[j][0] + bv[j];
                if (lane == 0 && half == 0) cache[(((size_t)b * a.h + head) * a.max_len + p) * dh + e0 + j] = (half_t)hv;
            }
            fence_w();
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

// Rows per wave held in registers: as many as fit in 40 chunk registers.
inline int qkv_rows_per_wave(int ch) { return ch <= 10 ? 4 : ch <= 20 ? 2 : 1; }

template <typename T, int NB, int CH, int R>
static dv_status qkv_go3(const QkvArgs& a_in, hipStream_t s) {
    QkvArgs a = a_in;
    const int rows = 3 * a.n_sel * a.dh;
    const size_t row = (size_t)a.d * sizeof(float);
    const bool holes = a.y_buf && a.valid_upto;
    const size_t yl = NB * row <= kQkvLdsMax ? NB * row : 0;   // y in LDS, else read from global memory
    // batch of one with inputs in LDS: one hole helper per K/V block of
    // 4 * qkv_hole_rows(R) rows (more items are taken in turn)
    const int hb = holes && yl + 2 * row <= kQkvLdsMax ? 2 : holes && yl + row <= kQkvLdsMax ? 1 : 0;
    // without staged stored inputs, rows are split over wave pairs, where a
    // wave holds at least two rows (with one, a workgroup would own two rows
    // and stage all of y for them)
    constexpr bool kSplitOk = CH % 2 == 0 && R >= 2;
    const bool split = kSplitOk && hb == 0;
    const int wg_rows = (split ? 2 : 4) * R;
    if (a.dh % wg_rows) return fail(DV_ERR_UNSUPPORTED, "Q/K/V projection: d_h=%d", a.dh);
    a.qkv_blocks = rows / wg_rows;
    a.pred_blocks = a.pred.w ? cdiv(a.pred.n_max, 4 * qkv_pred_rows(R, split ? 2 : 1)) : 0;
    a.hole_blocks = NB == 1 && a.B == 1 && yl && hb > 0 && a.n_sel <= kWave ? 2 * a.n_sel * (a.dh / (4 * qkv_hole_rows(R))) : 0;
    const int grid = a.pred_blocks + a.qkv_blocks + a.hole_blocks;
    const bool lnf = a.ln_g != nullptr;
    if (lnf && (NB != 1 || !yl)) return fail(DV_ERR_UNSUPPORTED, "Q/K/V with LayerNorm: B=%d d=%d", a.B, a.d);
    if (a.pred.w && (!lnf || a.pred.d != a.d)) return fail(DV_ERR_UNSUPPORTED, "predictor rows need the LayerNorm-folded Q/K/V");
#define DV_QKV(HB, LDS, SP)                                                                                          \
    do {                                                                                                             \
        if constexpr (NB == 1) {                                                                                     \
            if (lnf) {                                                                                               \
                DV_LAUNCH((k_qkv<T, NB, CH, R, HB, true, true, SP>), dim3(grid), dim3(kBlock), LDS, s, a);           \
                break;                                                                                               \
            }                                                                                                        \
        }                                                                                                            \
        if (yl) DV_LAUNCH((k_qkv<T, NB, CH, R, HB, true, false, SP>), dim3(grid), dim3(kBlock), LDS, s, a);          \
        else DV_LAUNCH((k_qkv<T, NB, CH, R, HB, false, false, SP>), dim3(grid), dim3(kBlock), LDS - yl, s, a);     \
    } while (0)
    if (hb == 2) DV_QKV(2, yl + 2 * row, 1);
    else if (hb == 1) DV_QKV(1, yl + row, 1);
    else if constexpr (kSplitOk) DV_QKV(0, yl, 2);
    else DV_QKV(0, yl, 1);
#undef DV_QKV
    return DV_OK;
}

// One (weight type, batch bucket) per translation unit: the instantiations
// are spread over several sources so that they compile in parallel.
template <typename T, int NB>
dv_status qkv_go(const QkvArgs& a, int ch, hipStream_t s) {
    switch (ch) {
        case 4: return qkv_go3<T, NB, 4, 4>(a, s);
        case 8: return qkv_go3<T, NB, 8, 4>(a, s);
        case 10: return qkv_go3<T, NB, 10, 4>(a, s);
        case 12: return qkv_go3<T, NB, 12, 2>(a, s);
        case 16: return qkv_go3<T, NB, 16, 2>(a, s);
        case 18: return qkv_go3<T, NB, 18, 2>(a, s);
        case 24: return qkv_go3<T, NB, 24, 1>(a, s);
        default: return fail(DV_ERR_UNSUPPORTED, "Q/K/V projection: rows of d=%d are too long", a.d);
    }
}

#define DV_QKV_EXTERN(T, NB) extern template dv_status qkv_go<T, NB>(const QkvArgs&, int, hipStream_t);
DV_QKV_EXTERN(half_t, 1) DV_QKV_EXTERN(half_t, 2) DV_QKV_EXTERN(half_t, 4) DV_QKV_EXTERN(half_t, 8)
DV_QKV_EXTERN(half_t, 16) DV_QKV_EXTERN(float, 1) DV_QKV_EXTERN(float, 2) DV_QKV_EXTERN(float, 4)
DV_QKV_EXTERN(float, 8) DV_QKV_EXTERN(float, 16)
#undef DV_QKV_EXTERN

}  // namespace dvh
