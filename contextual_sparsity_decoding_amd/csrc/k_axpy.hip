// Gather-AXPY: out[b] = residual[b] + bias + sum_u coef[b][u] * W[row(u)]
// for the second MLP layer (DejaVu Eq. 1, rows of W2^T) and the output
// projection (DejaVu Eq. 2, rows of W^O, d_h per selected head).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157); §4.4 stores W2 and W^O transposed so a
// selected neuron or head is a contiguous run of rows.
//
// Work split: the d output columns are cut into slices of one wave-load
// (64 lanes x 16 bytes); the selected rows into groups of 64.  A workgroup
// (4 waves) takes one (slice, group): it resolves its rows, issues all 64
// row loads at once (16 per wave), obtains the coefficients meanwhile, then
// accumulates, reduces its 4 waves in LDS and writes one partial sum.
//
// Coefficients come either from memory (compacted in order, dropping rows
// whose coefficients are all zero when asked) or, for the output projection
// of a decode layer, straight from the split-K attention partials: the
// workgroup merges a head's splits (running max, rescaled sums) for its own
// rows, so no separate combine pass runs.
//
// Batches of 2-16 run on the matrix cores instead (k_axpy_mfma): at 16
// FMAs per weight element the vector ALUs fall far behind HBM, and a partial
// of B x d floats per 64 rows would cost as many bytes as the weights, so a
// workgroup there covers 256 rows (at a batch of 2-4 the partials alone
// made the vector kernel slower).
//
// k_axpy_finalize then adds the partials in a fixed order, plus bias and
// residual, over the groups that hold live rows only (a device-side row count
// may leave the last groups empty; they write nothing).  Results do not
// depend on scheduling.
//
// In a look-ahead decode layer (DejaVu §4.3) these launches also carry the
// next layer's neuron selection (topk_split.h): one more column of
// workgroups, each taking 1024 scores, histograms their top key bits in the
// output projection; one more workgroup of its finalize finds the
// threshold; one more column emits the selected indices in the second MLP
// layer, while the other workgroups stream rows.
#include "topk_split.h"

#include <math.h>

namespace dv {

constexpr int kRowsPerGroup = 64;
constexpr int kAxpyU = kRowsPerGroup / 4;    // row loads per wave

struct AxpyArgs {
    const void* w;
    int d, w_rows, rows;      // W has w_rows rows of d; rows = selected rows (u)
    const int32_t* n_rows_dev;
    const int32_t* idx;       // row(u) = idx[u / blk] * blk + u % blk, or u when NULL
    int blk;
    const float* coef;        // coef[b * coef_stride + u]
    int coef_stride;
    int skip_zero;
    int thresh;               // coefficients of magnitude <= thr count as zero (threshold sparsity)
    float thr;
    const float* apart;       // attention partials [B][rows / blk][num_splits][blk + 2], or NULL
    int num_splits;
    int B, n_groups;
    float* partial;           // [n_groups][B][d], or [parts][B][d]
    int32_t* rows_read;
    // NB == 1, tk_s set: the last column of workgroups runs a selection
    // role over scores tk_s[0, tk_n), 1024 per workgroup: ATTN stores their
    // order keys in tk_keys and histograms them into tk_hist, otherwise
    // emits the indices of the keys above tk_thr into tk_idx
    const float* tk_s;
    uint32_t* tk_keys;
    int tk_n, tk_k;
    unsigned* tk_hist;
    const TopkThreshold* tk_thr;
    int32_t* tk_idx;
};

// Coefficient of row u = s * dh + e for batch row b: the attention output
// o[b][s][e] = sum_c 2^(m_c - M) acc_c[e] / sum_c 2^(m_c - M) l_c over the
// splits c with l_c > 0 (log2-domain partials).  Wave q merges its quarter
// of the splits with a running maximum per batch row; the quarters are
// merged in order.  A round of loads takes CB splits of every batch row
// (one round trip for all of them, not one per batch row).
// after_loads() runs once per wave, right after the first round of partial
// loads is issued (every lane loads; lanes past the live rows or batch rows
// read row 0 and discard it), so loads issued there queue behind these.
template <int NB, typename AfterLoads>
__device__ __forceinline__ void attn_coef(const AxpyArgs& a, int r0, int nlive, float* s_cf,
                                          float (*s_q)[kRowsPerGroup][NB][3], AfterLoads&& after_loads) {
    // splits per batch row in one round: 20 for one batch row (up to 80
    // splits a round), else about 12 of each kind of value per round (the
    // round's values are all in registers at once)
    constexpr int CB = NB == 1 ? 20 : (12 / NB > 0 ? 12 / NB : 1);
    const int t = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int dh = a.blk, ns = a.num_splits;
    const int n_sel = a.rows / dh;
    const bool ok = t < nlive;
    const int u = r0 + (ok ? t : 0);
    const int s = u / dh, e = u % dh;
    const int per = (ns + 3) / 4;
    const int c0 = q * per, c1 = min(ns, c0 + per);
    const size_t bstride = (size_t)n_sel * ns * (dh + 2);       // one batch row of partials
    const float* P0 = a.apart + ((size_t)s * ns) * (dh + 2);
    float m[NB], l[NB], num[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        m[b] = -INFINITY;
        l[b] = 0.f;
        num[b] = 0.f;
    }
    bool issued = false;
    for (int cb = c0; cb < c1; cb += CB) {             // uniform over the wave
        float mc[NB][CB], lc[NB][CB], ac[NB][CB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                const bool in = cb + i < c1;
                const float* pc = P0 + (size_t)(b < a.B ? b : 0) * bstride + (size_t)(in ? cb + i : c0) * (dh + 2);
                mc[b][i] = pc[dh];
                lc[b][i] = in ? pc[dh + 1] : 0.f;
                ac[b][i] = pc[e];
            }
        if (!issued) {
            issued = true;
            asm volatile("" ::: "memory");
            after_loads();
            asm volatile("" ::: "memory");
        }
        if (!ok) continue;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (b >= a.B) continue;
#pragma unroll
            for (int i = 0; i < CB; ++i) {
                if (!(lc[b][i] > 0.f)) continue;
                const float M = fmaxf(m[b], mc[b][i]);
                const float sa = exp2f(m[b] - M), sb = exp2f(mc[b][i] - M);
                num[b] = num[b] * sa + ac[b][i] * sb;
                l[b] = l[b] * sa + lc[b][i] * sb;
                m[b] = M;
            }
        }
    }
    if (!issued) {                                     // a wave without splits
        issued = true;
        after_loads();
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        s_q[q][t][b][0] = m[b];
        s_q[q][t][b][1] = l[b];
        s_q[q][t][b][2] = num[b];
    }
    __syncthreads();
    if (threadIdx.x < kRowsPerGroup) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float m = -INFINITY, l = 0.f, num = 0.f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float mq = s_q[qq][t][b][0], lq = s_q[qq][t][b][1], nq = s_q[qq][t][b][2];
                if (!(lq > 0.f)) continue;
                const float M = fmaxf(m, mq);
                const float sa = exp2f(m - M), sb = exp2f(mq - M);
                num = num * sa + nq * sb;
                l = l * sa + lq * sb;
                m = M;
            }
            s_cf[t * NB + b] = l > 0.f ? num / l : 0.f;
        }
    }
}

// This group's rows (and coefficients read from memory), in order, into
// s_row / s_cf; returns the live rows.  The output projection uses every
// selected row (an index outside W reads nothing: row -1); the second MLP
// layer compacts the rows, dropping those whose coefficients are all zero
// when asked.  Ends with a barrier.
template <int NB, bool ATTN>
__device__ __forceinline__ int axpy_group_rows(const AxpyArgs& a, int slice, int r0, int rows, int* s_row, float* s_cf,
                                               unsigned* tot) {
    int nlive = 0;
    if (ATTN) {
        // every selected row is used; an index outside W reads nothing
        nlive = max(0, min(kRowsPerGroup, rows - r0));
        if (threadIdx.x < kRowsPerGroup) {
            const int u = r0 + threadIdx.x;
            int row = -1;
            if ((int)threadIdx.x < nlive) {
                const int hb = a.idx ? a.idx[u / a.blk] : u / a.blk;
                if ((unsigned)hb < (unsigned)(a.w_rows / a.blk)) row = hb * a.blk + u % a.blk;
            }
            s_row[threadIdx.x] = row;
        }
    } else {
        bool live = false;
        int row = 0;
        float cf[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) cf[b] = 0.f;
        if (threadIdx.x < kRowsPerGroup && r0 + (int)threadIdx.x < rows) {
            const int u = r0 + threadIdx.x;
            row = a.idx ? a.idx[u / a.blk] * a.blk + u % a.blk : u;
            bool any = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                cf[b] = b < a.B ? a.coef[(size_t)b * a.coef_stride + u] : 0.f;
                if (a.thresh) cf[b] = fabsf(cf[b]) > a.thr ? cf[b] : 0.f;
                any |= cf[b] != 0.f;
            }
            live = (unsigned)row < (unsigned)a.w_rows && (any || !a.skip_zero);   // an index outside W selects nothing
        }
        // the group's rows are wave 0's lanes: a wave scan compacts them, and
        // the count reaches the other waves through LDS across the barrier
        static_assert(kRowsPerGroup == kWave, "one row per lane of wave 0");
        if (threadIdx.x < kWave) {
            const unsigned lv = live ? 1u : 0u;
            const unsigned incl = wave_incl_scan(lv);
            const unsigned nl = (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
            if (live) {
                const unsigned slot = incl - lv;
                s_row[slot] = row;
#pragma unroll
                for (int b = 0; b < NB; ++b) s_cf[slot * NB + b] = cf[b];
            }
            if (threadIdx.x == 0) {
                tot[0] = nl;
                if (a.rows_read && slice == 0 && nl > 0) atomicAdd(a.rows_read, (int)nl);
            }
        }
    }
    __syncthreads();
    if (!ATTN) nlive = (int)tot[0];
    return nlive;
}

template <typename T, int NB, bool ATTN>
__global__ __launch_bounds__(kBlock) void k_axpy(AxpyArgs a) {
    constexpr int E = Vec<T>::E;
    constexpr int SW = kWave * E;                  // columns per slice
    constexpr int NBC = NB < 4 ? NB : 4;           // batch rows per LDS reduction round
    constexpr int NQ = ATTN ? NB : 1;
    constexpr int RED = 3 * NBC * SW, QF = ATTN ? 4 * kRowsPerGroup * NQ * 3 : 0;
    __shared__ int s_row[kRowsPerGroup];
    __shared__ float s_cf[kRowsPerGroup * NB];
    __shared__ float shbuf[RED > QF ? RED : QF];   // split merging, then the wave reduction
    __shared__ unsigned tot[20];
    auto red = reinterpret_cast<float (*)[NBC][SW]>(shbuf);
    auto s_q = reinterpret_cast<float (*)[kRowsPerGroup][NQ][3]>(shbuf);
    const T* W = (const T*)a.w;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, g = blockIdx.y;
    if constexpr (NB == 1) {
        static_assert(kBlock == 256, "a selection slice takes one 256-thread workgroup");
        if (a.tk_s && slice == (int)gridDim.x - 1) {   // the extra column
            if (g * kTopkSlice < a.tk_n) {
                if constexpr (ATTN) {
                    __shared__ unsigned tk_lds[4096];
                    topk_hist_slice(a.tk_s, a.tk_n, g, tk_lds, a.tk_hist, a.tk_keys);
                } else {
                    topk_emit_slice(a.tk_keys, a.tk_n, a.tk_k, g, a.tk_thr, tot, a.tk_idx);
                }
            }
            return;
        }
    }
    if (g >= a.n_groups) return;                   // the extra column may be taller than the groups
    const int col = slice * SW + lane * E;
    const bool colok = col < a.d;
    const int rows = a.n_rows_dev ? min(*a.n_rows_dev, a.rows) : a.rows;
    const int r0 = g * kRowsPerGroup;
    if (r0 >= rows) return;                        // past the live rows: the finalize stops before this group

    // ---- this group's rows (and coefficients read from memory), in order
    const int nlive = axpy_group_rows<NB, ATTN>(a, slice, r0, rows, s_row, s_cf, tot);

    // ---- this wave's rows wv, wv + 4, ...: for the output projection the
    // first PF go out right behind the split-K partials' loads (which are
    // L2-resident and return first), each later one after the FMAs of the
    // row PF before it (a wave's loads go out only as fast as HBM drains
    // them; issuing them all first would leave the FMAs as a tail).  fc2,
    // with its coefficients already in LDS, measured faster with every row
    // issued first.
    constexpr int kAxpyPF = ATTN ? 8 : kAxpyU;
    u32x4 w[kAxpyU];
    auto load_row = [&](int t) {
        const int k = wv + 4 * t;
        const int rr = k < nlive ? s_row[k] : -1;
        w[t] = (rr >= 0 && colok) ? ld16_stream(W + (size_t)rr * a.d + col) : u32x4{0u, 0u, 0u, 0u};
    };
    auto first_rows = [&]() {
#pragma unroll
        for (int t = 0; t < kAxpyPF; ++t) load_row(t);
    };
    if (ATTN) {
        attn_coef<NQ>(a, r0, nlive, s_cf, s_q, first_rows);
        __syncthreads();
    } else {
        first_rows();
    }

    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;
#pragma unroll
    for (int t = 0; t < kAxpyU; ++t) {
        const int k = wv + 4 * t;
        if (k < nlive) {
            float f[E];
            unpack(w[t], f, T());
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float c = s_cf[k * NB + b];
#pragma unroll
                for (int e = 0; e < E; ++e) acc[b][e] = fmaf(c, f[e], acc[b][e]);
            }
        }
        if (t + kAxpyPF < kAxpyU) {
            asm volatile("" ::: "memory");
            load_row(t + kAxpyPF);
            asm volatile("" ::: "memory");
        }
    }

    // ---- reduce the 4 waves into wave 0, NBC batch rows at a time; wave 0
    // writes the group's partial
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += NBC) {
        if (wv > 0) {
#pragma unroll
            for (int bb = 0; bb < NBC; ++bb)
#pragma unroll
                for (int e = 0; e < E; ++e) red[wv - 1][bb][lane * E + e] = acc[b0 + bb][e];
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int bb = 0; bb < NBC; ++bb) {
                const int b = b0 + bb;
                if (b < a.B && colok) {
                    float o[E];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        o[e] = acc[b][e] + red[0][bb][lane * E + e] + red[1][bb][lane * E + e] + red[2][bb][lane * E + e];
                    float* dst = a.partial + ((size_t)g * a.B + b) * a.d + col;
#pragma unroll
                    for (int q = 0; q < E / 4; ++q)
                        reinterpret_cast<f32x4*>(dst)[q] = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
                }
            }
        }
        __syncthreads();
    }

}

// The gather-AXPY of a batch of 2-16 on the matrix cores (fp16 weights,
// coefficients read from memory; batches of up to 8 in the 8-row bucket):
//     partial[p][b][c] = sum over the part's rows u of coef[b][u] W[row(u)][c]
// as D = A B with v_mfma_f32_16x16x32_f16, A = the coefficients (16 batch
// rows x 32 rows of W, in fp16 hi + lo so that they keep about 22 bits) and
// B = those 32 rows of W x 16 columns.  Lane l supplies A row l % 16 and B
// column l % 16, both at rows 8 (l / 16) .. +7 of the step; D's register i
// holds batch row 4 (l / 16) + i, column l % 16.
//
// A workgroup takes one 256-column slice of a part of kAxG groups of 64 rows.
// Wave w first compacts group w's rows as the vector kernel does (dropping
// rows whose coefficients are all zero when asked) and writes their
// coefficients straight into the A operands.  Then each wave takes 64
// columns over all of the part's rows, 32 a step, with the weight loads of
// the next kAxPF steps in flight (a step of no live row is not multiplied,
// its loads re-read one row).  The B operand wants 8 rows of one column
// per lane while a row of W is contiguous along columns, so a step's 32 x 64
// tile goes through the wave's own LDS region: 16-byte loads (lane l: row
// 8 i + l / 8, columns 8 (l % 8) .. +7; 128 bytes, one line, of 8 rows a
// load), read back 2 bytes at a time.  Row r sits at position
// (r % 8) * 4 + r / 8 with a 160-byte stride, so that the 4 lane groups'
// reads (rows 8 apart) fall on disjoint banks.  One
// partial per part, not per group, keeps the partial sums (B x d floats a
// part, written and read back once) a quarter of what 64-row groups write
// (two groups a part, for twice the workgroups, measured slower).
typedef _Float16 f16x8a __attribute__((ext_vector_type(8)));
constexpr int kAxKS = 32;                      // rows per matrix-core step
constexpr int kAxWC = 64;                      // columns per wave (4 tiles of 16; 128 measured 2-11% slower)
constexpr int kAxLPR = kAxWC * 2 / 16;         // lanes per row in a load
constexpr int kAxRPL = kWave / kAxLPR;         // rows per load
constexpr int kAxNLD = kAxKS / kAxRPL;         // loads per step
constexpr int kAxNT = kAxWC / 16;              // column tiles
constexpr int kAxRS = kAxWC * 2 + 32;          // LDS bytes per tile row (the row + 32)
constexpr int kAxTile = kAxKS * kAxRS;         // one wave's tile
constexpr int kAxSlice = 4 * kAxWC;            // columns per workgroup
constexpr int kAxG = kBlock / kWave;           // 64-row groups per part (one per wave in the compaction)
constexpr int kAxSteps = kAxG * kRowsPerGroup / kAxKS;
constexpr int kAxPF = 4;                       // steps of weight loads in flight

template <int NB>
__global__ __launch_bounds__(kBlock) void k_axpy_mfma(AxpyArgs a) {
    static_assert(NB >= 8 && NB <= 16 && kRowsPerGroup == kWave && kRowsPerGroup % kAxKS == 0, "batch buckets of 8 and 16");
    __shared__ int s_row[kAxG][kRowsPerGroup];
    __shared__ int s_n[kAxG];
    __shared__ __align__(16) half_t aop[kAxSteps][2][16][kAxKS];     // [step][hi, lo][batch row][row of the step]
    __shared__ __align__(16) unsigned char tiles[kAxG * kAxTile];
    const half_t* W = (const half_t*)a.w;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, part = blockIdx.y;
    const int rows = a.n_rows_dev ? min(*a.n_rows_dev, a.rows) : a.rows;
    const int r0 = part * kAxG * kRowsPerGroup;
    if (r0 >= rows) return;                        // past the live rows: the finalize stops before this part
    {   // ---- wave wv compacts group wv's rows: live ones to slots 0 .. nl-1 in order
        const int u = r0 + wv * kRowsPerGroup + lane;
        bool live = false;
        int row = 0;
        float cf[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) cf[b] = 0.f;
        if (u < rows) {
            row = a.idx ? a.idx[u / a.blk] * a.blk + u % a.blk : u;
            bool any = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                cf[b] = b < a.B ? a.coef[(size_t)b * a.coef_stride + u] : 0.f;
                if (a.thresh) cf[b] = fabsf(cf[b]) > a.thr ? cf[b] : 0.f;
                any |= cf[b] != 0.f;
            }
            live = (unsigned)row < (unsigned)a.w_rows && (any || !a.skip_zero);   // an index outside W selects nothing
        }
        const unsigned lv = live ? 1u : 0u;
        const unsigned incl = wave_incl_scan(lv);
        const int nl = __builtin_amdgcn_readlane((int)incl, 63);
        // live lanes take slots 0 .. nl-1, the others the rest (zero coefficients)
        const int slot = live ? (int)incl - 1 : nl + lane - (int)incl;
        if (live) s_row[wv][slot] = row;
        const int st = wv * (kRowsPerGroup / kAxKS) + slot / kAxKS, k = slot % kAxKS;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const float c = (live && b < NB) ? cf[b < NB ? b : 0] : 0.f;
            const half_t hi = (half_t)c;
            aop[st][0][b][k] = hi;
            aop[st][1][b][k] = (half_t)(c - (float)hi);
        }
        if (lane == 0) {
            s_n[wv] = nl;
            if (a.rows_read && slice == 0 && nl > 0) atomicAdd(a.rows_read, nl);
        }
    }
    __syncthreads();
    // ---- this wave's 64 columns over the part's rows
    const int c0 = slice * kAxSlice + wv * kAxWC;  // d % 256 == 0
    int nlv[kAxG];
#pragma unroll
    for (int g = 0; g < kAxG; ++g) nlv[g] = __builtin_amdgcn_readfirstlane(s_n[g]);
    // a step's loads are unmasked: rows past a group's live ones read its last
    // live row (or row 0), their coefficients being zero
    u32x4 w[kAxPF][kAxNLD];
    auto load_step = [&](int st, int slot) {
        const int g = st / (kRowsPerGroup / kAxKS), kb = (st % (kRowsPerGroup / kAxKS)) * kAxKS;
#pragma unroll
        for (int i = 0; i < kAxNLD; ++i) {
            const int k = kb + kAxRPL * i + lane / kAxLPR;
            const int rr = nlv[g] > 0 ? s_row[g][k < nlv[g] ? k : nlv[g] - 1] : 0;
            const half_t* src = W + (size_t)rr * a.d + c0 + 8 * (lane % kAxLPR);
            w[slot][i] = ld16_stream(src);         // whole lines: the streaming hint measured faster here
        }
    };
#pragma unroll
    for (int p = 0; p < kAxPF; ++p) {
        load_step(p, p);
        asm volatile("" ::: "memory");
    }
    unsigned char* tile = tiles + wv * kAxTile;
    f32x4 acc[kAxNT];
#pragma unroll
    for (int nt = 0; nt < kAxNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < kAxSteps; ++st) {
        const int slot = st % kAxPF;
        const int g = st / (kRowsPerGroup / kAxKS), kb = (st % (kRowsPerGroup / kAxKS)) * kAxKS;
        if (kb < nlv[g]) {                         // uniform: a step with a live row
#pragma unroll
            for (int i = 0; i < kAxNLD; ++i) {     // row r of the step
                const int r = kAxRPL * i + lane / kAxLPR;
                *reinterpret_cast<u32x4*>(tile + ((r & 7) * 4 + (r >> 3)) * kAxRS + (lane % kAxLPR) * 16) = w[slot][i];
            }
            const f16x8a ahi = *reinterpret_cast<const f16x8a*>(&aop[st][0][lane & 15][8 * (lane >> 4)]);
            const f16x8a alo = *reinterpret_cast<const f16x8a*>(&aop[st][1][lane & 15][8 * (lane >> 4)]);
#pragma unroll
            for (int nt = 0; nt < kAxNT; ++nt) {
                f16x8a bop;
#pragma unroll
                for (int j = 0; j < 8; ++j)        // row 8 (l / 16) + j, column 16 nt + l % 16
                    bop[j] = *reinterpret_cast<const half_t*>(tile + (j * 4 + (lane >> 4)) * kAxRS +
                                                              (nt * 16 + (lane & 15)) * 2);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bop, acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bop, acc[nt], 0, 0, 0);
            }
        }
        if (st + kAxPF < kAxSteps) {               // the slot just consumed takes step st + PF
            asm volatile("" ::: "memory");
            load_step(st + kAxPF, slot);
            asm volatile("" ::: "memory");
        }
    }
#pragma unroll
    for (int nt = 0; nt < kAxNT; ++nt) {
        const int col = c0 + nt * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = 4 * (lane >> 4) + i;
            if (b < a.B) a.partial[((size_t)part * a.B + b) * a.d + col] = acc[nt][i];
        }
    }
}

// The rows a gather-AXPY covered, when a device-side count cut them short:
// its parts of rows_per_part rows past min(*n_rows_dev, rows) hold nothing.
struct FinLive {
    const int32_t* n_rows_dev = nullptr;
    int rows = 0, rows_per_part = 1;
};

// out[b][c] = residual[b][c] + bias[c] + sum_g partial[g][b][c].  A block
// covers 64 float4 columns of one batch row; its NT/64 waves each add a
// contiguous share of the groups (all loads of a share in flight together),
// then the shares are added in order.  One thread also advances a decode
// position when asked (nothing here reads it).  The epilogue stores the sum
// (FIN_STORE), its ReLU (FIN_RELU), or scatters a Q/K/V row (FIN_QKV): q in
// fp32, K and V into the caches' slot pos in fp16.
template <typename T, int NT = kBlock>
__device__ __forceinline__ void axpy_finalize_block(const float* __restrict__ partial, int n_groups, int B, int d,
                                                    const void* bias, const float* __restrict__ residual,
                                                    float* __restrict__ out, int32_t* advance,
                                                    const FinEpi& epi = FinEpi{}, const FinLive& lv = FinLive{}) {
    constexpr int NW = NT / kWave;
    constexpr int MAXQ = 16;                      // groups per share held in flight
    __shared__ f32x4 red[NW - 1][64];
    if (lv.n_rows_dev)                            // parts past the live rows were never written
        n_groups = min(n_groups, (max(0, min(*lv.n_rows_dev, lv.rows)) + lv.rows_per_part - 1) / lv.rows_per_part);
    const int b = blockIdx.y;
    const int c4 = blockIdx.x * 64 + (threadIdx.x & 63);
    const int q = threadIdx.x >> 6;
    const int n4 = d / 4;
    const int per = (n_groups + NW - 1) / NW;
    const int g0 = q * per, g1 = min(n_groups, g0 + per);
    // wave 0's bias and residual go out first, beside the partials, rather
    // than one more round trip after the reduction
    f32x4 bv = f32x4{0.f, 0.f, 0.f, 0.f}, rv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (q == 0 && c4 < n4) {
        if (bias) {
            const T* bb = (const T*)bias + (size_t)c4 * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = to_f32(bb[e]);
        }
        if (residual) rv = reinterpret_cast<const f32x4*>(residual + (size_t)b * d)[c4];
    }
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c4 < n4) {
        for (int gb = g0; gb < g1; gb += MAXQ) {
            f32x4 v[MAXQ];
#pragma unroll
            for (int i = 0; i < MAXQ; ++i)
                v[i] = gb + i < g1 ? reinterpret_cast<const f32x4*>(partial + ((size_t)(gb + i) * B + b) * d)[c4]
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < MAXQ; ++i) s += v[i];
        }
    }
    if (q > 0) red[q - 1][threadIdx.x & 63] = s;
    __syncthreads();
    if (q == 0 && c4 < n4) {
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) s = s + red[w][threadIdx.x];
        if (bias) s += bv;
        if (residual) s += rv;
        if (epi.mode == FIN_QKV) {
            const int c = c4 * 4, hd = epi.h * epi.dh;     // 4 columns of one head (d_h % 4 == 0)
            const int which = c / hd, head = (c % hd) / epi.dh, e = c % epi.dh;
            if (which == 0) {
                *reinterpret_cast<f32x4*>(epi.q + ((size_t)b * epi.h + head) * epi.dh + e) = s;
            } else {
                const int pos = epi.pos_dev ? *epi.pos_dev : epi.pos;
                if (pos >= 0 && pos < epi.max_len) {
                    half_t* dst = (which == 1 ? epi.k : epi.v) + (((size_t)b * epi.h + head) * epi.max_len + pos) * epi.dh + e;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[i] = (half_t)s[i];
                }
            }
        } else {
            if (epi.mode == FIN_RELU)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = fmaxf(s[i], 0.f);
            reinterpret_cast<f32x4*>(out + (size_t)b * d)[c4] = s;
        }
    }
    if (advance && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *advance += 1;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_axpy_finalize(const float* __restrict__ partial, int n_groups, int B, int d,
                                                          const void* bias, const float* __restrict__ residual,
                                                          float* __restrict__ out, int32_t* advance, FinEpi epi,
                                                          FinLive lv) {
    axpy_finalize_block<T>(partial, n_groups, B, d, bias, residual, out, advance, epi, lv);
}

// The finalize by 1024-thread workgroups, with one more workgroup (the last
// of row 0) that finds the selection threshold from the histogram the
// output projection built.
constexpr int kFinThrThreads = 1024;
struct FinThr {
    const uint32_t* keys;
    int n, k;
    const unsigned* hist;
    TopkThreshold* thr;
};

template <typename T>
__global__ __launch_bounds__(kFinThrThreads) void k_axpy_finalize_thr(const float* __restrict__ partial, int n_groups, int B,
                                                              int d, const void* bias, const float* __restrict__ residual,
                                                              float* __restrict__ out, int32_t* advance, FinThr f,
                                                              FinLive lv) {
    if (blockIdx.x == gridDim.x - 1) {
        if (blockIdx.y == 0) {
            __shared__ unsigned lds[kTopkThrWords];
            topk_threshold<kFinThrThreads>(f.keys, f.n, f.k, f.hist, lds, f.thr);
        }
        return;
    }
    axpy_finalize_block<T, kFinThrThreads>(partial, n_groups, B, d, bias, residual, out, advance, FinEpi{}, lv);
}

}  // namespace dv

namespace dvh {
using namespace dv;

bool topk_split_supported(int n, int k) { return k > 0 && k <= n && n % 4 == 0 && n <= kTopkRegN; }

AxpyPlan axpy_plan(int d, int rows, int wdt) {
    AxpyPlan p;
    const int E = 16 / elt_bytes(wdt);
    p.n_slices = cdiv(d, kWave * E);
    p.rows_per_group = kRowsPerGroup;
    p.n_groups = cdiv(rows < 1 ? 1 : rows, kRowsPerGroup);
    return p;
}

size_t axpy_ws_floats(const AxpyPlan& p, int B, int d) { return (size_t)p.n_groups * B * d; }

// Batches of 2-16 with fp16 weights, 256-column slices and coefficients in
// memory take the matrix cores (an output projection first merges its
// split-K partials into the attention output); a batch of one keeps the
// vector kernel, whose partials are a sixteenth of its weight bytes.
bool axpy_mfma_supported(int B, int d, int wdt) { return B >= 2 && B <= 16 && wdt == DV_F16 && d % kAxSlice == 0; }

static bool axpy_mfma_ok(const AxpyCall& c) { return axpy_mfma_supported(c.B, c.d, c.wdt) && !c.apart && !c.sel; }

template <int NB>
static void axpy_mfma_go(const AxpyArgs& a, int n_parts, hipStream_t s) {
    DV_LAUNCH((k_axpy_mfma<NB>), dim3(a.d / kAxSlice, n_parts), dim3(kBlock), 0, s, a);
}

template <typename T, int NB>
static void axpy_go(const AxpyArgs& a, int n_slices, hipStream_t s) {
    const int hs = a.tk_s ? cdiv(a.tk_n, kTopkSlice) : 0;
    const dim3 grid(n_slices + (hs ? 1 : 0), max(a.n_groups, hs));
    if (a.apart)
        DV_LAUNCH((k_axpy<T, NB, true>), grid, dim3(kBlock), 0, s, a);
    else
        DV_LAUNCH((k_axpy<T, NB, false>), grid, dim3(kBlock), 0, s, a);
}

dv_status launch_axpy_finalize(const float* partial, int n_groups, int B, int d, const void* bias, int bias_wdt,
                               const float* residual, float* out, hipStream_t s) {
    const dim3 fg(cdiv(d / 4, 64), B);
    if (bias_wdt == DV_F16)
        hipLaunchKernelGGL(k_axpy_finalize<half_t>, fg, dim3(kBlock), 0, s, partial, n_groups, B, d, bias, residual,
                           out, nullptr, FinEpi{}, FinLive{});
    else
        hipLaunchKernelGGL(k_axpy_finalize<float>, fg, dim3(kBlock), 0, s, partial, n_groups, B, d, bias, residual,
                           out, nullptr, FinEpi{}, FinLive{});
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DV_OK : fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
}

dv_status launch_axpy(const AxpyCall& c, hipStream_t s) {
    const AxpyPlan p = axpy_plan(c.d, c.rows, c.wdt);
    AxpyArgs a;
    a.w = c.w; a.d = c.d; a.w_rows = c.w_rows; a.rows = c.rows; a.n_rows_dev = c.n_rows_dev; a.idx = c.idx;
    a.blk = c.blk; a.coef = c.coef; a.coef_stride = c.coef_stride; a.skip_zero = c.skip_zero ? 1 : 0;
    a.apart = c.apart; a.num_splits = c.num_splits;
    a.thresh = c.thresh ? 1 : 0; a.thr = c.thr;
    a.B = c.B; a.n_groups = p.n_groups; a.partial = c.partial; a.rows_read = c.rows_read;
    a.tk_s = nullptr; a.tk_keys = nullptr; a.tk_n = a.tk_k = 0; a.tk_hist = nullptr; a.tk_thr = nullptr; a.tk_idx = nullptr;
    if (c.sel) {
        const TopkSel& t = *c.sel;
        if (c.B != 1 || !topk_split_supported(t.n, t.k) || ((uintptr_t)t.s & 15u) ||
            !t.hist || !t.thr || !t.idx || !t.keys || ((uintptr_t)t.hist & 15u) || ((uintptr_t)t.keys & 15u))
            return fail(DV_ERR_UNSUPPORTED, "selection slices beside a gather-AXPY: n=%d k=%d", t.n, t.k);
        a.tk_s = t.s; a.tk_keys = t.keys; a.tk_n = t.n; a.tk_k = t.k; a.tk_hist = t.hist; a.tk_thr = (const TopkThreshold*)t.thr;
        a.tk_idx = t.idx;
    }
    const int nb = c.B <= 1 ? 1 : c.B <= 2 ? 2 : c.B <= 4 ? 4 : c.B <= 8 ? 8 : 16;
#define DV_AXPY(NB)                                                            \
    case NB:                                                                   \
        if (c.wdt == DV_F16) axpy_go<half_t, NB>(a, p.n_slices, s);            \
        else axpy_go<float, NB>(a, p.n_slices, s);                             \
        break;
    const bool mf = axpy_mfma_ok(c);
    const int n_parts = mf ? cdiv(p.n_groups, kAxG) : p.n_groups;
    FinLive lv;
    lv.n_rows_dev = c.n_rows_dev; lv.rows = c.rows; lv.rows_per_part = mf ? kAxG * kRowsPerGroup : kRowsPerGroup;
    timed_begin(c.timed, s);
    if (mf) {
        if (nb <= 8) axpy_mfma_go<8>(a, n_parts, s);
        else axpy_mfma_go<16>(a, n_parts, s);
    } else {
        switch (nb) {
            DV_AXPY(1) DV_AXPY(2) DV_AXPY(4) DV_AXPY(8) DV_AXPY(16)
        }
    }
#undef DV_AXPY
    timed_end(c.timed, s);
    const dim3 fg(cdiv(c.d / 4, 64), c.B);
    if (c.sel && c.apart) {                        // the selection threshold rides in the finalize
        const FinThr f{c.sel->keys, c.sel->n, c.sel->k, c.sel->hist, (TopkThreshold*)c.sel->thr};
        const dim3 fg2(fg.x + 1, fg.y);
        if (c.wdt == DV_F16)
            hipLaunchKernelGGL(k_axpy_finalize_thr<half_t>, fg2, dim3(kFinThrThreads), 0, s, c.partial, n_parts, c.B,
                               c.d, c.bias, c.residual, c.out, c.advance, f, lv);
        else
            hipLaunchKernelGGL(k_axpy_finalize_thr<float>, fg2, dim3(kFinThrThreads), 0, s, c.partial, n_parts, c.B,
                               c.d, c.bias, c.residual, c.out, c.advance, f, lv);
    } else if (c.wdt == DV_F16)
        hipLaunchKernelGGL(k_axpy_finalize<half_t>, fg, dim3(kBlock), 0, s, c.partial, n_parts, c.B, c.d, c.bias,
                           c.residual, c.out, c.advance, c.epi, lv);
    else
        hipLaunchKernelGGL(k_axpy_finalize<float>, fg, dim3(kBlock), 0, s, c.partial, n_parts, c.B, c.d, c.bias,
                           c.residual, c.out, c.advance, c.epi, lv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
