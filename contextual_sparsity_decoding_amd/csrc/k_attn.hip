// Split-K decode attention over the selected heads, optionally over a
// retained subset of cached positions, and its combine step.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §2.3 Eq. (2) (attention of the selected
// heads S_A); ByteCross = "Where Activation Sparsity and KV-Cache Sparsity
// Cross in LLM Decoding" (arXiv 2609.33889v1), §4.1 / App. A (every mode
// reads the cache through one split-K kernel; retained positions per KV head
// plus the entries appended after selection, §3.2).
//
// A wave owns one (batch row, head, range of positions).  One cached K or V
// row of d_h fp16 is d_h/8 lanes x 16 bytes, so a wave load covers 64*8/d_h
// rows.  Scores live in the log2 domain (q is pre-scaled by scale*log2 e) so
// exp is the native exp2.  Each wave keeps a running (max, sum, weighted V),
// merges its row groups with shuffles and writes one partial; the combine
// kernel merges the partials of a head in split order.
//
// In the look-ahead schedule the launch also carries the next layer's
// predictor second layers (DejaVu §4.3): workgroups past the attention grid
// take that role, so the predictions need no launch or stream of their own.
#include "pred.h"

#include <math.h>

namespace dv {

struct AttnArgs {
    const float* q;
    int B, n_sel, h;
    const int32_t* head_idx;
    const half_t* K;
    const half_t* V;
    int max_len, n_ctx;       // n_ctx: the count, or its bound when n_dev is set
    const int32_t* n_dev;     // count read at run time (+ n_add), or NULL
    int n_add;
    const int32_t* sel_idx;
    const int32_t* sel_len;
    int sel_cap, sel_end;
    int win_sink, win_len;  // KV window: positions < win_sink and the last win_len (win_len > 0)
    float scale_log2;
    int num_splits, chunk;
    float* part;            // [B][n_sel][num_splits][DH + 2]
    int32_t* mark_valid;    // [B][h]: set the selected heads to mark_pos (decode layer), or NULL
    int mark_pos;
    const int32_t* mark_pos_dev;
    int attn_blocks;        // workgroups of attention; later ones run `pred` (weights of type T)
    Pred2Args pred;
};

template <int DH, typename T>
__global__ __launch_bounds__(kBlock) void k_attn_split(AttnArgs a) {
    constexpr int LPR = DH / 8;            // lanes per row
    constexpr int RPW = kWave / LPR;       // rows per wave load
    constexpr int U = 4;                   // wave loads in flight (K and V each)
    if ((int)blockIdx.x >= a.attn_blocks) {
        extern __shared__ float hid[];
        pred2_pair_block<T>(blockIdx.x - a.attn_blocks, hid, a.pred);
        return;
    }
    if (a.mark_valid && blockIdx.x == 0) {  // Q/K/V has finished: the selected heads hold K/V up to pos
        const int p = a.mark_pos_dev ? *a.mark_pos_dev : a.mark_pos;
        if (p >= 0 && p < a.max_len)
            for (int i = threadIdx.x; i < a.B * a.n_sel; i += kBlock) {
                const int hh = a.head_idx ? a.head_idx[i % a.n_sel] : i % a.n_sel;
                if ((unsigned)hh < (unsigned)a.h) a.mark_valid[(i / a.n_sel) * a.h + hh] = p;
            }
    }
    const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (task >= a.B * a.n_sel * a.num_splits) return;
    const int c = task % a.num_splits;
    const int bs = task / a.num_splits;
    const int s = bs % a.n_sel, b = bs / a.n_sel;
    int head = a.head_idx ? a.head_idx[s] : s;
    const bool head_ok = (unsigned)head < (unsigned)a.h;     // else: no positions, o = 0
    if (!head_ok) head = 0;
    const int lane = threadIdx.x & 63;
    const int g = lane / LPR, t = lane % LPR;

    float qv[8];
    {
        const float* qp = a.q + ((size_t)bs * DH + t * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qp[e] * a.scale_log2;
    }
    const int n_ctx = a.n_dev ? min(max(*a.n_dev + a.n_add, 0), a.n_ctx) : a.n_ctx;
    int cnt, sl = 0;
    const int32_t* sidx = nullptr;
    // KV window (ByteCross §5.1, App. A): the sinks [0, w0) and the recent
    // positions [wst, n_ctx), read in place
    const bool win = a.win_len > 0;
    const int w0 = win ? min(max(a.win_sink, 0), n_ctx) : 0;
    const int wst = win ? max(w0, n_ctx - a.win_len) : 0;
    if (a.sel_idx) {
        sl = min(max(a.sel_len[b * a.h + head], 0), a.sel_cap);
        sidx = a.sel_idx + ((size_t)b * a.h + head) * a.sel_cap;
        cnt = sl + max(0, n_ctx - a.sel_end);
    } else if (win) {
        cnt = w0 + (n_ctx - wst);
    } else {
        cnt = n_ctx;
    }
    if (!head_ok) cnt = 0;
    const int j0 = c * a.chunk;
    const int j1 = min(cnt, j0 + a.chunk);
    const size_t hb = ((size_t)b * a.h + head) * a.max_len;
    const half_t* Kh = a.K + hb * DH + t * 8;
    const half_t* Vh = a.V + hb * DH + t * 8;

    float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;

    for (int jb = j0; jb < j1; jb += RPW * U) {
        u32x4 kw[U], vw[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jb + u * RPW + g;
            valid[u] = j < j1;
            kw[u] = vw[u] = u32x4{0u, 0u, 0u, 0u};
            if (valid[u]) {
                const int p = sidx ? (j < sl ? sidx[j] : a.sel_end + (j - sl))
                              : win ? (j < w0 ? j : wst + (j - w0)) : j;
                valid[u] = (unsigned)p < (unsigned)n_ctx;         // a retained index past the cache reads nothing
                if (valid[u]) {
                    kw[u] = ld16(Kh + (size_t)p * DH);
                    vw[u] = ld16(Vh + (size_t)p * DH);
                }
            }
        }
        float sc[U];
        float mx = -INFINITY;
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
        if (mn == -INFINITY) continue;           // nothing valid in this group yet
        const float corr = exp2f(m - mn);        // m == -inf gives 0
        l *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = valid[u] ? exp2f(sc[u] - mn) : 0.f;
            float f[8];
            unpack(vw[u], f, half_t());
            l += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, f[e], acc[e]);
        }
        m = mn;
    }
    // merge the RPW row groups of the wave
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
        const float mo = __shfl_xor(m, off, kWave);
        const float lo = __shfl_xor(l, off, kWave);
        float ao[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ao[e] = __shfl_xor(acc[e], off, kWave);
        const float M = fmaxf(m, mo);
        if (M != -INFINITY) {
            const float ca = exp2f(m - M), cb = exp2f(mo - M);
            l = l * ca + lo * cb;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = acc[e] * ca + ao[e] * cb;
            m = M;
        }
    }
    if (g == 0) {
        float* out = a.part + (size_t)task * (DH + 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[t * 8 + e] = acc[e];
        if (t == 0) {
            out[DH] = m;
            out[DH + 1] = l;
        }
    }
}

// o = sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c over splits with l_c > 0.
// One workgroup per row: the block finds M, then each wave adds a contiguous
// quarter of the splits (up to 16 splits' loads in flight at once) and the
// quarters are added in order.
template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_combine(const float* __restrict__ part, int rows,
                                                         int num_splits, float* __restrict__ o) {
    constexpr int PER = DH >= 64 ? DH / 64 : 1;
    constexpr int MAXQ = 16;
    __shared__ float red_m[4];
    __shared__ float red_n[3][DH + 1];
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const float* P = part + (size_t)row * num_splits * (DH + 2);
    float M = -INFINITY;
    for (int c = threadIdx.x; c < num_splits; c += kBlock) {
        const float* pc = P + (size_t)c * (DH + 2);
        if (pc[DH + 1] > 0.f) M = fmaxf(M, pc[DH]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    if (lane == 0) red_m[wv] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
    const int per = (num_splits + 3) / 4;
    const int c0 = wv * per, c1 = min(num_splits, c0 + per);
    float num[PER], den = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = 0.f;
    if (M != -INFINITY) {
        for (int cb = c0; cb < c1; cb += MAXQ) {
            float ml[MAXQ][2], av[MAXQ][PER];
#pragma unroll
            for (int t = 0; t < MAXQ; ++t) {
                const bool ok = cb + t < c1;
                const float* pc = P + (size_t)(ok ? cb + t : c0) * (DH + 2);
                ml[t][0] = pc[DH];
                ml[t][1] = ok ? pc[DH + 1] : 0.f;
#pragma unroll
                for (int i = 0; i < PER; ++i) {
                    const int e = lane * PER + i;
                    av[t][i] = e < DH ? pc[e] : 0.f;
                }
            }
#pragma unroll
            for (int t = 0; t < MAXQ; ++t) {
                if (!(ml[t][1] > 0.f)) continue;
                const float wgt = exp2f(ml[t][0] - M);
                den = fmaf(wgt, ml[t][1], den);
#pragma unroll
                for (int i = 0; i < PER; ++i) num[i] = fmaf(wgt, av[t][i], num[i]);
            }
        }
    }
    if (wv > 0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane * PER + i;
            if (e < DH) red_n[wv - 1][e] = num[i];
        }
        if (lane == 0) red_n[wv - 1][DH] = den;
    }
    __syncthreads();
    if (wv == 0) {
        const float dt = den + red_n[0][DH] + red_n[1][DH] + red_n[2][DH];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane * PER + i;
            if (e < DH) {
                const float nt = num[i] + red_n[0][e] + red_n[1][e] + red_n[2][e];
                o[(size_t)row * DH + e] = dt > 0.f ? nt / dt : 0.f;
            }
        }
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

int splitk_auto(int max_positions, int rows) {
    if (max_positions < 1) max_positions = 1;
    if (rows < 1) rows = 1;
    // about 32 positions (16 KB of K and V at d_h = 128) per wave, but at
    // most about 8192 waves per launch and 128 splits: every split of a row
    // is merged again (in each column slice of the output projection at
    // batch 1, by the merge kernel at larger batches), and a wave keeps
    // streaming its longer range at HBM speed (OPT-175B width, batch 16:
    // 5 splits instead of 17, 5.72 -> 5.33 ms per 8 layers; d = 4096 at 32K
    // positions: 128 instead of 1024, 6.65 -> 5.05 ms per token)
    int splits = cdiv(max_positions, 32);
    const int cap = 8192 / rows > 1 ? 8192 / rows : 1;
    if (splits > cap) splits = cap;
    if (splits > 128) splits = 128;
    return splits < 1 ? 1 : splits;
}

int view_positions(const dv_kv_view* kv) {
    if (kv->sel_idx) return kv->sel_cap + (kv->n_ctx - kv->sel_end);
    if (kv->win_len > 0) return min(kv->n_ctx, kv->win_sink + kv->win_len);
    return kv->n_ctx;
}

dv_status launch_splitk(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel,
                        const dv_kv_view* kv, const int32_t* n_dev, int n_add, float scale, int num_splits, float* o,
                        float* part, int32_t* mark_valid, int mark_pos, const int32_t* mark_pos_dev, hipStream_t s,
                        int* splits_used, const Pred2Args* pred) {
    const bool win = kv->win_len > 0 && !kv->sel_idx;
    const int maxpos = view_positions(kv);
    if (num_splits <= 0) num_splits = splitk_auto(maxpos, B * n_sel);
    if (splits_used) *splits_used = num_splits;
    if (n_sel == 0 && !pred) return DV_OK;
    AttnArgs a;
    a.q = q; a.B = B; a.n_sel = n_sel; a.h = kv->h; a.head_idx = head_idx;
    a.K = (const half_t*)kv->k_cache; a.V = (const half_t*)kv->v_cache;
    a.max_len = kv->max_len; a.n_ctx = kv->n_ctx; a.n_dev = n_dev; a.n_add = n_add;
    a.sel_idx = kv->sel_idx; a.sel_len = kv->sel_len; a.sel_cap = kv->sel_cap; a.sel_end = kv->sel_end;
    a.win_sink = win ? kv->win_sink : 0; a.win_len = win ? kv->win_len : 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.num_splits = num_splits;
    a.chunk = cdiv(maxpos < 1 ? 1 : maxpos, num_splits);
    a.part = part;
    a.mark_valid = mark_valid; a.mark_pos = mark_pos; a.mark_pos_dev = mark_pos_dev;
    const int tasks = B * n_sel * num_splits;
    const int rows = B * n_sel;
    a.attn_blocks = cdiv(tasks, 4);
    a.pred = pred ? *pred : Pred2Args{};
    const int grid = a.attn_blocks + (pred ? pred2_blocks(*pred) : 0);
    const size_t lds = pred ? (size_t)((pred->r_m + 3) & ~3) * sizeof(float) : 0;
    const bool pf32 = pred && pred->wdt == DV_F32;
#define DV_ATT(DH)                                                                                   \
    case DH:                                                                                         \
        if (pf32) DV_LAUNCH((k_attn_split<DH, float>), dim3(grid), dim3(kBlock), lds, s, a);          \
        else DV_LAUNCH((k_attn_split<DH, half_t>), dim3(grid), dim3(kBlock), lds, s, a);             \
        if (o && rows)                                                                               \
            hipLaunchKernelGGL((k_attn_combine<DH>), dim3(rows), dim3(kBlock), 0, s, part, rows,    \
                               num_splits, o);                                                       \
        break;
    switch (d_h) {
        DV_ATT(32) DV_ATT(64) DV_ATT(128) DV_ATT(256)
        default:
            return fail(DV_ERR_UNSUPPORTED, "d_h %d", d_h);
    }
#undef DV_ATT
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
