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
#include "dv_internal.h"

#include <math.h>

namespace dv {

struct AttnArgs {
    const float* q;
    int B, n_sel, h;
    const int32_t* head_idx;
    const half_t* K;
    const half_t* V;
    int max_len, n_ctx;
    const int32_t* sel_idx;
    const int32_t* sel_len;
    int sel_cap, sel_end;
    float scale_log2;
    int num_splits, chunk;
    float* part;            // [B][n_sel][num_splits][DH + 2]
};

template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_split(AttnArgs a) {
    constexpr int LPR = DH / 8;            // lanes per row
    constexpr int RPW = kWave / LPR;       // rows per wave load
    constexpr int U = 4;                   // wave loads in flight (K and V each)
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
    int cnt, sl = 0;
    const int32_t* sidx = nullptr;
    if (a.sel_idx) {
        sl = min(max(a.sel_len[b * a.h + head], 0), a.sel_cap);
        sidx = a.sel_idx + ((size_t)b * a.h + head) * a.sel_cap;
        cnt = sl + max(0, a.n_ctx - a.sel_end);
    } else {
        cnt = a.n_ctx;
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
                const int p = sidx ? (j < sl ? sidx[j] : a.sel_end + (j - sl)) : j;
                valid[u] = (unsigned)p < (unsigned)a.n_ctx;       // a retained index past the cache reads nothing
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
template <int DH>
__global__ __launch_bounds__(kBlock) void k_attn_combine(const float* __restrict__ part, int rows,
                                                         int num_splits, float* __restrict__ o) {
    constexpr int PER = DH >= 64 ? DH / 64 : 1;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float* P = part + (size_t)row * num_splits * (DH + 2);
    float M = -INFINITY;
    for (int c = 0; c < num_splits; ++c) {
        const float* pc = P + (size_t)c * (DH + 2);
        if (pc[DH + 1] > 0.f) M = fmaxf(M, pc[DH]);
    }
    float num[PER], den = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) num[i] = 0.f;
    if (M != -INFINITY) {
        for (int c = 0; c < num_splits; ++c) {
            const float* pc = P + (size_t)c * (DH + 2);
            const float lc = pc[DH + 1];
            if (!(lc > 0.f)) continue;
            const float w = exp2f(pc[DH] - M);
            den = fmaf(w, lc, den);
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = lane * PER + i;
                if (e < DH) num[i] = fmaf(w, pc[e], num[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane * PER + i;
        if (e < DH) o[(size_t)row * DH + e] = den > 0.f ? num[i] / den : 0.f;
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

int splitk_auto(int max_positions, int rows) {
    if (max_positions < 1) max_positions = 1;
    if (rows < 1) rows = 1;
    // about 32 positions (16 KB of K and V at d_h = 128) per wave, at most
    // 64K waves per launch
    int splits = cdiv(max_positions, 32);
    const int cap = 65536 / rows > 1 ? 65536 / rows : 1;
    if (splits > cap) splits = cap;
    return splits < 1 ? 1 : splits;
}

dv_status launch_splitk(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel,
                        const dv_kv_view* kv, float scale, int num_splits, float* o, float* part,
                        hipStream_t s) {
    if (n_sel == 0) return DV_OK;
    const int maxpos = kv->sel_idx ? kv->sel_cap + (kv->n_ctx - kv->sel_end) : kv->n_ctx;
    if (num_splits <= 0) num_splits = splitk_auto(maxpos, B * n_sel);
    AttnArgs a;
    a.q = q; a.B = B; a.n_sel = n_sel; a.h = kv->h; a.head_idx = head_idx;
    a.K = (const half_t*)kv->k_cache; a.V = (const half_t*)kv->v_cache;
    a.max_len = kv->max_len; a.n_ctx = kv->n_ctx;
    a.sel_idx = kv->sel_idx; a.sel_len = kv->sel_len; a.sel_cap = kv->sel_cap; a.sel_end = kv->sel_end;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.num_splits = num_splits;
    a.chunk = cdiv(maxpos < 1 ? 1 : maxpos, num_splits);
    a.part = part;
    const int tasks = B * n_sel * num_splits;
    const int rows = B * n_sel;
#define DV_ATT(DH)                                                                                   \
    case DH:                                                                                         \
        hipLaunchKernelGGL((k_attn_split<DH>), dim3(cdiv(tasks, 4)), dim3(kBlock), 0, s, a);        \
        hipLaunchKernelGGL((k_attn_combine<DH>), dim3(cdiv(rows, 4)), dim3(kBlock), 0, s, part, rows, \
                           num_splits, o);                                                           \
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
