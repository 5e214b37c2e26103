// Sparse Q/K/V projections with KV append and hole fill (DejaVu §4.2):
// entry point (the kernel instantiations are in k_qkv_*.hip).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).
#include "qkv.h"

namespace dv {

// Selected heads now hold K/V up to pos (run after k_qkv has finished).
__global__ void k_mark_valid_qkv(const int32_t* __restrict__ head_idx, int n_sel, int B, int h, int pos,
                                 const int32_t* __restrict__ pos_dev, int max_len, int32_t* __restrict__ valid_upto) {
    const int p = pos_dev ? *pos_dev : pos;
    if (p < 0 || p >= max_len) return;
    for (int i = threadIdx.x; i < B * n_sel; i += blockDim.x) {
        const int b = i / n_sel, s = i % n_sel;
        const int head = head_idx ? head_idx[s] : s;
        if ((unsigned)head < (unsigned)h) valid_upto[b * h + head] = p;
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

template <typename T>
static dv_status qkv_launch_t(const QkvArgs& a, int ch, hipStream_t s) {
    switch (nb_bucket(a.B)) {
        case 1: return qkv_go<T, 1>(a, ch, s);
        case 2: return qkv_go<T, 2>(a, ch, s);
        case 4: return qkv_go<T, 4>(a, ch, s);
        case 8: return qkv_go<T, 8>(a, ch, s);
        default: return qkv_go<T, 16>(a, ch, s);
    }
}

bool qkv_supported(int B, int d, int wdt) {
    (void)B;
    return ch_tier(d, wdt) > 0;
}

dv_status launch_qkv(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                     const void* w, const void* bias, int wdt, float* q, const dv_kv_state* kv, bool mark_valid,
                     hipStream_t s, const float* ln_g, const float* ln_b, float eps, const RowArgs* pred) {
    if (n_sel == 0 && !pred) return DV_OK;
    QkvArgs a;
    a.ln_g = ln_g; a.ln_b = ln_b; a.eps = eps;
    a.pred = pred ? *pred : RowArgs{};
    a.y = y; a.B = B; a.d = d; a.h = h; a.dh = d_h; a.n_sel = n_sel;
    a.head_idx = head_idx; a.w = w; a.bias = bias; a.q = q;
    a.K = (half_t*)kv->k_cache; a.V = (half_t*)kv->v_cache;
    a.max_len = kv->max_len; a.pos = kv->pos; a.pos_dev = kv->pos_dev;
    a.y_buf = kv->y_buf; a.valid_upto = kv->valid_upto;
    const int ch = ch_tier(d, wdt);
    const dv_status st = wdt == DV_F16 ? qkv_launch_t<half_t>(a, ch, s) : qkv_launch_t<float>(a, ch, s);
    if (st != DV_OK) return st;
    DV_LAUNCH_CHECK();
    if (mark_valid && a.y_buf && a.valid_upto) {
        hipLaunchKernelGGL(k_mark_valid_qkv, dim3(1), dim3(256), 0, s, head_idx, n_sel, B, h, kv->pos, kv->pos_dev,
                           kv->max_len, kv->valid_upto);
        DV_LAUNCH_CHECK();
    }
    return DV_OK;
}

}  // namespace dvh
