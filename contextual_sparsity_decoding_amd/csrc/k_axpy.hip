// Gather-AXPY: out[b] = residual[b] + bias + sum_u coef[b][u] * W[row(u)]
// for the second MLP layer (DejaVu Eq. 1, rows of W2^T) and the output
// projection (DejaVu Eq. 2, rows of W^O, d_h per selected head).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157); §4.4 stores W2 and W^O transposed so a
// selected neuron or head is a contiguous run of rows.
//
// Work split: the d output columns are cut into slices of one wave-load
// (64 lanes x 16 bytes); the selected rows into groups of up to 64.  A
// workgroup (4 waves) first stages its group's row indices and coefficients
// in LDS (one batch of loads, an ordered compaction that drops rows whose
// coefficients are all zero when asked), then every wave issues its weight
// loads back to back, reduces across the 4 waves in LDS and writes one
// partial sum per group.  k_axpy_finalize adds the partials in a fixed
// order, plus bias and residual.  Results do not depend on scheduling.
#include "dv_internal.h"

namespace dv {

constexpr int kRowsPerGroup = 64;

struct AxpyArgs {
    const void* w;
    int d, w_rows, rows;      // W has w_rows rows of d; rows = selected rows (u)
    const int32_t* n_rows_dev;
    const int32_t* idx;       // row(u) = idx[u / blk] * blk + u % blk, or u when NULL
    int blk;
    const float* coef;        // coef[b * coef_stride + u]
    int coef_stride;
    int skip_zero;
    int B, n_groups;
    float* partial;           // [n_groups][B][d]
    int32_t* rows_read;
};

template <typename T, int NB, int U>
__global__ __launch_bounds__(kBlock) void k_axpy(AxpyArgs a) {
    constexpr int E = Vec<T>::E;
    constexpr int SW = kWave * E;                  // columns per slice
    constexpr int NBC = NB < 4 ? NB : 4;           // batch rows per LDS reduction round
    __shared__ int s_row[kRowsPerGroup];
    __shared__ float s_cf[kRowsPerGroup * NB];
    __shared__ float red[3][NBC][SW];
    __shared__ unsigned tot[17];
    const T* W = (const T*)a.w;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, g = blockIdx.y;
    const int col = slice * SW + lane * E;
    const bool colok = col < a.d;
    const int rows = a.n_rows_dev ? min(*a.n_rows_dev, a.rows) : a.rows;
    const int r0 = g * kRowsPerGroup;

    // ---- prologue: this group's rows and coefficients, compacted in order
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
            any |= cf[b] != 0.f;
        }
        live = (unsigned)row < (unsigned)a.w_rows && (any || !a.skip_zero);   // an index outside W selects nothing
    }
    unsigned nlive;
    const unsigned slot = block_excl_scan(live ? 1u : 0u, tot, &nlive);
    if (live) {
        s_row[slot] = row;
#pragma unroll
        for (int b = 0; b < NB; ++b) s_cf[slot * NB + b] = cf[b];
    }
    __syncthreads();
    if (a.rows_read && slice == 0 && threadIdx.x == 0 && nlive > 0) atomicAdd(a.rows_read, (int)nlive);

    // ---- stream the live rows: wave wv takes rows wv, wv+4, ...
    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;
    for (int k0 = wv; k0 < (int)nlive; k0 += 4 * U) {
        u32x4 w[U];
#pragma unroll
        for (int t = 0; t < U; ++t) {
            const int k = k0 + 4 * t;
            w[t] = (k < (int)nlive && colok) ? ld16_stream(W + (size_t)s_row[k] * a.d + col) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int t = 0; t < U; ++t) {
            const int k = k0 + 4 * t;
            if (k < (int)nlive) {
                float f[E];
                unpack(w[t], f, T());
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float c = s_cf[k * NB + b];
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[b][e] = fmaf(c, f[e], acc[b][e]);
                }
            }
        }
    }

    // ---- reduce the 4 waves into wave 0, NBC batch rows at a time
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

// out[b][c] = residual[b][c] + bias[c] + sum_g partial[g][b][c].  A block
// covers 64 float4 columns of one batch row; its 4 waves each add a
// contiguous quarter of the groups (all loads of a quarter in flight
// together), then the quarters are added in order.  One thread also
// advances a decode position when asked (nothing here reads it).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_axpy_finalize(const float* __restrict__ partial, int n_groups, int B, int d,
                                                          const void* bias, const float* __restrict__ residual,
                                                          float* __restrict__ out, int32_t* advance) {
    constexpr int MAXQ = 16;                      // groups per quarter held in flight
    __shared__ f32x4 red[3][64];
    const int b = blockIdx.y;
    const int c4 = blockIdx.x * 64 + (threadIdx.x & 63);
    const int q = threadIdx.x >> 6;
    const int n4 = d / 4;
    const int per = (n_groups + 3) / 4;
    const int g0 = q * per, g1 = min(n_groups, g0 + per);
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
        s = s + red[0][threadIdx.x] + red[1][threadIdx.x] + red[2][threadIdx.x];
        if (bias) {
            const T* bb = (const T*)bias + (size_t)c4 * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] += to_f32(bb[e]);
        }
        if (residual) s += reinterpret_cast<const f32x4*>(residual + (size_t)b * d)[c4];
        reinterpret_cast<f32x4*>(out + (size_t)b * d)[c4] = s;
    }
    if (advance && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *advance += 1;
}

}  // namespace dv

namespace dvh {
using namespace dv;

AxpyPlan axpy_plan(int d, int rows, int wdt) {
    AxpyPlan p;
    const int E = 16 / elt_bytes(wdt);
    p.n_slices = cdiv(d, kWave * E);
    p.rows_per_group = kRowsPerGroup;
    p.n_groups = cdiv(rows < 1 ? 1 : rows, kRowsPerGroup);
    return p;
}

size_t axpy_ws_floats(const AxpyPlan& p, int B, int d) { return (size_t)p.n_groups * B * d; }

template <typename T, int NB>
static void axpy_go(const AxpyArgs& a, int n_slices, hipStream_t s) {
    hipLaunchKernelGGL((k_axpy<T, NB, 16>), dim3(n_slices, a.n_groups), dim3(kBlock), 0, s, a);
}

dv_status launch_axpy(const void* w, int wdt, int d, int w_rows, int rows, const int32_t* n_rows_dev,
                      const int32_t* idx, int blk, const float* coef, int coef_stride, bool skip_zero,
                      int B, const void* bias, const float* residual, float* out, int32_t* rows_read,
                      float* partial, int32_t* advance, hipStream_t s) {
    const AxpyPlan p = axpy_plan(d, rows, wdt);
    AxpyArgs a;
    a.w = w; a.d = d; a.w_rows = w_rows; a.rows = rows; a.n_rows_dev = n_rows_dev; a.idx = idx; a.blk = blk;
    a.coef = coef; a.coef_stride = coef_stride; a.skip_zero = skip_zero ? 1 : 0;
    a.B = B; a.n_groups = p.n_groups; a.partial = partial; a.rows_read = rows_read;
    const int nb = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B <= 8 ? 8 : 16;
#define DV_AXPY(NB)                                                            \
    case NB:                                                                   \
        if (wdt == DV_F16) axpy_go<half_t, NB>(a, p.n_slices, s);              \
        else axpy_go<float, NB>(a, p.n_slices, s);                             \
        break;
    switch (nb) {
        DV_AXPY(1) DV_AXPY(2) DV_AXPY(4) DV_AXPY(8) DV_AXPY(16)
    }
#undef DV_AXPY
    const dim3 fg(cdiv(d / 4, 64), B);
    if (wdt == DV_F16)
        hipLaunchKernelGGL(k_axpy_finalize<half_t>, fg, dim3(kBlock), 0, s, partial, p.n_groups, B, d, bias, residual,
                           out, advance);
    else
        hipLaunchKernelGGL(k_axpy_finalize<float>, fg, dim3(kBlock), 0, s, partial, p.n_groups, B, d, bias, residual,
                           out, advance);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
