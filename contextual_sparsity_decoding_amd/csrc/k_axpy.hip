// Gather-AXPY: out[b] = residual[b] + bias + sum_u coef[b][u] * W[row(u)]
// for the second MLP layer (DejaVu Eq. 1, rows of W2^T) and the output
// projection (DejaVu Eq. 2, rows of W^O, d_h per selected head).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157); §4.4 stores W2 and W^O transposed so a
// selected neuron or head is a contiguous run of rows.
//
// Work split: the d output columns are cut into slices of one wave-load
// (64 lanes x 16 bytes); the selected rows into groups.  A workgroup
// (4 waves) streams one slice of its group's rows, reduces across its waves
// in LDS and writes one partial per group.  The last workgroup of a slice
// to finish (atomic counter) adds the partials in group order, plus bias and
// residual, so the result does not depend on scheduling.
#include "dv_internal.h"

namespace dv {

struct AxpyArgs {
    const void* w;
    int d, w_rows, rows;      // w has w_rows rows of d; rows = selected rows (u)
    const int32_t* n_rows_dev;
    const int32_t* idx;      // row(u) = idx[u / blk] * blk + u % blk, or u when NULL
    int blk;
    const float* coef;       // coef[b * coef_stride + u]
    int coef_stride;
    int skip_zero;
    int B, n_groups, rows_per_group;
    const void* bias;
    const float* residual;
    float* out;
    int32_t* rows_read;
    float* partial;          // [n_groups][B][d]
    unsigned* counters;      // [n_slices]
};

template <typename T, int NB, int U>
__global__ __launch_bounds__(kBlock) void k_axpy(AxpyArgs a) {
    constexpr int E = Vec<T>::E;
    constexpr int SW = kWave * E;                  // columns per slice
    constexpr int NBC = NB < 4 ? NB : 4;           // batch rows per LDS reduction round
    __shared__ float red[3][NBC][SW];
    __shared__ int last;
    const T* W = (const T*)a.w;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, g = blockIdx.y;
    const int col = slice * SW + lane * E;
    const bool colok = col < a.d;
    const int rows = a.n_rows_dev ? min(*a.n_rows_dev, a.rows) : a.rows;
    const int r0 = g * a.rows_per_group;
    const int r1 = min(rows, r0 + a.rows_per_group);

    float acc[NB][E];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[b][e] = 0.f;
    int nread = 0;

    for (int u0 = r0 + wv; u0 < r1; u0 += 4 * U) {
        u32x4 w[U];
        float cf[U][NB];
        bool live[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = u0 + 4 * i;
            live[i] = u < r1;
            bool any = false;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float c = (live[i] && b < a.B) ? a.coef[(size_t)b * a.coef_stride + u] : 0.f;
                cf[i][b] = c;
                any |= c != 0.f;
            }
            if (a.skip_zero) live[i] = live[i] && any;
            w[i] = u32x4{0u, 0u, 0u, 0u};
            int row = 0;
            if (live[i]) {
                row = a.idx ? a.idx[u / a.blk] * a.blk + u % a.blk : u;
                live[i] = (unsigned)row < (unsigned)a.w_rows;   // an index outside W selects nothing
            }
            if (live[i] && colok) w[i] = ld16_stream(W + (size_t)row * a.d + col);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (!live[i]) continue;
            ++nread;
            float f[E];
            unpack(w[i], f, T());
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[b][e] = fmaf(cf[i][b], f[e], acc[b][e]);
        }
    }
    if (a.rows_read && slice == 0 && lane == 0 && nread > 0) atomicAdd(a.rows_read, nread);

    // reduce the 4 waves into wave 0, NBC batch rows at a time
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
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float v = acc[b][e] + red[0][bb][lane * E + e] + red[1][bb][lane * E + e] +
                                    red[2][bb][lane * E + e];
                    if (b < a.B && colok) a.partial[((size_t)g * a.B + b) * a.d + col + e] = v;
                }
            }
        }
        __syncthreads();
    }

    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(&a.counters[slice], 1u) == gridDim.y - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();
    const T* bias = (const T*)a.bias;
    for (int i = threadIdx.x; i < a.B * SW; i += kBlock) {
        const int b = i / SW, c = slice * SW + i % SW;
        if (c >= a.d) continue;
        float s = 0.f;
        for (int gg = 0; gg < a.n_groups; ++gg) s += a.partial[((size_t)gg * a.B + b) * a.d + c];
        if (bias) s += to_f32(bias[c]);
        if (a.residual) s += a.residual[(size_t)b * a.d + c];
        a.out[(size_t)b * a.d + c] = s;
    }
    if (threadIdx.x == 0) a.counters[slice] = 0u;
}

}  // namespace dv

namespace dvh {
using namespace dv;

AxpyPlan axpy_plan(int d, int rows, int wdt) {
    AxpyPlan p;
    const int E = 16 / elt_bytes(wdt);
    p.n_slices = cdiv(d, kWave * E);
    // about 32 rows (8 per wave) per group; at most 128 groups
    int groups = cdiv(rows < 1 ? 1 : rows, 32);
    if (groups > 128) groups = 128;
    if (groups < 1) groups = 1;
    p.rows_per_group = cdiv(rows < 1 ? 1 : rows, groups);
    p.n_groups = cdiv(rows < 1 ? 1 : rows, p.rows_per_group);
    return p;
}

size_t axpy_ws_floats(const AxpyPlan& p, int B, int d) { return (size_t)p.n_groups * B * d; }

template <typename T, int NB>
static void axpy_go(const AxpyArgs& a, int n_slices, hipStream_t s) {
    hipLaunchKernelGGL((k_axpy<T, NB, 8>), dim3(n_slices, a.n_groups), dim3(kBlock), 0, s, a);
}

dv_status launch_axpy(const void* w, int wdt, int d, int w_rows, int rows, const int32_t* n_rows_dev,
                      const int32_t* idx, int blk, const float* coef, int coef_stride, bool skip_zero,
                      int B, const void* bias, const float* residual, float* out, int32_t* rows_read,
                      float* partial, unsigned* counters, hipStream_t s) {
    const AxpyPlan p = axpy_plan(d, rows, wdt);
    AxpyArgs a;
    a.w = w; a.d = d; a.w_rows = w_rows; a.rows = rows; a.n_rows_dev = n_rows_dev; a.idx = idx; a.blk = blk;
    a.coef = coef; a.coef_stride = coef_stride; a.skip_zero = skip_zero ? 1 : 0;
    a.B = B; a.n_groups = p.n_groups; a.rows_per_group = p.rows_per_group;
    a.bias = bias; a.residual = residual; a.out = out; a.rows_read = rows_read;
    a.partial = partial; a.counters = counters;
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
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
