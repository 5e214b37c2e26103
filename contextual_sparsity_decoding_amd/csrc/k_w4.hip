// 4-bit weights (W4A16) in the sparse MLP: the group-wise int4 quantizer,
// fc1 over selected rows and the fc2 gather-AXPY, dequantizing inside the
// gather.  DejaVu §5 (Compatibility with Quantization, Table 7) combines
// 4-bit weights with contextual sparsity; the pages do not give the
// quantizer, so the format is defined in include/dv.h (dv_quantize_w4):
// per row, groups of 128 entries, an fp16 scale s per group and codes
// v in [-8, 7] stored as nibbles v + 8, entry c of a row in byte c / 2
// (low nibble for even c).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).
#include "rowdot.h"
#include "w4.h"

namespace dv {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));


constexpr int kW4Group = 128;
constexpr int kW4Chunk = 32;            // codes in a 16-byte chunk (fc1)
constexpr int kW4Half = 16;             // codes in an 8-byte chunk (fc2)

// The 8 codes of a 32-bit word as the unsigned nibbles v + 8, in order:
// byte j of `lo` holds code 2j, byte j of `hi` code 2j + 1.  Each is
// turned into a float by one byte conversion; the offset 8 is taken out of
// the sums once (sum of c * (n - 8) = sum of c * n - 8 * sum of c).
__device__ __forceinline__ void w4_word(unsigned w, float (&f)[8]) {
    const unsigned lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = (float)((lo >> (8 * j)) & 0xFFu);
        f[2 * j + 1] = (float)((hi >> (8 * j)) & 0xFFu);
    }
}

// One thread per group of 128: the largest magnitude, the scale, then the
// codes (the group is read twice; the second read comes from the cache).
__global__ __launch_bounds__(kBlock) void k_quant_w4(const half_t* __restrict__ w, int rows, int cols,
                                                     uint8_t* __restrict__ q, half_t* __restrict__ s) {
    const int gpr = cols / kW4Group;
    const long g = (long)blockIdx.x * kBlock + threadIdx.x;
    if (g >= (long)rows * gpr) return;
    const long r = g / gpr;
    const int gi = (int)(g % gpr);
    const half_t* src = w + r * cols + (size_t)gi * kW4Group;
    float m = 0.f;
    for (int i = 0; i < kW4Group / 8; ++i) {
        float f[8];
        unpack(ld16(src + 8 * i), f, half_t());
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
    }
    const half_t s16 = (half_t)__fdiv_rn(m, 7.f);
    const float sf = (float)s16;
    uint8_t* dst = q + r * (cols / 2) + (size_t)gi * (kW4Group / 2);
    for (int i = 0; i < kW4Group / 32; ++i) {          // 32 codes -> 16 bytes
        u32x4 out;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            float f[8];
            unpack(ld16(src + 32 * i + 8 * wd), f, half_t());
            unsigned word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = sf > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(f[e], sf)), -8.f), 7.f) : 0.f;
                word |= (unsigned)((int)v + 8) << (4 * e);
            }
            out[wd] = word;
        }
        *reinterpret_cast<u32x4*>(dst + 16 * i) = out;
    }
    s[r * gpr + gi] = s16;
}

// fc1 over the selected rows, batch of one: a[u] = max(0, y . w'[idx[u]] + b1).
// Each wave takes R rows; lane l holds chunks l, l+64, ... (32 codes each,
// one scale: 32 divides 128).  y sits in LDS transposed, float4 k of chunk
// c at [k][c], so that for each k the lanes read consecutive 16 bytes.  A
// chunk's sum over its codes is taken first, less 8 times its inputs' sum
// (computed once per chunk for all the wave's rows), then scaled.
template <int CH, int R>
__global__ __launch_bounds__(kBlock) void k_rowdot_w4(W4RowArgs a) {
    extern __shared__ float ys[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int n = a.n_dev ? min(*a.n_dev, a.n_max) : a.n_max;
    const int u0 = (blockIdx.x * 4 + wv) * R;
    const int nchunk = a.d / kW4Chunk, rb = a.d / 2, sb = a.d / kW4Group;
    int j[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int u = u0 + r;
        int jj = -1;
        if (u < n) {
            jj = a.idx ? a.idx[u] : u;
            jj = (unsigned)jj < (unsigned)a.w_rows ? jj : -1;
        }
        j[r] = __builtin_amdgcn_readfirstlane(jj);
    }
    // Loads retire in issue order: y goes out first (into registers, on its
    // way to LDS), then the codes and the scales, so that staging y waits
    // for y only.  Every lane loads (one past the row, or of a row not
    // selected, reads row 0 and its scale is masked to 0), and the scales
    // are kept as stored and converted where they are used: a load under a
    // lane mask, or a conversion next to its load, would make that wait
    // cover every load before it.
    constexpr int KY = CH * kW4Chunk / 4 * kWave / kBlock;   // float4 of y per thread (d <= CH * 2048)
    f32x4 yr[KY];
    {
        const f32x4* y4 = reinterpret_cast<const f32x4*>(a.y);
#pragma unroll
        for (int k = 0; k < KY; ++k) {
            const int i = threadIdx.x + k * kBlock;
            yr[k] = i < a.d / 4 ? y4[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    u32x4 w[R][CH];
    unsigned scr[R][CH];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int c = lane + i * kWave;
            const size_t jr = (size_t)(j[r] >= 0 ? j[r] : 0), cc = (size_t)(c < nchunk ? c : 0);
            w[r][i] = ld16_stream(a.q + jr * rb + cc * 16);
            scr[r][i] = elt_bits(a.s + jr * sb + cc / 4);
        }
    {   // y into LDS, transposed
        f32x4* l4 = reinterpret_cast<f32x4*>(ys);
#pragma unroll
        for (int k = 0; k < KY; ++k) {
            const int i = threadIdx.x + k * kBlock;
            if (i < a.d / 4) l4[(i & 7) * nchunk + (i >> 3)] = yr[k];
        }
    }
    __syncthreads();
    const f32x4* l4 = reinterpret_cast<const f32x4*>(ys);
    float ysum[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        float t = 0.f;
        if (c < nchunk)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f32x4 v = l4[k * nchunk + c];
                t += (v[0] + v[1]) + (v[2] + v[3]);
            }
        ysum[i] = t;
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + i * kWave;
        if (c < nchunk) {
            float p[R];
#pragma unroll
            for (int r = 0; r < R; ++r) p[r] = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 ya = l4[(2 * m) * nchunk + c], yb = l4[(2 * m + 1) * nchunk + c];
                const float yv[8] = {ya[0], ya[1], ya[2], ya[3], yb[0], yb[1], yb[2], yb[3]};
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float f[8];
                    w4_word(w[r][i][m], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) p[r] = fmaf(f[e], yv[e], p[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = fmaf(p[r] - 8.f * ysum[i], j[r] >= 0 ? bits_f32<half_t>(scr[r][i]) : 0.f, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int u = u0 + r;
        float v = wave_sum(acc[r]);
        const float bj = j[r] >= 0 ? (float)a.bias[j[r]] : 0.f;
        v = j[r] >= 0 ? fmaxf(v + bj, 0.f) : 0.f;
        if (lane == 0 && u < n) a.out[u] = v;
    }
}

// fc2 gather-AXPY, batch of one: partial[g] = sum over the live rows of
// group g (64 selected rows) of a[u] * w'[idx[u]] restricted to one slice
// of 1024 columns (lane l: columns [16 l, 16 l + 16) of the slice, 8 bytes
// of codes per row, one scale).  Rows whose coefficient is zero are
// skipped when asked (the ReLU-sparsified second layer); the 4 waves' sums
// are added in order in LDS and written as the group's partial, which
// k_axpy_finalize adds up.
constexpr int kW4Rows = 64;
__global__ __launch_bounds__(kBlock) void k_axpy_w4(W4AxpyArgs a) {
    __shared__ int s_row[kW4Rows];
    __shared__ float s_cf[kW4Rows];
    __shared__ unsigned s_n;
    __shared__ f32x4 red[3][4][kWave];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int slice = blockIdx.x, g = blockIdx.y;
    const int rows = a.n_rows_dev ? min(*a.n_rows_dev, a.rows) : a.rows;
    const int r0 = g * kW4Rows;
    const int c = slice * kWave + lane;                // this lane's 8-byte chunk of the row
    const int nchunk = a.d / kW4Half, rb = a.d / 2, sb = a.d / kW4Group;
    const bool colok = c < nchunk;
    if (threadIdx.x < kWave) {
        bool live = false;
        int row = 0;
        float cf = 0.f;
        const int u = r0 + threadIdx.x;
        if (u < rows) {
            row = a.idx ? a.idx[u] : u;
            cf = a.coef[u];
            live = (unsigned)row < (unsigned)a.w_rows && (cf != 0.f || !a.skip_zero);
        }
        const unsigned lv = live ? 1u : 0u;
        const unsigned incl = wave_incl_scan(lv);
        if (live) {
            s_row[incl - 1] = row;
            s_cf[incl - 1] = cf;
        }
        if (threadIdx.x == 63) {
            s_n = incl;
            if (a.rows_read && slice == 0 && incl > 0) atomicAdd(a.rows_read, (int)incl);
        }
    }
    __syncthreads();
    const int nlive = (int)s_n;
    constexpr int U = kW4Rows / 4;                     // rows per wave
    // Every lane of a live row loads (one past the row's end reads the row's
    // first chunk; its scale is masked to 0), rows past the live ones are
    // neither loaded nor read, and the scales are kept as stored and
    // converted where they are used: a load under a lane mask, a value
    // merged with a constant, or a conversion next to its load would each
    // make a wait cover every load before it (one row at a time).
    unsigned w[U][2];
    unsigned scr[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
        const int k = wv + 4 * t;
        if (k < nlive) {                               // uniform over the wave
            const int rr = s_row[k];
            const size_t cc = (size_t)(colok ? c : 0);
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.q + (size_t)rr * rb + cc * 8));
            w[t][0] = v[0];
            w[t][1] = v[1];
            scr[t] = elt_bits(a.s + (size_t)rr * sb + cc / 8);
        }
    }
    float acc[kW4Half];
#pragma unroll
    for (int e = 0; e < kW4Half; ++e) acc[e] = 0.f;
    float csum = 0.f;
#pragma unroll
    for (int t = 0; t < U; ++t) {
        const int k = wv + 4 * t;
        if (k < nlive) {
            const float cs = s_cf[k] * (colok ? bits_f32<half_t>(scr[t]) : 0.f);
            csum += cs;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float f[8];
                w4_word(w[t][m], f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[8 * m + e] = fmaf(cs, f[e], acc[8 * m + e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < kW4Half; ++e) acc[e] = fmaf(-8.f, csum, acc[e]);
    // waves 1..3 hand their sums to wave 0, which adds them in order
    if (wv > 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            red[wv - 1][k][lane] = f32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
    }
    __syncthreads();
    if (wv == 0 && colok) {
        f32x4* dst = reinterpret_cast<f32x4*>(a.partial + (size_t)g * a.d + (size_t)c * kW4Half);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f32x4 o = f32x4{acc[4 * k], acc[4 * k + 1], acc[4 * k + 2], acc[4 * k + 3]};
#pragma unroll
            for (int q = 0; q < 3; ++q) o += red[q][k][lane];
            dst[k] = o;
        }
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

dv_status launch_quant_w4(const void* w, int rows, int cols, uint8_t* q, void* s, hipStream_t st) {
    const long groups = (long)rows * (cols / kW4Group);
    if (groups == 0) return DV_OK;
    hipLaunchKernelGGL(k_quant_w4, dim3((unsigned)((groups + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                       (const half_t*)w, rows, cols, q, (half_t*)s);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DV_OK : fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
}

int w4_chunks_per_lane(int d) { return cdiv(d / kW4Chunk, kWave); }

dv_status launch_rowdot_w4(const W4RowArgs& a, hipStream_t s) {
    constexpr int R = 2;
    const int grid = cdiv(a.n_max < 1 ? 1 : a.n_max, 4 * R);
    const size_t lds = (size_t)a.d * sizeof(float);
    switch (w4_chunks_per_lane(a.d)) {
#define DV_W4R(CH) case CH: DV_LAUNCH((k_rowdot_w4<CH, R>), dim3(grid), dim3(kBlock), lds, s, a); break;
        DV_W4R(1) DV_W4R(2) DV_W4R(3) DV_W4R(4) DV_W4R(5) DV_W4R(6) DV_W4R(7) DV_W4R(8)
#undef DV_W4R
        default: return fail(DV_ERR_UNSUPPORTED, "4-bit fc1: d=%d", a.d);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DV_OK : fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
}

int w4_axpy_groups(int rows) { return cdiv(rows < 1 ? 1 : rows, kW4Rows); }

dv_status launch_axpy_w4(const W4AxpyArgs& a, hipStream_t s) {
    const dim3 grid(cdiv(a.d / kW4Half, kWave), w4_axpy_groups(a.rows));
    DV_LAUNCH(k_axpy_w4, grid, dim3(kBlock), 0, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DV_OK : fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
}

}  // namespace dvh
