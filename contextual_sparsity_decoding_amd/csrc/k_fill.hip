// Seeded normal samples written straight into device memory, so that
// synthetic stacks of 100+ GB never pass through host memory.
//
// The generator is Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011) with Box-Muller; include/dv.h
// states the exact mapping from (seed, stream, element) to a value.  One
// thread takes one Philox block of four elements.
#include "dv_internal.h"

#include <math.h>

namespace dv {

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
        const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
        const uint32_t n0 = hi1 ^ c[1] ^ k0;
        const uint32_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
    }
}

struct FillArgs {
    void* out;
    uint64_t n, offset;
    uint32_t k0, k1, s0, s1;
    double mean, stdv;
    int dtype;
};

__global__ __launch_bounds__(kBlock) void k_fill_normal(FillArgs a) {
    const uint64_t b0 = a.offset >> 2, b1 = (a.offset + a.n + 3) >> 2;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t b = b0 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; b < b1; b += step) {
        uint32_t x[4] = {(uint32_t)b, (uint32_t)(b >> 32), a.s0, a.s1};
        philox4x32_10(x, a.k0, a.k1);
        const uint64_t i0 = b * 4;
        const bool whole = i0 >= a.offset && i0 + 4 <= a.offset + a.n;
        if (a.dtype == 2) {                         // raw words
            uint32_t* o = (uint32_t*)a.out;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint64_t i = i0 + j;
                if (i >= a.offset && i < a.offset + a.n) o[i - a.offset] = x[j];
            }
            continue;
        }
        float f[4];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const double u = ((double)x[2 * p] + 1.0) * (1.0 / 4294967296.0);
            const double v = (double)x[2 * p + 1] * (1.0 / 4294967296.0);
            const double r = sqrt(-2.0 * log(u));
            const double t = 6.283185307179586 * v;
            f[2 * p] = (float)(a.mean + a.stdv * (r * cos(t)));
            f[2 * p + 1] = (float)(a.mean + a.stdv * (r * sin(t)));
        }
        const uint64_t o0 = i0 - a.offset;          // meaningful when whole
        if (a.dtype == DV_F16) {
            half_t* o = (half_t*)a.out;
            if (whole && (o0 & 3) == 0) {
                typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
                *reinterpret_cast<f16x4*>(o + o0) = f16x4{(half_t)f[0], (half_t)f[1], (half_t)f[2], (half_t)f[3]};
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint64_t i = i0 + j;
                    if (i >= a.offset && i < a.offset + a.n) o[i - a.offset] = (half_t)f[j];
                }
            }
        } else {
            float* o = (float*)a.out;
            if (whole && (o0 & 3) == 0) {
                *reinterpret_cast<f32x4*>(o + o0) = f32x4{f[0], f[1], f[2], f[3]};
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint64_t i = i0 + j;
                    if (i >= a.offset && i < a.offset + a.n) o[i - a.offset] = f[j];
                }
            }
        }
    }
}

}  // namespace dv

namespace dvh {
using namespace dv;

dv_status launch_fill_normal(void* out, uint64_t n, int dtype, uint64_t seed, uint64_t stream, uint64_t offset,
                             float mean, float stdv, hipStream_t s) {
    if (n == 0) return DV_OK;
    FillArgs a;
    a.out = out; a.n = n; a.offset = offset; a.dtype = dtype;
    a.k0 = (uint32_t)seed; a.k1 = (uint32_t)(seed >> 32);
    a.s0 = (uint32_t)stream; a.s1 = (uint32_t)(stream >> 32);
    a.mean = (double)mean; a.stdv = (double)stdv;
    const uint64_t blocks = ((offset + n + 3) >> 2) - (offset >> 2);
    const uint64_t want = (blocks + kBlock - 1) / kBlock;
    const int grid = (int)(want < 65536 ? want : 65536);   // grid-stride past 16.7M blocks of four
    hipLaunchKernelGGL(k_fill_normal, dim3(grid), dim3(kBlock), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
