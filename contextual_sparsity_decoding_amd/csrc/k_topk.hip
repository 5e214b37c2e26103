// Top-k selection and batch union.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).  §2.3 defines the selected sets S_M and
// S_A under a size budget; §5.2 and App. C.1 take their union over a batch.
// The pages do not describe the selection kernel; this one is exact:
//
//   order:  score descending, ties to the lower index, NaN after numbers.
//   method: radix select on order-preserving uint32 keys, 8 bits per pass,
//           finds the k-th key T and how many keys equal to T to take; then
//           one ordered compaction (block prefix sums over contiguous index
//           ranges per thread) writes the set in ascending index order.
#include "dv_internal.h"

namespace dv {

__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum over the block (<= 1024 threads); *total gets the sum.
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* tot /* >= 17 */, unsigned* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const unsigned incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) tot[w] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned run = 0;
        for (int i = 0; i < nw; ++i) {
            const unsigned t = tot[i];
            tot[i] = run;
            run += t;
        }
        tot[16] = run;
    }
    __syncthreads();
    const unsigned r = tot[w] + incl - v;
    *total = tot[16];
    __syncthreads();
    return r;
}

template <int EMAX>
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ scores, int n, int k,
                                               int32_t* __restrict__ idx) {
    __shared__ unsigned hist[256];
    __shared__ unsigned tot[17];
    __shared__ unsigned sh_digit, sh_above;
    const float* s = scores + (size_t)blockIdx.x * n;
    int32_t* out = idx + (size_t)blockIdx.x * k;
    const int nt = blockDim.x, tid = threadIdx.x;
    const int E = (n + nt - 1) / nt;
    const int i0 = tid * E;
    uint32_t key[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) key[e] = (e < E && i0 + e < n) ? order_key(s[i0 + e]) : 0u;

    uint32_t prefix = 0u, pmask = 0u;
    unsigned krem = (unsigned)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += nt) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E && i0 + e < n && (key[e] & pmask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
        __syncthreads();
        // digits in descending order: position t holds digit 255 - t
        unsigned c = 0u, incl = 0u;
        if (tid < 256) {
            c = hist[255 - tid];
            incl = wave_incl_scan(c);
            if ((tid & 63) == 63) tot[tid >> 6] = incl;
        }
        __syncthreads();
        if (tid < 256) {
            for (int w = 0; w < (tid >> 6); ++w) incl += tot[w];
            if (incl >= krem && incl - c < krem) {
                sh_digit = 255u - tid;
                sh_above = incl - c;
            }
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        pmask |= 255u << shift;
        krem -= sh_above;
        __syncthreads();
    }
    // prefix is the k-th largest key; take every key above it and the first
    // krem keys equal to it in index order.
    unsigned gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        if (e < E && i0 + e < n) {
            gt += key[e] > prefix;
            eq += key[e] == prefix;
        }
    }
    unsigned total;
    const unsigned eq_before = block_excl_scan(eq, tot, &total);
    const unsigned take_eq = krem > eq_before ? min(eq, krem - eq_before) : 0u;
    unsigned pos = block_excl_scan(gt + take_eq, tot, &total);
    unsigned taken = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        if (e < E && i0 + e < n) {
            const bool sel = key[e] > prefix || (key[e] == prefix && taken++ < take_eq);
            if (sel && pos < (unsigned)k) out[pos++] = i0 + e;
        }
    }
}

// U = union of the B index sets (each ascending, values < n), written
// ascending, with its size.
__global__ __launch_bounds__(1024) void k_union(const int32_t* __restrict__ idx, int total_in, int n,
                                                int32_t* __restrict__ uidx, int32_t* __restrict__ ucount) {
    extern __shared__ unsigned bits[];
    __shared__ unsigned tot[17];
    const int nw = (n + 31) >> 5;
    for (int i = threadIdx.x; i < nw; i += blockDim.x) bits[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < total_in; i += blockDim.x) {
        const int j = idx[i];
        if ((unsigned)j < (unsigned)n) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    const int W = (nw + blockDim.x - 1) / blockDim.x;
    const int w0 = threadIdx.x * W;
    unsigned cnt = 0;
    for (int w = w0; w < min(nw, w0 + W); ++w) cnt += __popc(bits[w]);
    unsigned total;
    unsigned pos = block_excl_scan(cnt, tot, &total);
    for (int w = w0; w < min(nw, w0 + W); ++w) {
        unsigned m = bits[w];
        while (m) {
            const int b = __ffs(m) - 1;
            uidx[pos++] = w * 32 + b;
            m &= m - 1;
        }
    }
    if (threadIdx.x == 0 && ucount) *ucount = (int32_t)total;
}

__global__ void k_set_i32(int32_t* p, int v) { *p = v; }

}  // namespace dv

namespace dvh {
using namespace dv;

int topk_block_threads(int n) {
    int t = 256;                     // the digit scan needs one thread per digit
    while (t < 1024 && t * 16 < n) t *= 2;
    return t;
}

dv_status launch_topk(const float* scores, int B, int n, int k, int32_t* idx, hipStream_t s) {
    if (k == 0 || n == 0) return DV_OK;
    const int nt = topk_block_threads(n);
    const int E = cdiv(n, nt);
    if (E <= 16)
        hipLaunchKernelGGL((k_topk<16>), dim3(B), dim3(nt), 0, s, scores, n, k, idx);
    else if (E <= 32)
        hipLaunchKernelGGL((k_topk<32>), dim3(B), dim3(nt), 0, s, scores, n, k, idx);
    else if (E <= 48)
        hipLaunchKernelGGL((k_topk<48>), dim3(B), dim3(nt), 0, s, scores, n, k, idx);
    else
        hipLaunchKernelGGL((k_topk<64>), dim3(B), dim3(nt), 0, s, scores, n, k, idx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

dv_status launch_union(const int32_t* idx, int B, int k, int n, int32_t* union_idx, int32_t* union_count,
                       hipStream_t s) {
    const size_t lds = (size_t)((n + 31) / 32) * sizeof(unsigned);
    hipLaunchKernelGGL(k_union, dim3(1), dim3(1024), lds, s, idx, B * k, n, union_idx, union_count);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

dv_status launch_set_i32(int32_t* p, int v, hipStream_t s) {
    hipLaunchKernelGGL(k_set_i32, dim3(1), dim3(1), 0, s, p, v);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

}  // namespace dvh
