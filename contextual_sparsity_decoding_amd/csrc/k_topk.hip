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

__device__ __forceinline__ float key_value(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __builtin_bit_cast(float, u);
}

// Value-linear bin of a finite key: monotone in the score (the fp32
// subtraction, the product with a positive scale and the floor are all
// monotone), so equal scores share a bin and a larger score never falls in
// a lower bin.
__device__ __forceinline__ int value_bin(uint32_t k, float vmin, float scale) {
    const float t = (key_value(k) - vmin) * scale;
    const int b = (int)t;
    return b < 0 ? 0 : b > 4095 ? 4095 : b;
}

// Exact top-k of one row by a 4096-bin histogram pass over value-linear
// bins between the row's min and max, then radix passes of 12, 12 and 8 bits
// over the keys of the boundary bin only.  After any pass, when every
// candidate left in the chosen bin is needed, the selection is complete.
// Rows with NaN or infinite scores skip the value pass (plain key radix).
template <int EMAX>
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ scores, int n, int k,
                                               int32_t* __restrict__ idx) {
    constexpr int NBIN = 4096;
    __shared__ unsigned hist[NBIN];
    __shared__ unsigned tot[17];
    __shared__ uint32_t red_min[16], red_max[16];
    __shared__ unsigned red_nan[16];
    __shared__ unsigned sh_digit, sh_above, sh_bin;
    const float* s = scores + (size_t)blockIdx.x * n;
    int32_t* out = idx + (size_t)blockIdx.x * k;
    const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = (n + nt - 1) / nt;
    const int i0 = tid * E;
    uint32_t key[EMAX];
    if ((E & 3) == 0 && (n & 3) == 0 && ((uintptr_t)s & 15u) == 0) {   // contiguous float4 runs per thread
#pragma unroll
        for (int e = 0; e < EMAX; e += 4) {
            if (e < E && i0 + e < n) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(s + i0 + e);
                key[e] = order_key(v[0]); key[e + 1] = order_key(v[1]);
                key[e + 2] = order_key(v[2]); key[e + 3] = order_key(v[3]);
            } else {
                key[e] = key[e + 1] = key[e + 2] = key[e + 3] = 0u;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) key[e] = (e < E && i0 + e < n) ? order_key(s[i0 + e]) : 0u;
    }
    auto valid = [&](int e) { return e < E && i0 + e < n; };

    // ---- row statistics: NaN count (key 0), min and max key of the rest
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    unsigned nnan = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        if (valid(e)) {
            if (key[e] == 0u) {
                ++nnan;
            } else {
                kmin = min(kmin, key[e]);
                kmax = max(kmax, key[e]);
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, kWave));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, kWave));
        nnan += (unsigned)__shfl_xor((int)nnan, o, kWave);
    }
    if (lane == 0) {
        red_min[wv] = kmin;
        red_max[wv] = kmax;
        red_nan[wv] = nnan;
    }
    __syncthreads();
    kmin = 0xffffffffu; kmax = 0u; nnan = 0;
    for (int i = 0; i < (nt >> 6); ++i) {
        kmin = min(kmin, red_min[i]);
        kmax = max(kmax, red_max[i]);
        nnan += red_nan[i];
    }
    const float vmin = key_value(kmin), vmax = key_value(kmax);
    const bool binned = nnan == 0 && kmin <= kmax && isfinite(vmin) && isfinite(vmax) && isfinite(vmax - vmin);
    const float scale = (binned && vmax > vmin) ? (float)(NBIN - 1) / (vmax - vmin) : 0.f;

    unsigned krem = (unsigned)k;
    int bin_d = -1;                        // the boundary value bin (binned rows)
    bool early = false;
    if (binned) {
        for (int i = tid; i < NBIN; i += nt) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (valid(e)) atomicAdd(&hist[value_bin(key[e], vmin, scale)], 1u);
        __syncthreads();
        unsigned c[4], local = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * tid + i;
            c[i] = p < NBIN ? hist[NBIN - 1 - p] : 0u;
            local += c[i];
        }
        unsigned total;
        unsigned run = block_excl_scan(local, tot, &total);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * tid + i;
            if (p < NBIN && run < krem && run + c[i] >= krem) {
                sh_digit = (unsigned)(NBIN - 1 - p);
                sh_above = run;
                sh_bin = c[i];
            }
            run += c[i];
        }
        __syncthreads();
        bin_d = (int)sh_digit;
        krem -= sh_above;
        early = sh_bin == krem;
        __syncthreads();
    }
    auto cand = [&](int e) { return !binned || value_bin(key[e], vmin, scale) == bin_d; };
    auto above_bin = [&](int e) { return binned && value_bin(key[e], vmin, scale) > bin_d; };

    // ---- exact radix passes over the candidates
    uint32_t prefix = 0u, pmask = 0u;
    for (int ps = 0; ps < 3 && !early; ++ps) {
        const int shift = ps == 0 ? 20 : ps == 1 ? 8 : 0;
        const int nb = ps < 2 ? 4096 : 256;
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int i = tid; i < nb; i += nt) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (valid(e) && (key[e] & pmask) == prefix && cand(e)) atomicAdd(&hist[(key[e] >> shift) & dmask], 1u);
        __syncthreads();
        unsigned c[4], local = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * tid + i;
            c[i] = p < nb ? hist[nb - 1 - p] : 0u;
            local += c[i];
        }
        unsigned total;
        unsigned run = block_excl_scan(local, tot, &total);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * tid + i;
            if (p < nb && run < krem && run + c[i] >= krem) {
                sh_digit = (unsigned)(nb - 1 - p);
                sh_above = run;
                sh_bin = c[i];
            }
            run += c[i];
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        pmask |= dmask << shift;
        krem -= sh_above;
        early = sh_bin == krem;             // every candidate left in the bin is taken
        __syncthreads();
    }
    // ---- selection: elements above the boundary bin, then candidates above
    // the key threshold, then the first krem candidates equal to it in index
    // order (after an early stop every candidate in the last bin is taken).
    unsigned gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        if (valid(e)) {
            if (above_bin(e)) {
                ++gt;
            } else if (cand(e) && (key[e] & pmask) >= prefix) {
                if (early) ++gt;                                  // the whole chosen bin
                else if (key[e] > prefix) ++gt;
                else if (key[e] == prefix) ++eq;
            }
        }
    }
    unsigned total;
    const unsigned eq_before = block_excl_scan(eq, tot, &total);
    const unsigned take_eq = krem > eq_before ? min(eq, krem - eq_before) : 0u;
    unsigned pos = block_excl_scan(gt + (early ? 0u : take_eq), tot, &total);
    unsigned taken = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
        if (valid(e)) {
            bool sel = false;
            if (above_bin(e)) {
                sel = true;
            } else if (cand(e) && (key[e] & pmask) >= prefix) {
                if (early) sel = true;
                else if (key[e] > prefix) sel = true;
                else if (key[e] == prefix) sel = taken++ < take_eq;
            }
            if (sel && pos < (unsigned)k) out[pos++] = i0 + e;
        }
    }
}

// Small n (<= 256, e.g. heads): thread i holds element i; its rank is the
// number of elements before it in the order; rank < k selects it.
__global__ __launch_bounds__(256) void k_topk_small(const float* __restrict__ scores, int n, int k,
                                                    int32_t* __restrict__ idx) {
    __shared__ uint32_t keys[256];
    __shared__ unsigned tot[17];
    const int i = threadIdx.x;
    const float* s = scores + (size_t)blockIdx.x * n;
    const uint32_t ki = i < n ? order_key(s[i]) : 0u;
    keys[i] = ki;
    __syncthreads();
    unsigned rank = 0;
    for (int j = 0; j < n; ++j) {
        const uint32_t kj = keys[j];
        rank += (kj > ki) || (kj == ki && j < i);
    }
    const bool sel = i < n && rank < (unsigned)k;
    unsigned total;
    const unsigned pos = block_excl_scan(sel ? 1u : 0u, tot, &total);
    if (sel) idx[(size_t)blockIdx.x * k + pos] = i;
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
    (void)n;
    return 1024;                     // the 4096-bin digit scan: 4 bins per thread
}

dv_status launch_topk(const float* scores, int B, int n, int k, int32_t* idx, hipStream_t s) {
    if (k == 0 || n == 0) return DV_OK;
    if (n <= 256) {
        hipLaunchKernelGGL(k_topk_small, dim3(B), dim3(256), 0, s, scores, n, k, idx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return DV_OK;
    }
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
