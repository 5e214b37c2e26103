// Top-k selection and batch union.
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157).  §2.3 defines the selected sets S_M and
// S_A under a size budget; §5.2 and App. C.1 take their union over a batch.
// The pages do not describe the selection kernel; this one is exact:
//
//   order:  score descending, ties to the lower index, NaN after numbers.
//   method: radix select on order-preserving uint32 keys, 12, 12 and 8 bits
//           per pass (stopping once a bin is taken whole), finds the k-th
//           key T and how many keys equal to T to take; then one ordered
//           compaction (block prefix sums over contiguous index ranges per
//           thread) writes the set in ascending index order.
#include "dv_internal.h"

#include <type_traits>

namespace dv {

// Digit search over a filled histogram of nb bins: the digit whose bin
// holds the krem-th largest candidate (bins scanned from the top, 4 per
// thread).  *above = candidates in higher bins, *inbin = in the chosen bin.
// Each thread zeroes the bins it read, ready for the next pass (the
// barriers inside order that before any later histogram update).
__device__ __forceinline__ unsigned find_digit(unsigned* hist, int nb, unsigned krem, unsigned* tot,
                                               unsigned* sh, unsigned* above, unsigned* inbin) {
    unsigned c[4], local = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = 4 * (int)threadIdx.x + i;
        c[i] = p < nb ? hist[nb - 1 - p] : 0u;
        if (p < nb) hist[nb - 1 - p] = 0u;
        local += c[i];
    }
    unsigned total;
    unsigned run = block_excl_scan(local, tot, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = 4 * (int)threadIdx.x + i;
        if (p < nb && run < krem && run + c[i] >= krem) {
            sh[0] = (unsigned)(nb - 1 - p);
            sh[1] = run;
            sh[2] = c[i];
        }
        run += c[i];
    }
    __syncthreads();
    const unsigned d = sh[0];
    *above = sh[1];
    *inbin = sh[2];
    __syncthreads();
    return d;
}

// Add the valid keys (slot < lim) whose masked high bits equal `prefix` to
// the histogram of digit (key >> shift) & dmask.  After the first pass few
// keys are candidates, and a wave with none skips the update.
template <int E>
__device__ __forceinline__ void hist_keys(const uint32_t (&key)[E], int lim, uint32_t prefix, uint32_t pmask,
                                          int shift, uint32_t dmask, unsigned* hist) {
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (((key[e] & pmask) == prefix) && e < lim) atomicAdd(&hist[(key[e] >> shift) & dmask], 1u);
}

// Exact top-k of one row (row = blockIdx.x) by 1024 threads.  Thread t
// holds the E consecutive elements [i0, i0 + E) of each tile of 1024*E
// elements; keys stay in registers when the row is one tile, else every
// pass re-reads its tiles (the row is L2-resident).  Radix passes of 12,
// 12 and 8 bits over order keys find the k-th key; a pass stops the search
// early when every candidate left in its bin is needed.  The selected
// indices are written ascending by an ordered prefix sum over threads.
template <int E>
__device__ __forceinline__ void load_keys(const float* __restrict__ s, int n, int i0, bool vec, uint32_t (&key)[E]) {
    if (vec && i0 + E <= n) {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(s + i0 + e);
            key[e] = order_key(v[0]); key[e + 1] = order_key(v[1]);
            key[e + 2] = order_key(v[2]); key[e + 3] = order_key(v[3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) key[e] = i0 + e < n ? order_key(s[i0 + e]) : 0u;
    }
}

template <int E>
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ scores, int n, int k,
                                               int32_t* __restrict__ idx) {
    __shared__ unsigned hist[4096];
    __shared__ int32_t stage[kTopkStage];
    __shared__ unsigned tot[17];
    __shared__ unsigned sh[3];
    static_assert(E % 4 == 0, "E is a multiple of 4");
    const float* s = scores + (size_t)blockIdx.x * n;
    int32_t* out = idx + (size_t)blockIdx.x * k;
    const int tile = 1024 * E;
    const int ntile = (n + tile - 1) / tile;
    const bool vec = (n & 3) == 0 && ((uintptr_t)s & 15u) == 0;
    uint32_t key[E];
    if (ntile == 1) load_keys<E>(s, n, (int)threadIdx.x * E, vec, key);
    for (int i = threadIdx.x; i < 4096; i += blockDim.x) hist[i] = 0u;   // while the loads fly

    unsigned krem = (unsigned)k;
    uint32_t prefix = 0u, pmask = 0u;
    bool done = false;
    for (int ps = 0; ps < 3 && !done; ++ps) {
        const int shift = ps == 0 ? 20 : ps == 1 ? 8 : 0;
        const int nb = ps < 2 ? 4096 : 256;
        const uint32_t dmask = (uint32_t)nb - 1u;
        if (ps == 0) __syncthreads();       // the initial clear
        if (ntile == 1) {
            hist_keys<E>(key, min(E, n - (int)threadIdx.x * E), prefix, pmask, shift, dmask, hist);
        } else {
            for (int t = 0; t < ntile; ++t) {
                const int i0 = t * tile + (int)threadIdx.x * E;
                uint32_t kt[E];
                load_keys<E>(s, n, i0, vec, kt);
                hist_keys<E>(kt, min(E, n - i0), prefix, pmask, shift, dmask, hist);
            }
        }
        __syncthreads();
        unsigned above, inbin;
        const unsigned d = find_digit(hist, nb, krem, tot, sh, &above, &inbin);
        prefix |= d << shift;
        pmask |= dmask << shift;
        krem -= above;
        done = inbin == krem;               // every candidate left in the bin is taken
    }

    // ---- selection: keys above the threshold prefix (the whole last bin
    // after an early stop), then the first krem keys equal to the full
    // threshold in index order.  Tiles are written in order, through LDS
    // when the set fits so that the global writes are contiguous.
    const bool staged = k <= kTopkStage;
    unsigned base = 0u, eq_seen = 0u;
    for (int t = 0; t < ntile; ++t) {
        const int i0 = t * tile + (int)threadIdx.x * E;
        uint32_t kt[E];
        if (ntile == 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) kt[e] = key[e];
        } else {
            load_keys<E>(s, n, i0, vec, kt);
        }
        const int lim = min(E, n - i0);
        unsigned gt = 0u, eq = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t mk = kt[e] & pmask;
            const unsigned v = e < lim;
            gt += v & (mk > prefix || (done && mk == prefix));
            eq += v & (!done && kt[e] == prefix);
        }
        unsigned tsum;
        unsigned take_eq = 0u;
        if (!done) {
            unsigned eq_tot;
            const unsigned eq_before = eq_seen + block_excl_scan(eq, tot, &eq_tot);
            take_eq = krem > eq_before ? min(eq, krem - eq_before) : 0u;
            eq_seen += eq_tot;
        }
        unsigned pos = base + block_excl_scan(gt + take_eq, tot, &tsum);
        base += tsum;
        unsigned taken = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t mk = kt[e] & pmask;
            bool sel = e < lim && (mk > prefix || (done && mk == prefix));
            if (!done && e < lim && kt[e] == prefix) sel = taken++ < take_eq;
            if (sel) {
                if (pos < (unsigned)k) {
                    if (staged) stage[pos] = i0 + e;
                    else out[pos] = i0 + e;
                }
                ++pos;
            }
        }
    }
    if (staged) {
        __syncthreads();
        for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = stage[i];
    }
}

// The same selection for a row of one tile (n <= 1024 * E, E <= 32), with
// fewer instructions per element: per-thread bit masks (bit e = element
// i0 + e) for candidates and for the selection, so each pass costs a
// compare or two per element.  The first pass, where every key counts,
// spreads each bin over 4 copies (lane & 3) so that equal digits within a
// wave instruction rarely update the same LDS word.
template <typename M>
__device__ __forceinline__ unsigned popc_mask(M m) {
    if constexpr (sizeof(M) == 8) return (unsigned)__popcll(m);
    else return (unsigned)__popc(m);
}

template <int E>
__global__ __launch_bounds__(1024) void k_topk_tile(const float* __restrict__ scores, int n, int k,
                                                    int32_t* __restrict__ idx) {
    static_assert(E % 4 == 0 && E <= 64, "E in 4..64");
    using M = typename std::conditional<(E > 32), unsigned long long, unsigned>::type;   // bit e = element i0 + e
    __shared__ unsigned hist[4096 * 4];
    __shared__ int32_t stage[kTopkStage];
    __shared__ unsigned tot[17];
    __shared__ unsigned sh[3];
    const int tid = threadIdx.x, lane = tid & 63;
    const float* s = scores + (size_t)blockIdx.x * n;
    int32_t* out = idx + (size_t)blockIdx.x * k;
    const int i0 = tid * E;
    const int lim = max(0, min(E, n - i0));
    const M vmask = lim >= (int)(8 * sizeof(M)) ? ~(M)0 : ((M)1 << lim) - (M)1;
    const bool vec = (n & 3) == 0 && ((uintptr_t)s & 15u) == 0;
    uint32_t key[E];
    load_keys<E>(s, n, i0, vec, key);
    for (int i = tid; i < 4096; i += 1024) reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    // ---- pass 0: top 12 bits of every valid key, 4 copies per bin
    if (lim == E) {
#pragma unroll
        for (int e = 0; e < E; ++e) atomicAdd(&hist[(key[e] >> 20) * 4 + (lane & 3)], 1u);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (e < lim) atomicAdd(&hist[(key[e] >> 20) * 4 + (lane & 3)], 1u);
    }
    __syncthreads();
    unsigned krem = (unsigned)k;
    uint32_t prefix, pmask = 0xfff00000u;
    bool done;
    {
        // digit search over the summed copies (bins read and cleared 4 per thread)
        unsigned c[4], local = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bin = 4095 - (4 * tid + i);
            u32x4 v = reinterpret_cast<u32x4*>(hist)[bin];
            reinterpret_cast<u32x4*>(hist)[bin] = u32x4{0u, 0u, 0u, 0u};
            c[i] = v[0] + v[1] + v[2] + v[3];
            local += c[i];
        }
        unsigned total;
        unsigned run = block_excl_scan(local, tot, &total);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (run < krem && run + c[i] >= krem) {
                sh[0] = (unsigned)(4095 - (4 * tid + i));
                sh[1] = run;
                sh[2] = c[i];
            }
            run += c[i];
        }
        __syncthreads();
        prefix = sh[0] << 20;
        krem -= sh[1];
        done = sh[2] == krem;
        __syncthreads();
    }
    // ---- passes 1 and 2 over the candidates left in the chosen bin
    for (int ps = 1; ps < 3 && !done; ++ps) {
        const int shift = ps == 1 ? 8 : 0;
        const int nb = ps == 1 ? 4096 : 256;
        const uint32_t dmask = (uint32_t)nb - 1u;
        M cm = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) cm |= (M)((key[e] & pmask) == prefix) << e;
        cm &= vmask;
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (cm & ((M)1 << e)) atomicAdd(&hist[(key[e] >> shift) & dmask], 1u);
        __syncthreads();
        unsigned above, inbin;
        const unsigned d = find_digit(hist, nb, krem, tot, sh, &above, &inbin);
        prefix |= d << shift;
        pmask |= dmask << shift;
        krem -= above;
        done = inbin == krem;
    }

    // ---- selection mask: keys above the threshold prefix (the whole last
    // bin after an early stop), then the first krem keys equal to the full
    // threshold in index order
    M sel = 0, eqm = 0;
    if (done) {
#pragma unroll
        for (int e = 0; e < E; ++e) sel |= (M)((key[e] & pmask) >= prefix) << e;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            sel |= (M)(key[e] > prefix) << e;
            eqm |= (M)(key[e] == prefix) << e;
        }
    }
    sel &= vmask;
    eqm &= vmask;
    if (!done) {                                   // ties at the threshold: lowest indices first
        unsigned eq_tot;
        const unsigned eq_before = block_excl_scan(popc_mask(eqm), tot, &eq_tot);
        unsigned take = krem > eq_before ? min(popc_mask(eqm), krem - eq_before) : 0u;
        for (M m = eqm; take > 0; --take) {
            const M low = m & ((M)0 - m);
            sel |= low;
            m ^= low;
        }
    }
    const bool staged = k <= kTopkStage;
    unsigned tsum;
    unsigned pos = block_excl_scan(popc_mask(sel), tot, &tsum);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (sel & ((M)1 << e)) {
            if (pos < (unsigned)k) {
                if (staged) stage[pos] = i0 + e;
                else out[pos] = i0 + e;
            }
            ++pos;
        }
    }
    if (staged) {
        __syncthreads();
        for (int i = tid; i < k; i += 1024) out[i] = stage[i];
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
    if (sel && pos < (unsigned)k) idx[(size_t)blockIdx.x * k + pos] = i;
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
    // Coalesced loads of 4 consecutive entries a lane (a wave covers 256
    // entries an instruction, 8 instructions in flight): a set is ascending,
    // so a lane's 4 entries usually share one word and leave as one OR.
    // (A lane reading 32 consecutive entries of its own sent each load
    // instruction to 64 lines, which one compute unit serves a line a cycle.)
    constexpr int U = 8;
    const int nwv = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool vec = ((uintptr_t)idx & 15u) == 0;
    for (int base = wv * U * kWave * 4; base < total_in; base += nwv * U * kWave * 4) {
        int j[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e0 = base + (u * kWave + lane) * 4;
            if (vec && e0 + 4 <= total_in) {
                const int4 v = *reinterpret_cast<const int4*>(idx + e0);
                j[u][0] = v.x; j[u][1] = v.y; j[u][2] = v.z; j[u][3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) j[u][e] = e0 + e < total_in ? idx[e0 + e] : -1;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int cw = -1;
            unsigned acc = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = j[u][e];
                if ((unsigned)q >= (unsigned)n) continue;   // past the entries, or outside [0, n)
                if ((q >> 5) != cw) {
                    if (acc) atomicOr(&bits[cw], acc);
                    cw = q >> 5;
                    acc = 0u;
                }
                acc |= 1u << (q & 31);
            }
            if (acc) atomicOr(&bits[cw], acc);
        }
    }
    __syncthreads();
    // The rank of each word's first bit, then every bit position q in turn:
    // lane-consecutive positions write consecutive ranks, so the stores
    // coalesce (a thread writing its own words' runs sent a wave's 64
    // stores to 64 lines).  Ranks are kept in 16 bits (pre) beside the full
    // rank of each 256-word block's first word (brank), which is less than
    // 8192 below any rank in its block.
    unsigned* brank = bits + nw;
    unsigned short* pre = reinterpret_cast<unsigned short*>(brank + (nw + 255) / 256);
    const int W = (nw + blockDim.x - 1) / blockDim.x;
    const int w0 = threadIdx.x * W;
    unsigned cnt = 0;
    for (int w = w0; w < min(nw, w0 + W); ++w) cnt += __popc(bits[w]);
    unsigned total;
    unsigned run = block_excl_scan(cnt, tot, &total);
    for (int w = w0; w < min(nw, w0 + W); ++w) {
        pre[w] = (unsigned short)(run & 0xffffu);
        if ((w & 255) == 0) brank[w >> 8] = run;
        run += __popc(bits[w]);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n; q += blockDim.x) {
        const int w = q >> 5;
        const unsigned m = bits[w];
        if ((m >> (q & 31)) & 1u) {
            const unsigned b0 = brank[w >> 8];
            const unsigned r = b0 + ((pre[w] - b0) & 0xffffu) + __popc(m & ((1u << (q & 31)) - 1u));
            uidx[r] = q;
        }
    }
    if (threadIdx.x == 0 && ucount) *ucount = (int32_t)min(total, (unsigned)n);
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
    const int E = cdiv(n, 1024);     // elements per thread when the row is one tile
#define DV_TK(EE) hipLaunchKernelGGL((k_topk_tile<EE>), dim3(B), dim3(1024), 0, s, scores, n, k, idx)
    if (E <= 4) DV_TK(4);
    else if (E <= 8) DV_TK(8);
    else if (E <= 12) DV_TK(12);
    else if (E <= 16) DV_TK(16);
    else if (E <= 20) DV_TK(20);
    else if (E <= 24) DV_TK(24);
    else if (E <= 32) DV_TK(32);
    else if (E <= 40) DV_TK(40);
    else if (E <= 48) DV_TK(48);
    else if (E <= 56) DV_TK(56);
    else if (E <= 64) DV_TK(64);
    else hipLaunchKernelGGL((k_topk<16>), dim3(B), dim3(1024), 0, s, scores, n, k, idx);   // tiles of 16384
#undef DV_TK
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DV_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return DV_OK;
}

dv_status launch_union(const int32_t* idx, int B, int k, int n, int32_t* union_idx, int32_t* union_count,
                       hipStream_t s) {
    const size_t nw = (size_t)(n + 31) / 32;
    const size_t lds = nw * sizeof(unsigned) + (nw + 255) / 256 * sizeof(unsigned) + nw * sizeof(unsigned short);
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
