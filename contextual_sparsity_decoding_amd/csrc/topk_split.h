// Top-k of one score row split into three roles, each a few 256-thread
// workgroups that ride in a launch doing other work; the launches between
// them order the roles.  Same selection as the top-k kernels (score
// descending, ties to the lower index, NaN after numbers; the set ascending).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §2.3 (the sets S_M under a budget)
// and §4.3 (the next layer's selection overlaps this layer's work).
//
//   1. topk_hist_slice, one workgroup per 1024 scores: the histogram of the
//      keys' top 12 bits, added into a global histogram (cleared earlier).
//   2. topk_threshold, one workgroup: the k-th key by radix select, the
//      first digit read off that histogram, the next 12 and 8 bits
//      histogrammed in LDS over the keys still in the running (stopping once
//      a bin is taken whole); it writes the threshold.
//   3. topk_emit_slice, one workgroup per 1024 scores: counts the selected
//      keys before its slice itself (the row is L2-resident), then writes
//      its slice's selected indices in order.
#pragma once

#include "dv_internal.h"

namespace dv {

constexpr int kTopkSlice = 1024;                // scores per slice (256 threads x 4)

// Keys k with (k & pmask) > prefix are selected; with done, also those with
// (k & pmask) == prefix; else pmask is all ones and the first krem keys equal
// to prefix, in index order, are selected too.
struct TopkThreshold {
    uint32_t prefix, pmask, krem, done;
};

__device__ __forceinline__ void topk_hist_slice(const float* __restrict__ s, int n, int slice, unsigned* lds,
                                                unsigned* __restrict__ ghist) {
    const int tid = threadIdx.x;
    const int i = slice * kTopkSlice + 4 * tid;
    const f32x4 v = i < n ? *reinterpret_cast<const f32x4*>(s + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int b = tid; b < 4096; b += 256) lds[b] = 0u;
    __syncthreads();
    if (i < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&lds[order_key(v[e]) >> 20], 1u);
    }
    __syncthreads();
    for (int b = tid; b < 4096; b += 256) {     // at most one global add per bin and slice
        const unsigned c = lds[b];
        if (c) atomicAdd(&ghist[b], c);
    }
}

// The digit whose bin holds the krem-th largest candidate; thread t holds
// the counts of bins nb-1-(P*t+i), i < P (scanning from the top).
template <int P>
__device__ __forceinline__ unsigned topk_pick(const unsigned (&c)[P], int nb, unsigned krem, unsigned* tot,
                                              unsigned* sh, unsigned* above, unsigned* inbin) {
    unsigned local = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) local += c[i];
    unsigned total;
    unsigned run = block_excl_scan(local, tot, &total);
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int p = P * (int)threadIdx.x + i;
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

// Selected (gt) and equal-to-threshold (eq) bits of 4 keys.
__device__ __forceinline__ void topk_classify(const uint32_t (&key)[4], int valid, uint32_t prefix, uint32_t pmask,
                                              bool done, unsigned* gtm, unsigned* eqm) {
    unsigned g = 0u, q = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (e >= valid) continue;
        const uint32_t mk = key[e] & pmask;
        if (mk > prefix || (done && mk == prefix)) g |= 1u << e;
        else if (!done && key[e] == prefix) q |= 1u << e;
    }
    *gtm = g;
    *eqm = q;
}

// One workgroup of NT threads: the threshold, and per slice the counts of
// selected and equal keys in the slices before it (offs[j] = gt | eq << 16).
// Every load is issued at the start, so the role costs one memory round
// trip.  lds: 4096 unsigned; tot: NT/64 + 1.  0 < k <= n <= kTopkRegN,
// n % 4 == 0, s 16-byte aligned.
constexpr int kTopkRegN = 20480;
template <int NT>
__device__ __forceinline__ void topk_threshold(const float* __restrict__ s, int n, int k,
                                               const unsigned* __restrict__ ghist, unsigned* lds, unsigned* tot,
                                               unsigned* sh, TopkThreshold* out, unsigned* __restrict__ offs) {
    constexpr int Q = kTopkRegN / (4 * NT);              // float4 of scores per thread
    constexpr int P = 4096 / NT;                         // histogram bins per thread
    constexpr int NW = NT / kWave;
    static_assert(Q * 4 * NT == kTopkRegN && P % 4 == 0, "NT in 256, 512, 1024");
    const int tid = threadIdx.x;
    const int n4 = n >> 2;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(s);
    const uint4* h4 = reinterpret_cast<const uint4*>(ghist + 4096 - P * (tid + 1));
    uint4 hv[P / 4];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) hv[q] = h4[q];
    f32x4 v[Q];                                          // float4 tid + NT q
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = tid + NT * q;
        v[q] = s4[c < n4 ? c : 0];
    }
    unsigned c[P];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
        c[P - 1 - 4 * q] = hv[q].x; c[P - 2 - 4 * q] = hv[q].y; c[P - 3 - 4 * q] = hv[q].z; c[P - 4 - 4 * q] = hv[q].w;
    }
    unsigned krem = (unsigned)k;
    unsigned above, inbin;
    uint32_t prefix = topk_pick<P>(c, 4096, krem, tot, sh, &above, &inbin) << 20;
    uint32_t pmask = 0xFFF00000u;
    krem -= above;
    bool done = inbin == krem;
    for (int ps = 0; ps < 2 && !done; ++ps) {
        const int shift = ps == 0 ? 8 : 0;
        const int nb = ps == 0 ? 4096 : 256;
        const uint32_t dmask = (uint32_t)nb - 1u;
        for (int b = tid; b < nb; b += NT) lds[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (tid + NT * q >= n4) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = order_key(v[q][e]);
                if ((key & pmask) == prefix) atomicAdd(&lds[(key >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = P * tid + i;
            c[i] = p < nb ? lds[nb - 1 - p] : 0u;
        }
        const unsigned d = topk_pick<P>(c, nb, krem, tot, sh, &above, &inbin);
        prefix |= d << shift;
        pmask |= dmask << shift;
        krem -= above;
        done = inbin == krem;
    }
    // per-slice counts: a wave sum of gt + eq * 4096 per register (at most
    // 256 + 256 * 4096, exact in fp32), kept in LDS by (register, wave); a
    // wave of 64 float4 lies in one slice of 256 float4
    float* red = reinterpret_cast<float*>(lds);          // [Q][NW]
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        unsigned gm = 0u, em = 0u;
        if (tid + NT * q < n4) {
            const uint32_t key[4] = {order_key(v[q][0]), order_key(v[q][1]), order_key(v[q][2]), order_key(v[q][3])};
            topk_classify(key, 4, prefix, pmask, done, &gm, &em);
        }
        const float w = wave_sum((float)(__builtin_popcount(gm) + ((unsigned)__builtin_popcount(em) << 12)));
        if (lane == 0) red[q * NW + wv] = w;
    }
    __syncthreads();
    if (wv == 0) {
        // slice j = float4 [256 j, 256 j + 256) = register q = 256 j / NT, waves
        // (256 j % NT) / 64 .. + 3
        const int nsl = (n4 + 255) / 256;
        unsigned cnt = 0u;                                // gt | eq << 16 of slice `lane`
        if (lane < nsl) {
            const int q = (256 * lane) / NT, w0 = ((256 * lane) % NT) / kWave;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                const unsigned p = (unsigned)red[q * NW + w0 + w4];
                cnt += (p & 0xFFFu) + ((p >> 12) << 16);
            }
        }
        const unsigned incl = wave_incl_scan(cnt);
        if (lane < nsl) offs[lane] = incl - cnt;
        if (lane == 0) *out = TopkThreshold{prefix, pmask, krem, done ? 1u : 0u};
    }
}

// One workgroup per slice of 1024 scores: the slice's selected indices at
// their place in the ascending set, from the threshold and the counts of
// the slices before it.
__device__ __forceinline__ void topk_emit_slice(const float* __restrict__ s, int n, int k, int slice,
                                                const TopkThreshold* __restrict__ thr,
                                                const unsigned* __restrict__ offs, unsigned* tot,
                                                int32_t* __restrict__ idx) {
    const int tid = threadIdx.x;
    const f32x4* s4 = reinterpret_cast<const f32x4*>(s);
    const int n4 = n >> 2;
    const int own = slice * (kTopkSlice / 4) + tid;
    const f32x4 mine = s4[own < n4 ? own : 0];
    const TopkThreshold t = *thr;
    const unsigned off = offs[slice];
    const uint32_t key[4] = {order_key(mine[0]), order_key(mine[1]), order_key(mine[2]), order_key(mine[3])};
    unsigned gm, em;
    topk_classify(key, own < n4 ? 4 : 0, t.prefix, t.pmask, t.done != 0u, &gm, &em);
    unsigned tsum;
    const unsigned ex = block_excl_scan(__builtin_popcount(gm) + ((unsigned)__builtin_popcount(em) << 16), tot, &tsum);
    unsigned eq_rank = (off >> 16) + (ex >> 16);        // equal keys before this thread's
    unsigned pos = (off & 0xFFFFu) + (ex & 0xFFFFu) + min(eq_rank, t.krem);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bool sel = (gm >> e) & 1u;
        if ((em >> e) & 1u) sel = eq_rank++ < t.krem;
        if (sel) {
            if (pos < (unsigned)k) idx[pos] = own * 4 + e;
            ++pos;
        }
    }
}

}  // namespace dv
