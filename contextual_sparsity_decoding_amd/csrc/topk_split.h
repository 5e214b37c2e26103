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

// The digit whose bin holds the krem-th largest candidate (0 < krem <= the
// candidates counted); thread t holds the counts of bins nb-1-(P*t+i),
// i < P (scanning from the top).  Two barriers.  buf holds 19 words that
// the previous call's readers may still hold: calls alternate two buffers.
template <int P, int NT>
__device__ __forceinline__ unsigned topk_pick(const unsigned (&c)[P], int nb, unsigned krem, unsigned* buf,
                                              unsigned* above, unsigned* inbin) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    unsigned local = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i) local += c[i];
    const unsigned incl = wave_incl_scan(local);
    if (lane == 63) buf[w] = incl;
    __syncthreads();
    const unsigned ts = wave_incl_scan(lane < NW ? buf[lane] : 0u);
    unsigned run = (w > 0 ? (unsigned)__builtin_amdgcn_readlane((int)ts, w - 1) : 0u) + incl - local;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int p = P * (int)threadIdx.x + i;
        if (p < nb && run < krem && run + c[i] >= krem) {
            buf[16] = (unsigned)(nb - 1 - p);
            buf[17] = run;
            buf[18] = c[i];
        }
        run += c[i];
    }
    __syncthreads();
    *above = buf[17];
    *inbin = buf[18];
    return buf[16];
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
// Every load is issued at the start and the keys stay in registers, so the
// role costs one memory round trip; the per-slice counts come from wave
// ballots.  lds: kTopkThrWords.  0 < k <= n <= kTopkRegN, n % 4 == 0, s
// 16-byte aligned.
constexpr int kTopkRegN = 20480;
constexpr int kTopkThrWords = 4096 + 256 + kTopkRegN / 256 + 2 * 20;
template <int NT>
__device__ __forceinline__ void topk_threshold(const float* __restrict__ s, int n, int k,
                                               const unsigned* __restrict__ ghist, unsigned* lds,
                                               TopkThreshold* out, unsigned* __restrict__ offs) {
    constexpr int Q = kTopkRegN / (4 * NT);              // float4 of scores per thread
    constexpr int P = 4096 / NT;                         // histogram bins per thread
    constexpr int NW = NT / kWave;
    static_assert(Q * 4 * NT == kTopkRegN && P % 4 == 0 && NW <= 16, "NT in 256, 512, 1024");
    unsigned* bins12 = lds;                              // second digit (bits 8..19)
    unsigned* bins8 = lds + 4096;                        // third digit (bits 0..7)
    unsigned* red = lds + 4096 + 256;                    // per (register, wave) counts
    unsigned* pbuf = red + Q * NW;                       // two pick buffers of 20 words
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
    // both later histograms cleared while the loads are in flight (the
    // first pick's barriers order this before their use)
    for (int b = tid; b < 4096 + 256; b += NT) lds[b] = 0u;
    unsigned c[P];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
        c[P - 1 - 4 * q] = hv[q].x; c[P - 2 - 4 * q] = hv[q].y; c[P - 3 - 4 * q] = hv[q].z; c[P - 4 - 4 * q] = hv[q].w;
    }
    uint32_t key[Q][4];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) key[q][e] = order_key(v[q][e]);
    unsigned krem = (unsigned)k;
    unsigned above, inbin;
    uint32_t prefix = topk_pick<P, NT>(c, 4096, krem, pbuf, &above, &inbin) << 20;
    uint32_t pmask = 0xFFF00000u;
    krem -= above;
    bool done = inbin == krem;
    if (!done) {                                         // bits 8..19 of the keys in the chosen bin
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (tid + NT * q >= n4) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((key[q][e] & pmask) == prefix) atomicAdd(&bins12[(key[q][e] >> 8) & 0xFFFu], 1u);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) c[i] = bins12[4095 - (P * tid + i)];
        const unsigned d = topk_pick<P, NT>(c, 4096, krem, pbuf + 20, &above, &inbin);
        prefix |= d << 8;
        pmask = 0xFFFFFF00u;
        krem -= above;
        done = inbin == krem;
    }
    if (!done) {                                         // bits 0..7
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (tid + NT * q >= n4) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((key[q][e] & pmask) == prefix) atomicAdd(&bins8[key[q][e] & 0xFFu], 1u);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = P * tid + i;
            c[i] = p < 256 ? bins8[255 - p] : 0u;
        }
        const unsigned d = topk_pick<P, NT>(c, 256, krem, pbuf, &above, &inbin);
        prefix |= d;
        pmask = 0xFFFFFFFFu;
        krem -= above;
        done = inbin == krem;
    }
    // per-slice counts: per register q, this wave's selected and equal keys
    // (ballots; a wave of 64 float4 lies in one slice of 256 float4)
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const bool ok = tid + NT * q < n4;
        unsigned g = 0u, eq = 0u;
        if (done) {                                      // uniform: every key at or above the prefix
#pragma unroll
            for (int e = 0; e < 4; ++e) g += (unsigned)__popcll(__ballot(ok && (key[q][e] & pmask) >= prefix));
        } else {                                         // pmask is all ones
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                g += (unsigned)__popcll(__ballot(ok && key[q][e] > prefix));
                eq += (unsigned)__popcll(__ballot(ok && key[q][e] == prefix));
            }
        }
        if (lane == 0) red[q * NW + wv] = g | eq << 16;
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
            for (int w4 = 0; w4 < 4; ++w4) cnt += red[q * NW + w0 + w4];
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
