// Top-k of one score row split into three roles that ride as extra
// workgroups in launches doing other work; the launches between them order
// the roles.  Same selection as the top-k kernels (score
// descending, ties to the lower index, NaN after numbers; the set ascending).
//
// Pages: DejaVu = "Deja Vu: Contextual Sparsity for Efficient LLMs at
// Inference Time" (arXiv 2310.17157), §2.3 (the sets S_M under a budget)
// and §4.3 (the next layer's selection overlaps this layer's work).
//
//   1. topk_hist_slice, one workgroup per 1024 scores: stores the scores'
//      order keys and adds the histogram of their top 12 bits into a global
//      histogram (cleared earlier).
//   2. topk_threshold, one workgroup (1024 threads in the finalize that
//      hosts it): the k-th key by radix select, the
//      first digit read off that histogram, the next 12 and 8 bits
//      histogrammed in LDS over the keys still in the running (stopping once
//      a bin is taken whole); it writes the threshold.
//   3. topk_emit_slice, one workgroup per 1024 keys: counts the selected
//      keys in the slices before its own (they are L2-resident), then writes
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
                                                unsigned* __restrict__ ghist, uint32_t* __restrict__ keys) {
    const int tid = threadIdx.x;
    const int i = slice * kTopkSlice + 4 * tid;
    const f32x4 v = i < n ? *reinterpret_cast<const f32x4*>(s + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int b = tid; b < 4096; b += 256) lds[b] = 0u;
    __syncthreads();
    if (i < n) {
        const uint4 kk{order_key(v[0]), order_key(v[1]), order_key(v[2]), order_key(v[3])};
        *reinterpret_cast<uint4*>(keys + i) = kk;
        atomicAdd(&lds[kk.x >> 20], 1u);
        atomicAdd(&lds[kk.y >> 20], 1u);
        atomicAdd(&lds[kk.z >> 20], 1u);
        atomicAdd(&lds[kk.w >> 20], 1u);
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

// One workgroup of NT threads: the threshold of the k largest of n order
// keys.  Every load is issued at the start and the keys stay in registers,
// so the role costs one memory round trip.  lds: kTopkThrWords.
// 0 < k <= n <= kTopkRegN, n % 4 == 0, keys 16-byte aligned.
constexpr int kTopkRegN = 49152;                 // 48 keys per thread of 1024; d_ffn of OPT-175B
constexpr int kTopkThrWords = 4096 + 256 + 2 * 20;
template <int NT>
__device__ __forceinline__ void topk_threshold(const uint32_t* __restrict__ keys, int n, int k,
                                               const unsigned* __restrict__ ghist, unsigned* lds,
                                               TopkThreshold* out) {
    constexpr int Q = kTopkRegN / (4 * NT);              // uint4 of keys per thread
    constexpr int P = 4096 / NT;                         // histogram bins per thread
    static_assert(Q * 4 * NT == kTopkRegN && P % 4 == 0 && NT / kWave <= 16, "NT in 256, 512, 1024");
    unsigned* bins12 = lds;                              // second digit (bits 8..19)
    unsigned* bins8 = lds + 4096;                        // third digit (bits 0..7)
    unsigned* pbuf = lds + 4096 + 256;                   // two pick buffers of 20 words
    const int tid = threadIdx.x;
    const int n4 = n >> 2;
    const uint4* k4 = reinterpret_cast<const uint4*>(keys);
    const uint4* h4 = reinterpret_cast<const uint4*>(ghist + 4096 - P * (tid + 1));
    uint4 hv[P / 4];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) hv[q] = h4[q];
    uint4 kv[Q];                                         // uint4 tid + NT q
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int c = tid + NT * q;
        kv[q] = k4[c < n4 ? c : 0];
    }
    // both later histograms cleared while the loads are in flight (the
    // first pick's barriers order this before their use)
    for (int b = tid; b < 4096 + 256; b += NT) lds[b] = 0u;
    unsigned c[P];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
        c[P - 1 - 4 * q] = hv[q].x; c[P - 2 - 4 * q] = hv[q].y; c[P - 3 - 4 * q] = hv[q].z; c[P - 4 - 4 * q] = hv[q].w;
    }
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
            const uint32_t kq[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((kq[e] & pmask) == prefix) atomicAdd(&bins12[(kq[e] >> 8) & 0xFFFu], 1u);
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
            const uint32_t kq[4] = {kv[q].x, kv[q].y, kv[q].z, kv[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((kq[e] & pmask) == prefix) atomicAdd(&bins8[kq[e] & 0xFFu], 1u);
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
    if (tid == 0) *out = TopkThreshold{prefix, pmask, krem, done ? 1u : 0u};
}

// One workgroup per slice of 1024 keys: the slice's selected indices at
// their place in the ascending set.  The selected and equal keys of the
// slices before it are counted here too, EB slices' loads issued at once
// (each workgroup reads at most kTopkRegN - 1024 keys, L2-resident).  tot:
// 20 words.
__device__ __forceinline__ void topk_emit_slice(const uint32_t* __restrict__ keys, int n, int k, int slice,
                                                const TopkThreshold* __restrict__ thr, unsigned* tot,
                                                int32_t* __restrict__ idx) {
    constexpr int EB = 12;                               // earlier slices per round of loads
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint4* k4 = reinterpret_cast<const uint4*>(keys);
    const int n4 = n >> 2;
    const int own = slice * (kTopkSlice / 4) + tid;
    const uint4 mine = k4[own < n4 ? own : 0];
    const TopkThreshold t = *thr;
    const bool done = t.done != 0u;
    unsigned pc = 0u;                                    // gt | eq << 16 over this thread's earlier keys
    for (int j0 = 0; j0 < slice; j0 += EB) {             // uniform over the workgroup
        uint4 pre[EB];                                   // uint4 tid + 256 j of slice j < slice
#pragma unroll
        for (int j = 0; j < EB; ++j)
            pre[j] = j0 + j < slice ? k4[tid + (kTopkSlice / 4) * (j0 + j)] : uint4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < EB; ++j) {
            if (j0 + j < slice) {
                const uint32_t kq[4] = {pre[j].x, pre[j].y, pre[j].z, pre[j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t mk = kq[e] & t.pmask;
                    pc += (mk > t.prefix || (done && mk == t.prefix)) ? 1u
                          : (!done && kq[e] == t.prefix)             ? 0x10000u
                                                                     : 0u;
                }
            }
        }
    }
    const unsigned pw = (unsigned)__builtin_amdgcn_readlane((int)wave_incl_scan(pc), 63);
    if (lane == 0) tot[16 + wv] = pw;
    const uint32_t key[4] = {mine.x, mine.y, mine.z, mine.w};
    unsigned gm, em;
    topk_classify(key, own < n4 ? 4 : 0, t.prefix, t.pmask, done, &gm, &em);
    unsigned tsum;
    const unsigned ex = block_excl_scan(__builtin_popcount(gm) + ((unsigned)__builtin_popcount(em) << 16), tot, &tsum);
    const unsigned off = (tot[16] + tot[17]) + (tot[18] + tot[19]);   // written before the scan's barriers
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
