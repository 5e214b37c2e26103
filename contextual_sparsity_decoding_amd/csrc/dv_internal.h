// Internal declarations of libdv: device helpers and kernel launchers.
//
// Target: gfx950 (CDNA4), wave64.  Every kernel here is bandwidth-bound at
// batch 1, so the helpers are about moving bytes: 16-byte vector loads,
// rows split across the 64 lanes of a wave, fp32 accumulation and
// fixed-order (deterministic) reductions.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dv.h"

namespace dv {

typedef _Float16 half_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;          // 4 waves per workgroup
constexpr size_t kYLdsMax = 64 * 1024;
constexpr size_t kQkvLdsMax = 64 * 1024;     // Q/K/V inputs staged in LDS (two workgroups per CU, with room)
constexpr int kTopkMaxN = 1 << 22;          // longest row dv_topk_select takes
constexpr int kUnionMaxN = 1 << 18;         // union bitmap in LDS: n / 8 bytes
constexpr int kTopkStage = 8192;            // selected sets up to this size leave through LDS

// ---- element traits: E elements of T per 16-byte chunk --------------------
template <typename T> struct Vec;
template <> struct Vec<half_t> { static constexpr int E = 8; };
template <> struct Vec<float> { static constexpr int E = 4; };

__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[8], half_t) {
    f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ __forceinline__ void unpack(const u32x4& w, float (&f)[4], float) {
    f32x4 v = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = v[i];
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return (float)v; }

// An element held as its bits in a 32-bit register (fp16 zero-extended)
// until it is used, converted then by bits_f32: an fp16 value converted
// next to its load, or held as fp16 (packed two to a register), makes the
// compiler wait for that load, and so for every load issued before it.
__device__ __forceinline__ unsigned elt_bits(const half_t* p) { return *reinterpret_cast<const unsigned short*>(p); }
__device__ __forceinline__ unsigned elt_bits(const float* p) { return *reinterpret_cast<const unsigned*>(p); }
template <typename T> __device__ __forceinline__ float bits_f32(unsigned b);
template <> __device__ __forceinline__ float bits_f32<half_t>(unsigned b) {
    return (float)__builtin_bit_cast(half_t, (unsigned short)b);
}
template <> __device__ __forceinline__ float bits_f32<float>(unsigned b) { return __builtin_bit_cast(float, b); }

// ---- cross-lane moves and reductions --------------------------------------
// DPP (data-parallel primitives) move values between lanes inside the VALU
// instruction itself, with no trip through the LDS crossbar.  gfx9 control
// words: quad_perm 0x00-0xff, row_shr:n 0x110+n, row_ror:n 0x120+n,
// row_mirror 0x140, row_half_mirror 0x141, row_bcast:15 0x142,
// row_bcast:31 0x143.  A row is 16 lanes.  Lanes that a control word or a
// row mask leaves without a source keep `old`, here 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of G lanes (G divides 16, or 64), every lane of a
// group gets its group's sum.  The order of additions is fixed, so results
// are deterministic.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "power of two lanes");
    if constexpr (G >= 2) v += dpp_f32<0xb1>(v);          // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v += dpp_f32<0x4e>(v);          // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v += dpp_f32<0x141>(v);         // half-row mirror: the other quad
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);        // row mirror: the other half-row
    if constexpr (G == 32) v += __shfl_xor(v, 16, kWave);  // the neighbouring row
    if constexpr (G == 64)
        v = (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float group_sum_dyn(float v, int G) {
    switch (G) {
        case 1: return v;
        case 2: return group_sum<2>(v);
        case 4: return group_sum<4>(v);
        case 8: return group_sum<8>(v);
        case 16: return group_sum<16>(v);
        case 32: return group_sum<32>(v);
        default: return group_sum<64>(v);
    }
}

// Dot products of one weight row (nchunk 16-byte chunks of T) with NB fp32
// vectors, by one wave.  Lane l covers chunks l, l+64, ...; U chunk loads
// are issued before any is used.  `ys` may point to LDS or global memory
// (vector b at ys + b * ystride; vectors b >= nvalid read vector 0 and
// their sums are to be discarded).  Each lane returns its partial sums.
template <typename T, int NB, int U, bool STREAM>
__device__ __forceinline__ void wave_rowdot(const T* __restrict__ row, int nchunk,
                                            const float* __restrict__ ys, int ystride, int nvalid,
                                            float (&acc)[NB]) {
    constexpr int E = Vec<T>::E;
    const int lane = threadIdx.x & (kWave - 1);
    for (int base = 0; base < nchunk; base += kWave * U) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = base + lane + kWave * u;
            if (c < nchunk)
                w[u] = STREAM ? ld16_stream(row + (size_t)c * E) : ld16(row + (size_t)c * E);
            else
                w[u] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = base + lane + kWave * u;
            if (c < nchunk) {
                float f[E];
                unpack(w[u], f, T());
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int bb = b < nvalid ? b : 0;
                    const f32x4* yv = reinterpret_cast<const f32x4*>(ys + (size_t)bb * ystride + (size_t)c * E);
#pragma unroll
                    for (int q = 0; q < E / 4; ++q) {
                        const f32x4 y4 = yv[q];
                        acc[b] = fmaf(f[4 * q + 0], y4[0], acc[b]);
                        acc[b] = fmaf(f[4 * q + 1], y4[1], acc[b]);
                        acc[b] = fmaf(f[4 * q + 2], y4[2], acc[b]);
                        acc[b] = fmaf(f[4 * q + 3], y4[3], acc[b]);
                    }
                }
            }
        }
    }
}

// Order-preserving map of fp32 to uint32 for selection: larger float ->
// larger key; -0 and +0 map to the same key; NaN maps to 0, below -inf.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (f != f) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the wave: shifts of 1, 2, 4, 8 inside each row,
// then row totals carried forward by the row broadcasts.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
    v += dpp_u32<0x111>(v);
    v += dpp_u32<0x112>(v);
    v += dpp_u32<0x114>(v);
    v += dpp_u32<0x118>(v);
    v += dpp_u32<0x142, 0xa>(v);                          // lane 15 of rows 0, 2 into rows 1, 3
    v += dpp_u32<0x143, 0xc>(v);                          // lane 31 into rows 2, 3
    return v;
}

// Exclusive prefix sum over the block (<= 1024 threads); *total gets the sum.
// Every wave combines the wave totals itself, so no lane waits on a serial
// pass.  `tot` holds >= 16 words and may be reused by the next call.
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* tot, unsigned* total) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nw = (int)(blockDim.x >> 6);
    const unsigned incl = wave_incl_scan(v);
    __syncthreads();                                      // a previous call may still read tot
    if (lane == 63) tot[w] = incl;
    __syncthreads();
    const unsigned ts = wave_incl_scan(lane < nw ? tot[lane] : 0u);
    const unsigned before = w > 0 ? (unsigned)__builtin_amdgcn_readlane((int)ts, w - 1) : 0u;
    *total = (unsigned)__builtin_amdgcn_readlane((int)ts, 63);
    return before + incl - v;
}

// Load a small vector from global memory into LDS with the whole block.
__device__ __forceinline__ void block_copy_f32(float* __restrict__ dst, const float* __restrict__ src, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src[i];
}

struct RowArgs;    // rowdot.h
struct Pred2Args;  // pred.h

// The finalize's epilogue (gather-AXPY): store the sums, store their ReLU,
// or scatter a Q/K/V output row (columns [which][h][d_h]) into q (fp32
// [B][h][d_h]) and the K/V caches' slot pos (*pos_dev when set).
enum { FIN_STORE = 0, FIN_RELU = 1, FIN_QKV = 2 };
struct FinEpi {
    int mode;
    float* q;
    half_t* k;
    half_t* v;
    int h, dh, max_len, pos;
    const int32_t* pos_dev;
};

}  // namespace dv

// ---- host side --------------------------------------------------------------
namespace dvh {

dv_status fail(dv_status code, const char* fmt, ...);
void clear_error();
// dv_time_launches: an event before and after each launch of the kernel
// role being timed (no-ops otherwise).
void timed_begin(int kind, hipStream_t s);
void timed_end(int kind, hipStream_t s);
bool timed_take(hipEvent_t* ev);   // the role's two events, for its first DV_LAUNCH

// A kernel launch that, inside a timed role, carries the role's events on
// the dispatch itself (hipExtLaunchKernelGGL): they then mark the kernel's
// own start and end rather than the points around its launch.
#define DV_LAUNCH(K, GRID, BLOCK, LDS, S, ...)                                                    \
    do {                                                                                          \
        hipEvent_t dv_ev_[2];                                                                     \
        if (dvh::timed_take(dv_ev_))                                                              \
            hipExtLaunchKernelGGL(K, GRID, BLOCK, LDS, S, dv_ev_[0], dv_ev_[1], 0, __VA_ARGS__);   \
        else                                                                                      \
            hipLaunchKernelGGL(K, GRID, BLOCK, LDS, S, __VA_ARGS__);                              \
    } while (0)
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
int elt_bytes(int wdt);

// Every workspace starts with a fixed block of counters (zero between calls;
// the kernels that use one reset it), so calls of any shape can share one
// workspace.  Scratch buffers are carved after it.
constexpr size_t kCounterBytes = 4096;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(unsigned));
inline unsigned* ws_counters(void* ws, int i = 0) { return ws ? (unsigned*)ws + i : nullptr; }

// Workspace carving: a bump allocator over the caller's buffer.
struct Carve {
    char* base;
    size_t off = kCounterBytes;
    explicit Carve(void* p) : base((char*)p) {}
    template <typename T> T* take(size_t n) {
        off = align_up(off, 256);
        T* p = base ? (T*)(base + off) : nullptr;
        off += n * sizeof(T);
        return p;
    }
};

// Kernel launchers (no validation; the entry points validate first).
dv_status launch_layernorm(const float* x, int B, int d, const float* g, const float* b, float eps,
                           float* y, hipStream_t s);
size_t pred_partials(int B, int d, int r, int wdt);
// With mpart (rowdot_mfma_rows_part_floats of both layers) and a batch the
// matrix cores take, both layers run there.
dv_status launch_predict(const float* y, int B, int d, const void* p1_t, int r, const void* p2_t,
                         int n_out, int wdt, int act, float* scores, float* hid_part,
                         hipStream_t s, float* mpart = nullptr);
dv_status launch_fc1(const float* y, int B, int d, const void* w1_t, const void* b1, int wdt,
                     const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a, hipStream_t s);
struct AxpyPlan {
    int n_slices, n_groups, rows_per_group;
};
AxpyPlan axpy_plan(int d, int rows, int wdt);
size_t axpy_ws_floats(const AxpyPlan& p, int B, int d);
// A top-k over n scores split into roles that ride in other launches
// (topk_split.h): histogram slices, the threshold, ordered emission.
struct TopkSel {
    const float* s;           // scores [n], 16-byte aligned
    int n, k;                 // 0 < k <= n <= 20480, n % 4 == 0
    unsigned* hist;           // [4096], cleared before the histogram role
    uint32_t* keys;           // [n] order keys, written by the histogram role; 16-byte aligned
    void* thr;                // the threshold (16 bytes)
    int32_t* idx;             // [k] selected, ascending
};
bool topk_split_supported(int n, int k);

struct AxpyCall {
    const void* w;            // W [w_rows][d]
    int wdt, d, w_rows, rows;
    const int32_t* n_rows_dev;
    const int32_t* idx;       // row(u) = idx[u / blk] * blk + u % blk, or u when NULL
    int blk;
    const float* coef;        // [B][coef_stride], or NULL with apart
    int coef_stride;
    bool skip_zero;
    bool thresh;              // with skip_zero: coefficients of magnitude <= thr count as zero
    float thr;
    dv::FinEpi epi;           // the finalize's epilogue (FIN_STORE by default)
    const float* apart;       // split-K attention partials giving the coefficients, or NULL
    int num_splits;
    int B;
    const void* bias;
    const float* residual;
    float* out;
    int32_t* rows_read;
    float* partial;
    int32_t* advance;
    const TopkSel* sel;       // B == 1: also run a role of this selection in one more column of
                              // workgroups (the last), or NULL
    int timed;                // DV_KERNEL_* role of the main launch for dv_time_launches, or 0
};
dv_status launch_axpy(const AxpyCall& c, hipStream_t s);
// batches whose gather-AXPY runs on the matrix cores when its coefficients are in memory
bool axpy_mfma_supported(int B, int d, int wdt);
bool qkv_supported(int B, int d, int wdt);
dv_status launch_qkv(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                     const void* w, const void* bias, int wdt, float* q, const dv_kv_state* kv, bool mark_valid,
                     hipStream_t s, const float* ln_g = nullptr, const float* ln_b = nullptr, float eps = 0.f,
                     const dv::RowArgs* pred = nullptr);
dv_status launch_fc1_ln(const float* x, int d, const float* g, const float* b, float eps, const void* w1_t,
                        const void* b1, int wdt, const int32_t* idx, int n_max, const int32_t* n_dev, int N, float* a_out,
                        hipStream_t s);
bool ln_fusable(int B, int d);
dv_status launch_predict_ln(const float* x, int B, int d, const float* g, const float* b, float eps, float* y_out,
                            const void* p1_t, int r, const void* p2_t, int n_out, int wdt, int act, float* scores,
                            float* hid, hipStream_t s, float* mpart = nullptr);
bool pred_topk_fusable(int B, int n_out, int r);
bool row_ln_supported(int d, int wdt);
dv_status launch_predict_pair_ln(const float* x, int d, const float* g, const float* b, float eps, float* y_out,
                                 const void* pa1_t, int rA, const void* pa2_t, int h, int kA, int32_t* idxA,
                                 const void* pm1_t, int rM, const void* pm2_t, int N, float* sA, float* sM, float* hid,
                                 int wdt, int act, hipStream_t s);
dv_status launch_predict_ln_topk(const float* x, int d, const float* g, const float* b, float eps, float* y_out,
                                 const void* p1_t, int r, const void* p2_t, int n_out, int wdt, int act,
                                 float* scores, float* hid, int k, int32_t* idx, hipStream_t s);
int topk_block_threads(int n);
dv_status launch_set_i32(int32_t* p, int v, hipStream_t s);
dv_status launch_topk(const float* scores, int B, int n, int k, int32_t* idx, hipStream_t s);
dv_status launch_union(const int32_t* idx, int B, int k, int n, int32_t* union_idx,
                       int32_t* union_count, hipStream_t s);
int splitk_auto(int max_positions, int rows);
// Most positions one head of the view reads: the retained set plus the
// appended tail, the sinks plus the recent window, or every position.
int view_positions(const dv_kv_view* kv);
dv_status launch_splitk(const float* q, int B, int d_h, const int32_t* head_idx, int n_sel,
                        const dv_kv_view* kv, const int32_t* n_dev, int n_add, float scale, int num_splits, float* o,
                        float* part, int32_t* mark_valid, int mark_pos, const int32_t* mark_pos_dev, hipStream_t s,
                        int* splits_used = nullptr, const dv::Pred2Args* pred = nullptr);
dv::Pred2Args pred2_args(const float* hid_a, int r_a, const void* p2_a, int n_a, float* s_a, int k_a, int32_t* idx_a,
                         const float* hid_m, int r_m, const void* p2_m, int n_m, float* s_m, int act, int wdt);
dv_status launch_kv_score(const void* q_obs, int B, int h, int d_h, int n_obs, const dv_kv_view* kv,
                          float scale, int n_sink, int n_window, int width, float* scores,
                          float* raw, float* stats, hipStream_t s);
size_t kv_score_stats_floats(int B, int h, int n, int n_obs);
dv_status sparse_mlp_call(const char* who, const float* y, int B, int d, int N, const void* w1_t, const void* b1,
                          const void* w2_t, const void* b2, int wdt, const int32_t* idx, int n_idx_max,
                          const int32_t* n_idx_dev, const float* residual, float* out, float* act_out,
                          int32_t* fc2_rows, unsigned flags, void* ws, size_t ws_bytes, hipStream_t s,
                          bool run = true);
// Batched row-dots on the matrix cores (k_rowdot_mfma.hip), B in [8, 16],
// fp16 weights, d % 32 == 0; `part` holds rowdot_mfma_part_floats floats.
bool rowdot_mfma_ok(int B, int d, int wdt);
size_t rowdot_mfma_part_floats(int n_max);
// out[b][j] = y[b] . W[j] (its ReLU when asked) for every row j < n_rows of W,
// on the matrix cores; `part` holds rowdot_mfma_rows_part_floats(n_rows, d) floats
size_t rowdot_mfma_rows_part_floats(int n_rows, int d);
dv_status launch_rows_mfma(const float* y, int B, int d, const void* w, int n_rows, bool relu, float* out,
                           float* part, hipStream_t s);
dv_status launch_fc1_mfma(const float* y, int B, int d, const void* w1_t, const void* b1, const int32_t* idx,
                          int n_max, const int32_t* n_dev, int N, float* a_out, float* part, hipStream_t s);
dv_status launch_qkv_mfma(const float* y, int B, int d, int h, int d_h, const int32_t* head_idx, int n_sel,
                          const void* w, const void* bias, float* q, const dv_kv_state* kv, float* part,
                          hipStream_t s);
dv_status launch_fill_normal(void* out, uint64_t n, int dtype, uint64_t seed, uint64_t stream, uint64_t offset,
                             float mean, float stdv, hipStream_t s);

}  // namespace dvh
