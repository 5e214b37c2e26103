// dv_sparse_mlp for callers that cannot allocate device memory: its scratch
// (the fc1 activations and the fc2 partial sums) lives in a file-scope
// device array of fixed size instead of a caller's workspace.
//
// Host code never passes the array's name to a kernel or a copy: on the
// host that name is only a stand-in.  The array's device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// that address is what the kernels get.
#include <mutex>

#include "dv_internal.h"

namespace {

constexpr size_t kScratchBytes = DV_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];        // the array's address on each device, once looked up
std::mutex g_scratch_mu;

dv_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dvh::fail(DV_ERR_HIP, "dv_sparse_mlp_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return dvh::fail(DV_ERR_UNSUPPORTED, "dv_sparse_mlp_noalloc: device %d past the %d this build tracks", dev,
                         kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return dvh::fail(DV_ERR_HIP, "dv_sparse_mlp_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return DV_OK;
}

}  // namespace

extern "C" dv_status dv_sparse_mlp_noalloc(const float* y, int B, int d, int N, const void* w1_t, const void* b1,
                                           const void* w2_t, const void* b2, int wdt, const int32_t* idx,
                                           int n_idx_max, const int32_t* n_idx_dev, const float* residual, float* out,
                                           float* act_out, int32_t* fc2_rows, unsigned flags, void* stream) {
    dvh::clear_error();
    // shapes past the array are refused before anything else touches it
    const size_t need = dv_sparse_mlp_workspace_bytes(B, d, n_idx_max, wdt);
    if (need > kScratchBytes)
        return dvh::fail(DV_ERR_WORKSPACE,
                         "dv_sparse_mlp_noalloc: B=%d d=%d n_idx_max=%d needs %zu bytes of scratch, more than the "
                         "%zu this entry point holds",
                         B, d, n_idx_max, need, kScratchBytes);
    // every argument is checked (on the host) before the scratch is looked up
    dv_status st = dvh::sparse_mlp_call("dv_sparse_mlp_noalloc", y, B, d, N, w1_t, b1, w2_t, b2, wdt, idx, n_idx_max,
                                        n_idx_dev, residual, out, act_out, fc2_rows, flags, (void*)&g_scratch,
                                        kScratchBytes, (hipStream_t)stream, false);
    if (st != DV_OK) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != DV_OK) return st;
    // nothing in the scratch needs to start at zero: every fc1 activation
    // and fc2 partial is written by this call before it is read, and the
    // counter block at its start is not used by this path
    return dvh::sparse_mlp_call("dv_sparse_mlp_noalloc", y, B, d, N, w1_t, b1, w2_t, b2, wdt, idx, n_idx_max,
                                n_idx_dev, residual, out, act_out, fc2_rows, flags, ws, kScratchBytes,
                                (hipStream_t)stream);
}
