// Sparse Q/K/V projection kernels: fp32 weights, batches of 2 to 16.
#include "qkv.h"

namespace dvh {
template dv_status qkv_go<float, 2>(const QkvArgs&, int, hipStream_t);
template dv_status qkv_go<float, 4>(const QkvArgs&, int, hipStream_t);
template dv_status qkv_go<float, 8>(const QkvArgs&, int, hipStream_t);
template dv_status qkv_go<float, 16>(const QkvArgs&, int, hipStream_t);
}  // namespace dvh
