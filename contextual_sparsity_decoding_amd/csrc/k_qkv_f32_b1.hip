// Sparse Q/K/V projection kernels: fp32 weights, batch of one.
#include "qkv.h"

namespace dvh {
template dv_status qkv_go<float, 1>(const QkvArgs&, int, hipStream_t);
}  // namespace dvh
