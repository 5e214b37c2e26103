// Sparse Q/K/V projection kernels: fp16 weights, batches of 8 and 16.
#include "qkv.h"

namespace dvh {
template dv_status qkv_go<half_t, 8>(const QkvArgs&, int, hipStream_t);
template dv_status qkv_go<half_t, 16>(const QkvArgs&, int, hipStream_t);
}  // namespace dvh
