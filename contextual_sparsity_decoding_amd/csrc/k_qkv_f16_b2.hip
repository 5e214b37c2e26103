// Sparse Q/K/V projection kernels: fp16 weights, batches of 2 and 4.
#include "qkv.h"

namespace dvh {
template dv_status qkv_go<half_t, 2>(const QkvArgs&, int, hipStream_t);
template dv_status qkv_go<half_t, 4>(const QkvArgs&, int, hipStream_t);
}  // namespace dvh
