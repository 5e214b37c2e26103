// fp32 instantiation of the sparse Q/K/V projection kernels.
#include "qkv.h"

namespace dvh {
template dv_status qkv_launch_t<float>(const QkvArgs&, int, hipStream_t);
}  // namespace dvh
