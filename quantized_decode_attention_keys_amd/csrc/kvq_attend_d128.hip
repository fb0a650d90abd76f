// kvq_attend_d128.hip -- decode-attention kernels instantiated for head_dim 128.
#include "kvq_attend_kernel.h"

namespace kvqi {

hipError_t launch_attend_d128(const Planes& p, const void* q, float* out, int n, int splits,
                             int waves, const void* k_new, const void* v_new, hipStream_t stream)
{
    return launch_attend_d<128>(p, q, out, n, splits, waves, k_new, v_new, stream);
}

}  // namespace kvqi
