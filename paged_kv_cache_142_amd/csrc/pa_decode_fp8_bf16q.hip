// Partition-kernel instantiations for FP8 KV with BF16 queries.  Groups of
// eight query heads at head_dim 128 use the matrix-core kernel; other shapes
// use the generic vector kernel.
#include "pa_decode_mfma.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_fp8_bf16q_generic, Fmt::FP8, Fmt::BF16)

int launch_partition_fp8_bf16q(const DecodeArgs& a, int head_dim, int group, hipStream_t stream) {
#ifndef PA_DISABLE_MFMA8
    if (group == 8 && head_dim == 128) return dispatch_mfma8(a, head_dim, stream);
#endif
    return launch_partition_fp8_bf16q_generic(a, head_dim, group, stream);
}
}  // namespace pa
