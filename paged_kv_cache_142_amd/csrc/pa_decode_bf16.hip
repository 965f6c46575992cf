// Partition-kernel instantiations for BF16 KV with BF16 queries.  Groups of
// four query heads use the head-in-lane score layout; other groups use the
// generic kernel.
#include "pa_decode_gqa.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_bf16_generic, Fmt::BF16, Fmt::BF16)

int launch_partition_bf16(const DecodeArgs& a, int head_dim, int group, hipStream_t stream) {
#ifndef PA_DISABLE_GQA4
    if (group == 4) return dispatch_gqa4<Fmt::BF16>(a, head_dim, stream);
#endif
    return launch_partition_bf16_generic(a, head_dim, group, stream);
}
}  // namespace pa
