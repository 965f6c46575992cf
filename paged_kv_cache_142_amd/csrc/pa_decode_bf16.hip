// Partition-kernel instantiations for BF16 KV with BF16 queries.
#include "pa_decode_kernel.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_bf16, Fmt::BF16, Fmt::BF16)
}  // namespace pa
