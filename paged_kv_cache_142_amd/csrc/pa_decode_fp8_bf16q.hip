// Partition-kernel instantiations for FP8 KV with BF16 queries.
#include "pa_decode_kernel.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_fp8_bf16q, Fmt::FP8, Fmt::BF16)
}  // namespace pa
