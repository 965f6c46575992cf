// Partition-kernel instantiations for F32 KV with F32 queries.
#include "pa_decode_kernel.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_f32, Fmt::F32, Fmt::F32)
}  // namespace pa
