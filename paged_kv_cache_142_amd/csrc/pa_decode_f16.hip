// Partition-kernel instantiations for F16 KV with F16 queries.
#include "pa_decode_kernel.hpp"

namespace pa {
PA_DEFINE_PARTITION_DISPATCH(launch_partition_f16, Fmt::F16, Fmt::F16)
}  // namespace pa
