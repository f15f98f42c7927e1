// Instantiation of the prefill kernels for storage BF16, head dim 128,
// top-k register list of 64 entries (query-group sizes up to 4).
#include "prefill_kernels.hpp"

namespace hsa_attn {
template hipError_t launch_prefill_g<BF16, 128, 64>(const PrefillArgs&, hipStream_t);
}  // namespace hsa_attn
