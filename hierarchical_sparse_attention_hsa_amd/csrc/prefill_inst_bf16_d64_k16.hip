// Instantiation of the prefill kernels for storage BF16, head dim 64,
// top-k register list of 16 entries (all query-group sizes).
#include "prefill_kernels.hpp"

namespace hsa_attn {
template hipError_t launch_prefill_g<BF16, 64, 16>(const PrefillArgs&, hipStream_t);
}  // namespace hsa_attn
