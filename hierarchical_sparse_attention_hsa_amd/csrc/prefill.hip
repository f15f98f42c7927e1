// HSA prefill: host-side planning and dispatch.  The kernels live in
// prefill_kernels.hpp and are instantiated in prefill_inst_*.hip.
#include "prefill_kernels.hpp"

namespace hsa_attn {

// Each instantiation unit that is part of the build defines
// HSA_ATTN_HAVE_<dtype>_D<d>_K<list> for this file (see build.py; a full
// build has all eight).  A missing one makes the call report "unsupported".
#define HSA_ATTN_PREFILL_EXTERN(T, D, K) \
  extern template hipError_t launch_prefill_g<T, D, K>(const PrefillArgs&, hipStream_t);
HSA_ATTN_PREFILL_EXTERN(BF16, 128, 16)
HSA_ATTN_PREFILL_EXTERN(BF16, 128, 32)
HSA_ATTN_PREFILL_EXTERN(BF16, 64, 16)
HSA_ATTN_PREFILL_EXTERN(BF16, 64, 32)
HSA_ATTN_PREFILL_EXTERN(FP32, 128, 16)
HSA_ATTN_PREFILL_EXTERN(FP32, 128, 32)
HSA_ATTN_PREFILL_EXTERN(FP32, 64, 16)
HSA_ATTN_PREFILL_EXTERN(FP32, 64, 32)

#define HSA_ATTN_CALL(HAVE, T, D, K)                   \
  do {                                                 \
    if constexpr (HAVE) return launch_prefill_g<T, D, K>(a, st); \
    return hipErrorNotSupported;                       \
  } while (0)

// ---------------------------------------------------------------- host side
static size_t align_up_p(size_t x, size_t a) { return (x + a - 1) / a * a; }

PrefillPlan plan_prefill(const Geometry& g, bool own_sel) {
  PrefillPlan p{};
  size_t off = 0;
  if (own_sel) {
    const size_t rows = (size_t)g.B * g.Hq * (size_t)g.T;
    p.off_sel_idx = off;
    off = align_up_p(off + rows * g.k * sizeof(int32_t), 256);
    p.off_sel_score = off;
    off = align_up_p(off + rows * g.k * sizeof(float), 256);
  }
  p.bytes = off;
  return p;
}

size_t prefill_attn_lds_bytes(const Geometry& g) {
  const size_t esz = g.bf16 ? 2 : 4;
  const size_t nwords = (size_t)((g.Nc + 31) / 32);
  return 2 * (size_t)kChunk * g.D * esz + (size_t)32 * g.G * g.k * 8 + nwords * 4;
}

#ifndef HSA_ATTN_HAVE_BF16_D128_K16
#define HSA_ATTN_HAVE_BF16_D128_K16 0
#endif
#ifndef HSA_ATTN_HAVE_BF16_D128_K32
#define HSA_ATTN_HAVE_BF16_D128_K32 0
#endif
#ifndef HSA_ATTN_HAVE_BF16_D64_K16
#define HSA_ATTN_HAVE_BF16_D64_K16 0
#endif
#ifndef HSA_ATTN_HAVE_BF16_D64_K32
#define HSA_ATTN_HAVE_BF16_D64_K32 0
#endif
#ifndef HSA_ATTN_HAVE_FP32_D128_K16
#define HSA_ATTN_HAVE_FP32_D128_K16 0
#endif
#ifndef HSA_ATTN_HAVE_FP32_D128_K32
#define HSA_ATTN_HAVE_FP32_D128_K32 0
#endif
#ifndef HSA_ATTN_HAVE_FP32_D64_K16
#define HSA_ATTN_HAVE_FP32_D64_K16 0
#endif
#ifndef HSA_ATTN_HAVE_FP32_D64_K32
#define HSA_ATTN_HAVE_FP32_D64_K32 0
#endif

// the register top-k list holds 16 or 32 entries; k <= 16 uses the short list
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const bool shortlist = a.g.k <= 16;
  if (a.g.bf16) {
    if (a.g.D == 128) {
      if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D128_K16, BF16, 128, 16);
      HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D128_K32, BF16, 128, 32);
    }
    if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D64_K16, BF16, 64, 16);
    HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D64_K32, BF16, 64, 32);
  }
  if (a.g.D == 128) {
    if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D128_K16, FP32, 128, 16);
    HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D128_K32, FP32, 128, 32);
  }
  if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D64_K16, FP32, 64, 16);
  HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D64_K32, FP32, 64, 32);
}

}  // namespace hsa_attn
