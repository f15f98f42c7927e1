// 32x32 MFMA tiles for gfx950, shared by the prefill kernels.
//
// Layout of one 32x32 output tile C (16 fp32 per lane):
//   lane l holds column j = l % 32 and rows i = 8*(r/4) + 4*(l/32) + r%4,
//   r = 0..15.
// Operand fragments: for one "k-chunk" of 16 contraction indices, lane l
// supplies row/column (l % 32) and the 8 contraction indices
// 8*(l/32) .. 8*(l/32)+7 of that chunk.  Both operands use the same
// assignment, so the contraction is exact whatever order the hardware sums in.
//   bf16: one v_mfma_f32_32x32x16_bf16 per k-chunk (8 bf16 per lane)
//   fp32: eight v_mfma_f32_32x32x2_f32 per k-chunk (the e-th element of
//         both operands in the e-th instruction)
#pragma once

#include "common.hpp"

namespace hsa_attn {

template <typename T>
struct Frag;

template <>
struct Frag<BF16> {
  bf16x8 v;
  __device__ __forceinline__ void load16(const void* p) {  // 8 bf16 = 16 bytes
    v = as_bf16x8(*reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void from_f32(const float* x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<__bf16>(x[e]);
  }
};

template <>
struct Frag<FP32> {
  float v[8];
};

__device__ __forceinline__ void mfma(f32x16& acc, const Frag<BF16>& a, const Frag<BF16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x16& acc, const Frag<FP32>& a, const Frag<FP32>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 consecutive elements of a global row (zero when !ok)
__device__ __forceinline__ void load_frag_global(Frag<BF16>& f, const uint16_t* p, bool ok) {
  const u32x4 z = ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
  f.v = as_bf16x8(z);
}
__device__ __forceinline__ void load_frag_global(Frag<FP32>& f, const float* p, bool ok) {
  const f32x4 z{0.f, 0.f, 0.f, 0.f};
  const f32x4 a = ok ? reinterpret_cast<const f32x4*>(p)[0] : z;
  const f32x4 b = ok ? reinterpret_cast<const f32x4*>(p)[1] : z;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}

// C-tile row of accumulator register r for a lane in half h (= lane / 32).
__device__ __forceinline__ constexpr int tile_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

}  // namespace hsa_attn
