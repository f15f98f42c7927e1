// Device helpers shared by the HSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hsa_attn.h"  // HSA_ATTN_DEBUG_* flag bits

namespace hsa_attn {

constexpr int kWave = 64;

// ---------------------------------------------------------------- debug build
// Compiled with HSA_ATTN_DEBUG=1 (libhsa_attn_debug.so), a kernel checks each
// index it reads back from the workspace before using it: a failed check
// sets its HSA_ATTN_DEBUG_* bit in the call's flag word `dbg` and the caller
// skips the access.  In the release library the check is the constant true.
#ifndef HSA_ATTN_DEBUG
#define HSA_ATTN_DEBUG 0
#endif
__device__ __forceinline__ bool dbg_ok(uint32_t* dbg, bool cond, uint32_t bit) {
#if HSA_ATTN_DEBUG
  if (!cond) {
    if (dbg) atomicOr(dbg, bit);
    return false;
  }
  return true;
#else
  (void)dbg;
  (void)cond;
  (void)bit;
  return true;
#endif
}

// ---------------------------------------------------------------- storage types
// Storage dtypes of Q/K/V/landmarks.  Every kernel reads 16-byte vectors; a
// lane holds kVec elements of one row per vector.
struct BF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kVec = 8;
};
struct FP32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kVec = 4;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Reinterpret bits through memcpy: a __builtin_bit_cast of a single element
// of an ext_vector value has been seen to read element 0 regardless of the
// index, so element-wise reinterpretation always goes through memory here.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  bf16x2 r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& w) {
  bf16x8 r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp64 -> bf16 bits with a single rounding to nearest even.  The value is
// first truncated to fp32 with the sticky bit folded into the last place
// (round-to-odd), which keeps 24 >= 8 + 2 bits, so the final RNE step to bf16
// gives the correctly rounded result (no double-rounding error).
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- lane exchange
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of W lanes (W in {4, 8, 16, 32, 64}); every lane of
// a group ends with the same bits.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  if constexpr (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (W >= 32) v += __shfl_xor(v, 16);
  if constexpr (W >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  if constexpr (W >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (W >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  if constexpr (W >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (W >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// ---------------------------------------------------------------- selection order
// Total order of (score, chunk index) candidates: higher score first, lower
// index first among equal scores.  -0.0 == +0.0 under the float compare.
__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Wave-uniform broadcast of lane `src` (src must be uniform).
__device__ __forceinline__ float bcast_f(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}
__device__ __forceinline__ int bcast_i(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Whole-wave shift by one lane toward higher lanes (DPP wave_shr:1); lane 0
// keeps its own value.
__device__ __forceinline__ int wave_shr1(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x138, 0xf, 0xf, false); }

// A wave-resident sorted list of up to 64 candidates: lane i holds the i-th
// best.  Empty slots hold (-inf, INT_MAX).
struct WaveTopK {
  float s;
  int i;
  __device__ __forceinline__ void init() {
    s = -__builtin_inff();
    i = 0x7fffffff;
  }
  // Offer one wave-uniform candidate (cs, ci); keeps the best `k` entries.
  __device__ __forceinline__ void insert(float cs, int ci, int k) {
    const int lane = __lane_id();
    // entries strictly better than the candidate stay in place
    const bool keep = better(s, i, cs, ci);
    const uint64_t m = __ballot(keep) & ((k >= 64) ? ~0ull : ((1ull << k) - 1));
    const int pos = __popcll(m);
    if (pos >= k) return;
    const float ps = __int_as_float(wave_shr1(__float_as_int(s)));
    const int pi = wave_shr1(i);
    if (lane > pos) {
      s = ps;
      i = pi;
    }
    if (lane == pos) {
      s = cs;
      i = ci;
    }
  }
  // Current k-th best (the admission threshold), wave-uniform.
  __device__ __forceinline__ void kth(int k, float& ts, int& ti) const {
    ts = bcast_f(s, k - 1);
    ti = bcast_i(i, k - 1);
  }
};

// Offer the wave's 64 candidates (one per lane; inactive lanes pass
// valid=false) to the list, in lane order.
__device__ __forceinline__ void offer_wave(WaveTopK& list, int k, float cs, int ci, bool valid) {
  float ts;
  int ti;
  list.kth(k, ts, ti);
  uint64_t m = __ballot(valid && better(cs, ci, ts, ti));
  while (m) {
    const int src = __builtin_ctzll(m);
    m &= m - 1;
    const float s = bcast_f(cs, src);
    const int i = bcast_i(ci, src);
    list.kth(k, ts, ti);
    if (better(s, i, ts, ti)) list.insert(s, i, k);
  }
}

}  // namespace hsa_attn
