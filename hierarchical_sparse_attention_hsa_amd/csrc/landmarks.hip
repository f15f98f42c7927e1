// Landmark builder: mean of each chunk's keys (skill card "Every Token
// Counts 16m Context", section "Implementation": mean pooling of a chunk's
// tokens).  One wave per (b, g, chunk); HBM-bound streaming read of K.
//
// A lane owns one 16-byte column slice of a key row; the wave reads whole
// rows per instruction (LPR lanes per row, RPI = 64/LPR rows per load), so
// every load instruction covers 1 KiB of consecutive bytes.  Sums are kept in
// fp64, which is exact for bf16 keys; the mean is rounded once to the storage
// dtype.  append_kv_kernel (incremental decoding) writes one new token per
// sequence and builds the landmark of a chunk it completes the same way.
#include "common.hpp"
#include "kernels.hpp"

namespace hsa_attn {

template <typename T, int D>
__global__ __launch_bounds__(256) void landmarks_kernel(const typename T::storage* __restrict__ k,
                                                        typename T::storage* __restrict__ lm,
                                                        int64_t T_len, int S, int64_t Nc,
                                                        int64_t c0, int64_t n_chunks,
                                                        int64_t total) {
  constexpr int EPL = T::kVec;            // elements per lane
  constexpr int LPR = D / EPL;            // lanes per row
  constexpr int RPI = kWave / LPR;        // rows per load instruction
  const int lane = __lane_id();
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (item >= total) return;
  const int64_t bg = item / n_chunks;     // b * Hkv + g
  const int64_t c = c0 + item % n_chunks;
  const int col = (lane % LPR) * EPL;
  const int r0 = lane / LPR;
  const typename T::storage* src = k + (bg * T_len + c * S) * D + col;

  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;

  // rows r0, r0 + RPI, ...; unrolled so that several loads are in flight
  constexpr int U = 8;
  int r = r0;
  for (; r + (U - 1) * RPI < S; r += U * RPI) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)(r + u * RPI) * D));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (T::kBytes == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += (double)bf16_lo(v[u][w]);
          acc[2 * w + 1] += (double)bf16_hi(v[u][w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] += (double)__uint_as_float(v[u][w]);
      }
    }
  }
  for (; r < S; r += RPI) {
    u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)r * D);
    if constexpr (T::kBytes == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += (double)bf16_lo(v[w]);
        acc[2 * w + 1] += (double)bf16_hi(v[w]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += (double)__uint_as_float(v[w]);
    }
  }
  // combine the RPI row groups: lanes that share (lane % LPR)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane < LPR) {
    typename T::storage* dst = lm + (bg * Nc + c) * D + col;
    if constexpr (T::kBytes == 2) {
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = f64_to_bf16_bits(acc[2 * w] / (double)S);
        const uint32_t hi = f64_to_bf16_bits(acc[2 * w + 1] / (double)S);
        o[w] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(dst) = o;
    } else {
      f32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __double2float_rn(acc[w] / (double)S);
      *reinterpret_cast<f32x4*>(dst) = o;
    }
  }
}

template <typename T, int D>
static hipError_t launch_landmarks_t(const LandmarkArgs& a, hipStream_t st) {
  const int64_t total = a.bh * (a.c1 - a.c0);
  if (total <= 0) return hipSuccess;
  constexpr int kWavesPerBlock = 4;
  const int64_t blocks = (total + kWavesPerBlock - 1) / kWavesPerBlock;
  launch_kernel((landmarks_kernel<T, D>), dim3((unsigned)blocks), dim3(kWave * kWavesPerBlock), 0, st,
                static_cast<const typename T::storage*>(a.k), static_cast<typename T::storage*>(a.lm),
                a.T, a.S, a.Nc, a.c0, a.c1 - a.c0, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- append
// Incremental decode: one new token per sequence is written at position
// lens[b] of the K and V caches (capacity T); when it completes a chunk, the
// chunk's landmark is built on the spot (same fp64 sum and single rounding
// as landmarks_kernel; the new key is taken from registers, the chunk's
// other S-1 keys from the cache); lens[b] then advances by one.  One
// workgroup per sequence, one wave per KV head (strided).  A sequence whose
// cache is full (lens[b] >= T) is left unchanged.
template <typename T, int D>
__global__ __launch_bounds__(256) void append_kv_kernel(const typename T::storage* __restrict__ k_new,
                                                        const typename T::storage* __restrict__ v_new,
                                                        typename T::storage* __restrict__ kc,
                                                        typename T::storage* __restrict__ vc,
                                                        typename T::storage* __restrict__ lm,
                                                        int64_t* __restrict__ lens, int Hkv, int64_t T_len, int S,
                                                        int64_t Nc) {
  using st = typename T::storage;
  constexpr int EPL = T::kVec;      // elements per lane (16 bytes)
  constexpr int LPR = D / EPL;      // lanes per row
  constexpr int RPI = kWave / LPR;  // rows per load instruction
  __shared__ int64_t pos_s;
  const int b = blockIdx.x;
  const int lane = __lane_id(), wave = threadIdx.x / kWave, waves = blockDim.x / kWave;
  if (threadIdx.x == 0) pos_s = lens[b];
  __syncthreads();
  const int64_t pos = pos_s;
  if (pos < 0 || pos >= T_len) return;
  const int col = (lane % LPR) * EPL;
  const int r0 = lane / LPR;
  const bool completes = (pos + 1) % S == 0;
  for (int g = wave; g < Hkv; g += waves) {
    const int64_t bg = (int64_t)b * Hkv + g;
    u32x4 kn = {0u, 0u, 0u, 0u};
    if (lane < LPR) {
      kn = *reinterpret_cast<const u32x4*>(k_new + bg * D + col);
      const u32x4 vn = *reinterpret_cast<const u32x4*>(v_new + bg * D + col);
      *reinterpret_cast<u32x4*>(kc + (bg * T_len + pos) * D + col) = kn;
      *reinterpret_cast<u32x4*>(vc + (bg * T_len + pos) * D + col) = vn;
    }
    if (!completes) continue;
    const int64_t c = (pos + 1) / S - 1;
    const st* src = kc + (bg * T_len + c * S) * D + col;
    double acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
    auto add = [&](const u32x4& v) {
      if constexpr (T::kBytes == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += (double)bf16_lo(v[w]);
          acc[2 * w + 1] += (double)bf16_hi(v[w]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] += (double)__uint_as_float(v[w]);
      }
    };
    for (int r = r0; r < S - 1; r += RPI) add(*reinterpret_cast<const u32x4*>(src + (int64_t)r * D));
    if (lane < LPR) add(kn);  // the chunk's last key (row S-1), held by row group 0
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (lane < LPR) {
      st* dst = lm + (bg * Nc + c) * D + col;
      if constexpr (T::kBytes == 2) {
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = f64_to_bf16_bits(acc[2 * w] / (double)S);
          const uint32_t hi = f64_to_bf16_bits(acc[2 * w + 1] / (double)S);
          o[w] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dst) = o;
      } else {
        f32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) o[w] = __double2float_rn(acc[w] / (double)S);
        *reinterpret_cast<f32x4*>(dst) = o;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) lens[b] = pos + 1;
}

template <typename T, int D>
static hipError_t launch_append_t(const AppendArgs& a, hipStream_t st) {
  if (a.B <= 0) return hipSuccess;
  using stg = typename T::storage;
  const int waves = a.Hkv < 4 ? a.Hkv : 4;
  launch_kernel((append_kv_kernel<T, D>), dim3(a.B), dim3(kWave * waves), 0, st,
                static_cast<const stg*>(a.k_new), static_cast<const stg*>(a.v_new), static_cast<stg*>(a.k),
                static_cast<stg*>(a.v), static_cast<stg*>(a.lm), a.lens, a.Hkv, a.T, a.S, a.Nc);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 128 ? launch_append_t<BF16, 128>(a, st) : launch_append_t<BF16, 64>(a, st);
  return a.D == 128 ? launch_append_t<FP32, 128>(a, st) : launch_append_t<FP32, 64>(a, st);
}

hipError_t launch_landmarks(const LandmarkArgs& a, hipStream_t st) {
  if (a.bf16) return a.D == 128 ? launch_landmarks_t<BF16, 128>(a, st) : launch_landmarks_t<BF16, 64>(a, st);
  return a.D == 128 ? launch_landmarks_t<FP32, 128>(a, st) : launch_landmarks_t<FP32, 64>(a, st);
}

}  // namespace hsa_attn
