// HSA decode: B single-token queries, each after its own cache of T tokens.
//
// Pipeline on one stream (skill card "Every Token Counts 16m Context",
// sections "Core Technique" and "Implementation"):
//   1. decode_scan   per (b, g, split): stream a contiguous range of landmark
//                    rows once, score them against the G query heads of the
//                    group (bandwidth-bound GEMV, fp32 accumulation) and keep
//                    the split-local top-k of every head.
//   2. decode_merge  per (b, h): merge the split candidates into the global
//                    top-k under the total order (score desc, index asc).
//   3. decode_attn   per (b, g, selected (head, slot) pair): each distinct
//                    chunk of the group is loaded once; softmax attention of
//                    every head that selected it; writes the per-chunk output.
//   4. decode_fuse   per (b, h): softmax over the kept scores, weighted sum.
// The score vector never reaches HBM; the selected K/V tiles are read once
// per KV group.
#include <climits>

#include "common.hpp"
#include "kernels.hpp"

namespace hsa_attn {

constexpr int kScanThreads = 256;
constexpr int kScanUnroll = 4;

// dot product of a 16-byte slice of a bf16 landmark row with the matching
// slice of a bf16 query (both as packed pairs), fp32 accumulation
__device__ __forceinline__ float dot_slice(const u32x4& a, const u32x4& b, BF16) {
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a[w]), as_bf16x2(b[w]), acc, false);
  return acc;
}
__device__ __forceinline__ float dot_slice(const u32x4& a, const u32x4& b, FP32) {
  float acc = 0.0f;
#pragma unroll
  for (int w = 0; w < 4; ++w) acc = fmaf(__uint_as_float(a[w]), __uint_as_float(b[w]), acc);
  return acc;
}

// ---------------------------------------------------------------- 1. scan
template <typename T, int D, int G>
__global__ __launch_bounds__(kScanThreads) void decode_scan_kernel(const typename T::storage* __restrict__ q,
                                                                   const typename T::storage* __restrict__ lm,
                                                                   float2* __restrict__ cand, int Hkv, int64_t Nc,
                                                                   int rows_per_split, int splits, int k,
                                                                   float scale) {
  constexpr int EPL = T::kVec;
  constexpr int LPR = D / EPL;       // lanes per landmark row
  constexpr int RPI = kWave / LPR;   // rows per load instruction
  constexpr int WAVES = kScanThreads / kWave;
  constexpr int ROWS_PER_ITER = WAVES * kScanUnroll * RPI;
  static_assert(LPR >= G, "each head's score is written by one lane of the row group");
  extern __shared__ float sc[];  // [G][rows_per_split]

  const int b = blockIdx.z, g = blockIdx.y, sp = blockIdx.x;
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int64_t r_begin = (int64_t)sp * rows_per_split;
  const int n = (int)min((int64_t)rows_per_split, Nc - r_begin);
  const int col = (lane % LPR) * EPL;

  u32x4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hkv * G + (int64_t)g * G + h) * D + col);

  const typename T::storage* base = lm + (((int64_t)b * Hkv + g) * Nc + r_begin) * D + col;
  for (int it = 0; it < n; it += ROWS_PER_ITER) {
    u32x4 v[kScanUnroll];
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int r = it + (wave * kScanUnroll + u) * RPI + lane / LPR;
      if (r < n) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)r * D));
      else v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int r = it + (wave * kScanUnroll + u) * RPI + lane / LPR;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s = group_sum<LPR>(dot_slice(v[u], qv[h], T{}));
        if (r < n && (lane % LPR) == h) sc[h * rows_per_split + r] = s * scale + 0.0f;
      }
    }
  }
  __syncthreads();

  for (int h = wave; h < G; h += WAVES) {
    WaveTopK list;
    list.init();
    for (int i0 = 0; i0 < n; i0 += kWave) {
      const int r = i0 + lane;
      const bool valid = r < n;
      const float s = valid ? sc[h * rows_per_split + r] : -__builtin_inff();
      offer_wave(list, k, s, (int)(r_begin + r), valid);
    }
    if (lane < k) {
      float2 c;
      c.x = list.s;
      c.y = __int_as_float(list.i);
      cand[((((int64_t)b * Hkv + g) * splits + sp) * G + h) * k + lane] = c;
    }
  }
}

// ---------------------------------------------------------------- 2. merge
__global__ __launch_bounds__(kWave) void decode_merge_kernel(const float2* __restrict__ cand,
                                                             int32_t* __restrict__ sel_idx,
                                                             float* __restrict__ sel_score, int Hq, int Hkv,
                                                             int G, int splits, int k) {
  const int bh = blockIdx.x;
  const int b = bh / Hq, h = bh % Hq, g = h / G, hh = h % G;
  const int lane = __lane_id();
  WaveTopK list;
  list.init();
  const int total = splits * k;
  for (int i0 = 0; i0 < total; i0 += kWave) {
    const int j = i0 + lane;
    bool valid = j < total;
    float s = -__builtin_inff();
    int ci = INT_MAX;
    if (valid) {
      const int sp = j / k, e = j % k;
      const float2 c = cand[((((int64_t)b * Hkv + g) * splits + sp) * G + hh) * k + e];
      s = c.x;
      ci = __float_as_int(c.y);
      valid = ci != INT_MAX;
    }
    offer_wave(list, k, s, ci, valid);
  }
  if (lane < k) {
    const bool ok = list.i != INT_MAX;
    sel_idx[(int64_t)bh * k + lane] = ok ? list.i : -1;
    sel_score[(int64_t)bh * k + lane] = ok ? list.s : -__builtin_inff();
  }
}

// ---------------------------------------------------------------- 3. chunk attention
// One workgroup per (b, g, j) where j enumerates the G*k (head, slot) pairs of
// the group; the pair that first names a chunk owns it, so every distinct
// selected chunk of the group is read from HBM once.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(const typename T::storage* __restrict__ q,
                                                          const typename T::storage* __restrict__ kc,
                                                          const typename T::storage* __restrict__ vc,
                                                          const int32_t* __restrict__ sel_idx,
                                                          float* __restrict__ partial, int Hkv, int64_t T_len,
                                                          int k, float scale) {
  constexpr int S = 64;                 // tokens per chunk (4 threads per token)
  constexpr int EPT = D / 4;            // key elements per thread
  constexpr int LOADS = EPT * T::kBytes / 16;
  constexpr int NT = 256 / D;           // threads per output column in P.V
  constexpr int TPT = S / NT;           // tokens per thread in P.V
  using st = typename T::storage;
  __shared__ int sel[G * 64];
  __shared__ int slot_of[G];
  __shared__ float qs[G][D];
  __shared__ float red[256];
  __shared__ st vs[S * D];

  const int b = blockIdx.z, g = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int Hq = Hkv * G;
  for (int i = tid; i < G * k; i += 256) sel[i] = sel_idx[((int64_t)b * Hq + (int64_t)g * G + i / k) * k + i % k];
  __syncthreads();
  const int c = sel[j];
  if (c < 0) return;
  bool dup = false;
  for (int i = tid; i < j; i += 256) dup |= sel[i] == c;
  if (__syncthreads_or(dup)) return;

  // K slice of this thread into registers, V tile into LDS, queries into LDS
  const int t = tid / 4, qd = tid % 4;
  const int64_t tile = (((int64_t)b * Hkv + g) * T_len + (int64_t)c * S) * D;
  u32x4 kr[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i)
    kr[i] = *reinterpret_cast<const u32x4*>(kc + tile + (int64_t)t * D + qd * EPT + i * (16 / T::kBytes));
  for (int i = tid; i < S * D * T::kBytes / 16; i += 256)
    reinterpret_cast<u32x4*>(vs)[i] = reinterpret_cast<const u32x4*>(vc + tile)[i];
  for (int i = tid; i < G * D; i += 256) {
    const st x = q[((int64_t)b * Hq + (int64_t)g * G) * D + i];
    if constexpr (T::kBytes == 2) qs[i / D][i % D] = __uint_as_float((uint32_t)x << 16);
    else qs[i / D][i % D] = x;
  }
  if (wave < G && lane < k) {
    const uint64_t m = __ballot(sel[wave * k + lane] == c);
    if (lane == 0) slot_of[wave] = m ? __builtin_ctzll(m) : -1;
  }
  for (int hh = 4 + wave; hh < G; hh += 4) {  // G == 8: waves cover two heads each
    const uint64_t m = __ballot(lane < k && sel[hh * k + lane] == c);
    if (lane == 0) slot_of[hh] = m ? __builtin_ctzll(m) : -1;
  }
  __syncthreads();

  for (int hh = 0; hh < G; ++hh) {
    const int slot = slot_of[hh];
    if (slot < 0) continue;
    // logits: 4 threads per token
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int e = qd * EPT + i * (16 / T::kBytes);
        if constexpr (T::kBytes == 2) {
          acc = fmaf(bf16_lo(kr[i][w]), qs[hh][e + 2 * w], acc);
          acc = fmaf(bf16_hi(kr[i][w]), qs[hh][e + 2 * w + 1], acc);
        } else {
          acc = fmaf(__uint_as_float(kr[i][w]), qs[hh][e + w], acc);
        }
      }
    }
    acc = group_sum<4>(acc) * scale;
    if (qd == 0) red[t] = acc;
    __syncthreads();
    // softmax over the 64 tokens, computed redundantly by every wave (lane = token)
    const float l = red[lane];
    const float mx = group_max<64>(l);
    const float p = __expf(l - mx);
    const float den = group_sum<64>(p);
    const float pn = p / den;
    __syncthreads();  // red[] is reused below
    // P.V: thread -> output column d, token range
    const int d = tid % D, tr = tid / D;
    float o = 0.0f;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int tok = tr * TPT + i;
      const float pt = __shfl(pn, tok);
      float vv;
      if constexpr (T::kBytes == 2) vv = __uint_as_float((uint32_t)vs[tok * D + d] << 16);
      else vv = vs[tok * D + d];
      o = fmaf(pt, vv, o);
    }
    red[tid] = o;
    __syncthreads();
    if (tid < D) {
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < NT; ++r) sum += red[r * D + tid];
      partial[(((int64_t)b * Hq + (int64_t)g * G + hh) * k + slot) * D + tid] = sum;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- 4. fusion
__global__ void decode_fuse_kernel(const float* __restrict__ partial, const int32_t* __restrict__ sel_idx,
                                   const float* __restrict__ sel_score, float* __restrict__ out, int k, int D) {
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const float mx = sel_score[bh * k];
  float den = 0.0f, num = 0.0f;
  for (int s = 0; s < k; ++s) {
    if (sel_idx[bh * k + s] < 0) break;
    const float w = __expf(sel_score[bh * k + s] - mx);
    den += w;
    num = fmaf(w, partial[(bh * k + s) * D + d], num);
  }
  out[bh * D + d] = den > 0.0f ? num / den : 0.0f;
}

// ---------------------------------------------------------------- host side
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

DecodePlan plan_decode(const Geometry& g, bool own_sel) {
  DecodePlan p{};
  const int64_t bh = (int64_t)g.B * g.Hkv;
  int64_t rows = (g.Nc * bh + 2047) / 2048;
  rows = (rows + 63) / 64 * 64;
  rows = rows < 256 ? 256 : (rows > 2048 ? 2048 : rows);
  p.rows_per_split = (int)rows;
  p.splits = g.Nc > 0 ? (int)((g.Nc + rows - 1) / rows) : 0;
  size_t off = 0;
  p.off_cand = off;
  off = align_up(off + (size_t)bh * p.splits * g.G * g.k * sizeof(float2), 256);
  const size_t rows_q = (size_t)g.B * g.Hq;
  if (own_sel) {
    p.off_sel_idx = off;
    off = align_up(off + rows_q * g.k * sizeof(int32_t), 256);
    p.off_sel_score = off;
    off = align_up(off + rows_q * g.k * sizeof(float), 256);
  }
  p.off_partial = off;
  off = align_up(off + rows_q * g.k * g.D * sizeof(float), 256);
  p.bytes = off;
  return p;
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  const Geometry& g = a.g;
  char* ws = static_cast<char*>(a.ws);
  float2* cand = reinterpret_cast<float2*>(ws + p.off_cand);
  float* partial = reinterpret_cast<float*>(ws + p.off_partial);
  const float scale = 1.0f / sqrtf((float)D);
  using stg = typename T::storage;
  if (p.splits > 0) {
    const size_t lds = (size_t)G * p.rows_per_split * sizeof(float);
    mark_launch(st);
    hipLaunchKernelGGL((decode_scan_kernel<T, D, G>), dim3(p.splits, g.Hkv, g.B), dim3(kScanThreads), lds, st,
                       static_cast<const stg*>(a.q), static_cast<const stg*>(a.lm), cand, g.Hkv, g.Nc,
                       p.rows_per_split, p.splits, g.k, scale);
    mark_launch(st);
  }
  mark_launch(st);
  hipLaunchKernelGGL(decode_merge_kernel, dim3(g.B * g.Hq), dim3(kWave), 0, st, cand, a.sel_idx, a.sel_score,
                     g.Hq, g.Hkv, G, p.splits, g.k);
  mark_launch(st);
  if (p.splits > 0) {
    mark_launch(st);
    hipLaunchKernelGGL((decode_attn_kernel<T, D, G>), dim3(G * g.k, g.Hkv, g.B), dim3(256), 0, st,
                       static_cast<const stg*>(a.q), static_cast<const stg*>(a.k), static_cast<const stg*>(a.v),
                       a.sel_idx, partial, g.Hkv, g.T, g.k, scale);
    mark_launch(st);
  }
  mark_launch(st);
  hipLaunchKernelGGL(decode_fuse_kernel, dim3(g.B * g.Hq), dim3(D), 0, st, partial, a.sel_idx, a.sel_score, a.out,
                     g.k, D);
  mark_launch(st);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_decode_t<T, D, 1>(a, p, st);
    case 2: return launch_decode_t<T, D, 2>(a, p, st);
    case 4: return launch_decode_t<T, D, 4>(a, p, st);
    default: return launch_decode_t<T, D, 8>(a, p, st);
  }
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  if (a.g.bf16) return a.g.D == 128 ? launch_decode_d<BF16, 128>(a, p, st) : launch_decode_d<BF16, 64>(a, p, st);
  return a.g.D == 128 ? launch_decode_d<FP32, 128>(a, p, st) : launch_decode_d<FP32, 64>(a, p, st);
}

}  // namespace hsa_attn
