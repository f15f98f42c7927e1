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

// ---- remote-pair bucketing (chunk-major lists of the scattered pairs)
__global__ void prefill_zero_kernel(int* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// exclusive prefix sum of n counts into off[0..n] (off[n] = total), one
// workgroup of 1024 threads
__global__ __launch_bounds__(1024) void prefill_scan_kernel(const int* __restrict__ cnt, int* __restrict__ off,
                                                            int64_t n) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = tid * per, hi = min(n, lo + per);
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += cnt[i];
  part[tid] = s;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? part[tid - 1] : 0;
  for (int64_t i = lo; i < hi; ++i) {
    off[i] = run;
    run += cnt[i];
  }
  if (tid == 1023) off[n] = part[1023];
}

// pairs[pos] = row of each remote pair; pair_pos becomes the global position
__global__ void prefill_scatter_kernel(const int32_t* __restrict__ sel_idx, const int* __restrict__ off,
                                       int32_t* __restrict__ pair_pos, int32_t* __restrict__ pairs, int Hq, int G,
                                       int64_t T_len, int64_t Nc, int k, int64_t total) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= total) return;
  const int32_t inb = pair_pos[i];
  if (inb < 0) return;
  const int row = i / k;
  const int bh = row / (int)T_len;
  const int h = bh % Hq;
  const int b = bh / Hq;
  const int64_t bucket = ((int64_t)b * (Hq / G) + h / G) * Nc + sel_idx[i];
  const int32_t pos = off[bucket] + inb;
  pairs[pos] = (int32_t)row;
  pair_pos[i] = pos;
}


hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0,
                     st, p, n);
  return hipGetLastError();
}

hipError_t launch_exclusive_scan(const int* cnt, int* off, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, off, n);
  return hipGetLastError();
}

hipError_t launch_prefill_zero_counts(const PrefillArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;
  mark_launch(st);
  hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)std::min<int64_t>((nb + 255) / 256, 4096)), dim3(256), 0,
                     st, a.cnt, nb);
  mark_launch(st);
  return hipGetLastError();
}

hipError_t launch_prefill_bucketing(const PrefillArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const int64_t total = (int64_t)g.B * g.Hq * g.Tq * g.k;
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;
  const unsigned pb = (unsigned)((total + 255) / 256);
  mark_launch(st);
  hipLaunchKernelGGL(prefill_scan_kernel, dim3(1), dim3(1024), 0, st, a.cnt, a.off, nb);
  mark_launch(st);
  mark_launch(st);
  hipLaunchKernelGGL(prefill_scatter_kernel, dim3(pb), dim3(256), 0, st, a.sel_idx, a.off, a.pair_pos, a.pairs, g.Hq,
                     g.G, g.Tq, g.Nc, g.k, total);
  mark_launch(st);
  return hipGetLastError();
}

PrefillPlan plan_prefill(const Geometry& g, bool own_sel) {
  PrefillPlan p{};
  size_t off = 0;
  const size_t pairs = (size_t)g.B * g.Hq * (size_t)g.Tq * g.k;
  const size_t nb = (size_t)g.B * g.Hkv * (size_t)g.Nc;
  if (own_sel) {
    p.off_sel_idx = off;
    off = align_up_p(off + pairs * sizeof(int32_t), 256);
    p.off_sel_score = off;
    off = align_up_p(off + pairs * sizeof(float), 256);
  }
  p.off_pair_pos = off;
  off = align_up_p(off + pairs * sizeof(int32_t), 256);
  p.off_cnt = off;
  off = align_up_p(off + nb * sizeof(int), 256);
  p.off_off = off;
  off = align_up_p(off + (nb + 1) * sizeof(int), 256);
  p.off_pairs = off;
  off = align_up_p(off + pairs * sizeof(int32_t), 256);
  p.off_partial = off;
  off = align_up_p(off + pairs * g.D * sizeof(float), 256);
  p.off_vt = off;
  off = align_up_p(off + nb * kChunk * g.D * (g.bf16 ? 2 : 4), 256);
  p.bytes = off;
  return p;
}

size_t prefill_local_lds_bytes(const Geometry& g, int nbuf) {
  const size_t esz = g.bf16 ? 2 : 4;
  return (size_t)nbuf * 2 * kChunk * g.D * esz + (size_t)32 * g.G * g.k * 8;
}

// two chunk images when two such workgroups still fit in the 160 KiB of LDS
// of a CU; otherwise one image, which keeps two workgroups per CU (the
// 32-slot tables)
int prefill_local_buffers(const Geometry& g) { return 2 * prefill_local_lds_bytes(g, 2) <= 160 * 1024 ? 2 : 1; }

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
