// HSA prefill: host-side planning and dispatch.  The kernels live in
// prefill_kernels.hpp and are instantiated in prefill_inst_*.hip.
#include <algorithm>

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
HSA_ATTN_PREFILL_EXTERN(BF16, 128, 64)
HSA_ATTN_PREFILL_EXTERN(BF16, 64, 64)
HSA_ATTN_PREFILL_EXTERN(FP32, 128, 64)
HSA_ATTN_PREFILL_EXTERN(FP32, 64, 64)

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

// exclusive prefix sums of blockIdx.x's n counts cnt[x * n ..] into
// off[x * (n + 1) ..] (off[.. n] = the total); one workgroup of 1024
// threads per array: each thread sums a contiguous run, the runs' sums are
// scanned by the waves (shuffles) and across the waves, then each thread
// writes its run's offsets
__global__ __launch_bounds__(1024) void prefill_scan_kernel(const int* __restrict__ cnt, int* __restrict__ off,
                                                            int64_t n) {
  __shared__ int wsum[1024 / kWave];
  cnt += (int64_t)blockIdx.x * n;
  off += (int64_t)blockIdx.x * (n + 1);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = min(n, tid * per), hi = min(n, lo + per);
  int s = 0;
  for (int64_t i = lo; i < hi; ++i) s += cnt[i];
  int x = s;  // inclusive scan over the wave
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  int run = base + x - s;
  for (int64_t i = lo; i < hi; ++i) {
    off[i] = run;
    run += cnt[i];
  }
  if (tid == 1023) off[n] = base + x;
}

// For the remote pairs of the rows [r0, r0 + rn) of every (b, h), one
// thread per row: the row's slab is sl = (t - r0) / slab_rows, whose
// bucket offsets are off[sl * (nb + 1) ..]; pairs[sl * slab_cap + pos] =
// the pair's query row (b * Hq + h) * T_len + t, and pair_pos becomes pos,
// the position in the slab's pair list.  K4 > 0: k = 4 * K4, the row's
// slots as 16-byte loads.
template <int K4>
__global__ __launch_bounds__(256) void prefill_scatter_kernel(const int32_t* __restrict__ sel_idx,
                                                              const int* __restrict__ off,
                                                              int32_t* __restrict__ pair_pos,
                                                              int32_t* __restrict__ pairs, int Hq, int G,
                                                              int64_t T_len, int64_t Nc, int k, int64_t r0,
                                                              int64_t rn, int64_t slab_rows, int64_t slab_cap,
                                                              int64_t nb, int64_t nrows, uint32_t* __restrict__ dbg) {
  const int64_t rl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (rl >= nrows) return;
  const int64_t bh = rl / rn, tr = rl % rn;
  const int64_t row = bh * T_len + r0 + tr;
  const int h = (int)(bh % Hq);
  const int b = (int)(bh / Hq);
  const int64_t sl = tr / slab_rows;
  const int* o = off + sl * (nb + 1) + ((int64_t)b * (Hq / G) + h / G) * Nc;
  int32_t* pp = pair_pos + row * k;
  const int32_t* si = sel_idx + row * k;
  int32_t* pr = pairs + sl * slab_cap;
  if constexpr (K4 > 0) {
    u32x4 p4[K4], c4[K4];
#pragma unroll
    for (int e4 = 0; e4 < K4; ++e4) {
      p4[e4] = *reinterpret_cast<const u32x4*>(pp + 4 * e4);
      c4[e4] = *reinterpret_cast<const u32x4*>(si + 4 * e4);
    }
    // every slot's bucket offset is read at once (a slot that is not a
    // chunk-major pair reads bucket 0), so the row's offsets arrive in one
    // round trip instead of one per pair
    int ob[K4][4];
#pragma unroll
    for (int e4 = 0; e4 < K4; ++e4)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = (int)c4[e4][u];
        ob[e4][u] = o[(int)p4[e4][u] >= 0 && c >= 0 && c < Nc ? c : 0];
      }
#pragma unroll
    for (int e4 = 0; e4 < K4; ++e4) {
      bool any = false;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int inb = (int)p4[e4][u];
        if (inb >= 0) {
          const int c = (int)c4[e4][u];
          if (!dbg_ok(dbg, c >= 0 && c < Nc, HSA_ATTN_DEBUG_SCATTER_CHUNK)) continue;
          const int pos = ob[e4][u] + inb;
          if (!dbg_ok(dbg, pos >= 0 && pos < slab_cap, HSA_ATTN_DEBUG_SCATTER_POS)) continue;
          pr[pos] = (int32_t)row;
          p4[e4][u] = (uint32_t)pos;
          any = true;
        }
      }
      if (any) *reinterpret_cast<u32x4*>(pp + 4 * e4) = p4[e4];
    }
  } else {
    for (int e = 0; e < k; ++e) {
      const int inb = pp[e];
      if (inb < 0) continue;
      const int c = si[e];
      if (!dbg_ok(dbg, c >= 0 && c < Nc, HSA_ATTN_DEBUG_SCATTER_CHUNK)) continue;
      const int pos = o[c] + inb;
      if (!dbg_ok(dbg, pos >= 0 && pos < slab_cap, HSA_ATTN_DEBUG_SCATTER_POS)) continue;
      pr[pos] = (int32_t)row;
      pp[e] = pos;
    }
  }
}

hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t st) {
  launch_kernel(prefill_zero_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 4096)), dim3(256), 0, st, p,
                n);
  return hipGetLastError();
}

hipError_t launch_exclusive_scan(const int* cnt, int* off, int64_t n, hipStream_t st) {
  launch_kernel(prefill_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, off, n);
  return hipGetLastError();
}

hipError_t launch_prefill_zero_counts(const PrefillArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc * a.slab_group;
  launch_kernel(prefill_zero_kernel, dim3((unsigned)std::min<int64_t>((nb + 255) / 256, 4096)), dim3(256), 0,
                     st, a.cnt, nb);
  return hipGetLastError();
}

hipError_t launch_prefill_bucketing(const PrefillArgs& a, int nslab, int64_t r0, int64_t rn, hipStream_t st) {
  const Geometry& g = a.g;
  const int64_t nrows = (int64_t)g.B * g.Hq * rn;
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;
  const int64_t cap = (int64_t)g.B * g.Hq * a.slab_rows * g.k;  // one slab's pair list
  const unsigned pb = (unsigned)((nrows + 255) / 256);
  launch_kernel(prefill_scan_kernel, dim3((unsigned)nslab), dim3(1024), 0, st, a.cnt, a.off, nb);
#define HSA_SCATTER(K4)                                                                                         \
  launch_kernel(prefill_scatter_kernel<K4>, dim3(pb), dim3(256), 0, st, a.sel_idx, a.off, a.pair_pos, a.pairs, \
                g.Hq, g.G, g.Tq, g.Nc, g.k, r0, rn, a.slab_rows, cap, nb, nrows, a.dbg)
  switch (g.k) {
    case 16: HSA_SCATTER(4); break;
    case 32: HSA_SCATTER(8); break;
    case 64: HSA_SCATTER(16); break;
    default: HSA_SCATTER(0); break;
  }
#undef HSA_SCATTER
  return hipGetLastError();
}

// Workspace layout: [selection if the library keeps it] pair positions,
// bucket counts and offsets, transposed V (all per call), then one slab's
// pair list and pair outputs.
void prefill_workspace_parts(const Geometry& g, bool own_sel, size_t* fixed, size_t* per_row) {
  const size_t pairs = (size_t)g.B * g.Hq * (size_t)g.Tq * g.k;
  const size_t nb = (size_t)g.B * g.Hkv * (size_t)g.Nc;
  size_t f = 0;
  if (own_sel) f += align_up_p(pairs * sizeof(int32_t), 256) + align_up_p(pairs * sizeof(float), 256);
  // (an estimate for planning: the counts, offsets and pair lists of a
  // group of slabs are taken as those of one slab and of every row)
  f += 2 * align_up_p(pairs * sizeof(int32_t), 256) + align_up_p(nb * sizeof(int), 256) +
       align_up_p((nb + 1) * sizeof(int), 256) + align_up_p(nb * kChunk * g.D * (g.bf16 ? 2 : 4), 256);
  *fixed = f;
  *per_row = (size_t)g.B * g.Hq * g.k * g.D * sizeof(float);
}

PrefillPlan plan_prefill_slab(const Geometry& g, bool own_sel, int64_t slab_rows) {
  PrefillPlan p{};
  const int64_t nqc = (g.Tq + kChunk - 1) / kChunk;
  // equal slabs of whole 64-row chunks: the fewest slabs of at most
  // slab_rows rows, then the chunks spread evenly over them
  int64_t cps = std::max<int64_t>(1, slab_rows / kChunk);
  if (nqc > 0) {
    cps = std::min(cps, nqc);
    const int64_t nslab = (nqc + cps - 1) / cps;
    cps = (nqc + nslab - 1) / nslab;
  } else {
    cps = 1;  // no query rows: the smallest plan (the call returns before using it)
  }
  p.slab_rows = cps * kChunk;
  const int64_t nslab = nqc > 0 ? (nqc + cps - 1) / cps : 1;
  p.slab_group = (int)std::min<int64_t>(nslab, kPrefillCountSlabs);
  size_t off = 0;
  const size_t pairs = (size_t)g.B * g.Hq * (size_t)g.Tq * g.k;
  const size_t spairs = (size_t)g.B * g.Hq * (size_t)p.slab_rows * g.k;
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
  off = align_up_p(off + nb * p.slab_group * sizeof(int), 256);
  p.off_off = off;
  off = align_up_p(off + (nb + 1) * p.slab_group * sizeof(int), 256);
  p.off_vt = off;
  off = align_up_p(off + nb * kChunk * g.D * (g.bf16 ? 2 : 4), 256);
  p.off_pairs = off;
  off = align_up_p(off + spairs * p.slab_group * sizeof(int32_t), 256);
  p.off_partial = off;
  off = align_up_p(off + spairs * g.D * sizeof(float), 256);
  p.bytes = off;
  return p;
}

PrefillPlan plan_prefill_for(const Geometry& g, bool own_sel, size_t bytes) {
  size_t fixed, per_row;
  prefill_workspace_parts(g, own_sel, &fixed, &per_row);
  const int64_t nqc = std::max<int64_t>(1, (g.Tq + kChunk - 1) / kChunk);
  // the most chunks per slab whose plan fits (the plan's size only shrinks
  // as its slabs do; the estimate ignores the two arrays' alignment)
  int64_t cps = bytes > fixed ? (int64_t)std::min<size_t>((bytes - fixed) / (per_row * kChunk), (size_t)nqc) : 0;
  while (cps > 0 && plan_prefill_slab(g, own_sel, cps * kChunk).bytes > bytes) --cps;
  if (cps == 0) {
    PrefillPlan p = plan_prefill_slab(g, own_sel, kChunk);  // bytes: the smallest workable workspace
    p.slab_rows = 0;
    return p;
  }
  return plan_prefill_slab(g, own_sel, cps * kChunk);
}

PrefillPlan plan_prefill(const Geometry& g, bool own_sel) {
  size_t fixed, per_row;
  prefill_workspace_parts(g, own_sel, &fixed, &per_row);
  const int64_t rows = (int64_t)std::max<size_t>(1, kPrefillSlabBudget / (per_row * kChunk)) * kChunk;
  return plan_prefill_slab(g, own_sel, rows);
}

size_t prefill_local_lds_bytes(const Geometry& g, int nbuf) {
  const size_t esz = g.bf16 ? 2 : 4;
  return (size_t)nbuf * 2 * kChunk * g.D * esz + (size_t)32 * g.G * g.k * 8;
}

// two chunk images when two such workgroups still fit in the 160 KiB of LDS
// of a CU; otherwise one image, which keeps two workgroups per CU (the
// 32-slot tables)
int prefill_local_buffers(const Geometry& g) { return 2 * prefill_local_lds_bytes(g, 2) <= 160 * 1024 ? 2 : 1; }

// the register top-k list holds 16, 32 or 64 entries: the shortest that
// holds k (64-entry lists serve query groups of at most 4 heads)
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  const bool shortlist = a.g.k <= 16, longlist = a.g.k > 32;
  if (a.g.bf16) {
    if (a.g.D == 128) {
      if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D128_K16, BF16, 128, 16);
      if (longlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D128_K64, BF16, 128, 64);
      HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D128_K32, BF16, 128, 32);
    }
    if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D64_K16, BF16, 64, 16);
    if (longlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D64_K64, BF16, 64, 64);
    HSA_ATTN_CALL(HSA_ATTN_HAVE_BF16_D64_K32, BF16, 64, 32);
  }
  if (a.g.D == 128) {
    if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D128_K16, FP32, 128, 16);
    if (longlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D128_K64, FP32, 128, 64);
    HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D128_K32, FP32, 128, 32);
  }
  if (shortlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D64_K16, FP32, 64, 16);
  if (longlist) HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D64_K64, FP32, 64, 64);
  HSA_ATTN_CALL(HSA_ATTN_HAVE_FP32_D64_K32, FP32, 64, 32);
}

}  // namespace hsa_attn
