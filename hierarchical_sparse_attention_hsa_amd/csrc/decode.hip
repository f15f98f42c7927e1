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
#include "mfma.hpp"

namespace hsa_attn {

// Tuning knobs of the landmark scan (compile-time; defaults are the measured
// best on MI355X): loads in flight per lane, register double-buffering,
// largest landmark range per workgroup, non-temporal loads.
#ifndef HSA_ATTN_SCAN_UNROLL
#define HSA_ATTN_SCAN_UNROLL 16
#endif
#ifndef HSA_ATTN_SCAN_PREFETCH
#define HSA_ATTN_SCAN_PREFETCH 0
#endif
#ifndef HSA_ATTN_SCAN_MAX_ROWS
#define HSA_ATTN_SCAN_MAX_ROWS 1024
#endif
#ifndef HSA_ATTN_SCAN_NT
#define HSA_ATTN_SCAN_NT 1
#endif
constexpr int kScanThreads = 256;
constexpr int kScanUnroll = HSA_ATTN_SCAN_UNROLL;

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

// ---------------------------------------------------------------- split top-k
// Exact top-m (m = min(k, n)) of n scores held in LDS, under the order
// (score desc, index asc), by one wave, without per-candidate insertions:
//   1. the score range [lo, hi] (wave min / max);
//   2. a 256-bin histogram of t = (s - lo) * 256 / (hi - lo) (the bin is
//      monotone in s) gives the bin B1 holding the m-th best; a second
//      256-bin histogram of the fraction of t inside B1 narrows it to B2;
//   3. every candidate in a higher (bin, sub-bin) plus every candidate of
//      (B1, B2) is gathered (at most kGather; otherwise the caller falls
//      back to list insertion) and
//   4. a bitonic sort of the gathered (score, index) pairs across the wave
//      leaves the e-th best in lane e.
// Returns false when the gathered set does not fit.
constexpr int kGather = 128;

__device__ __forceinline__ float wave_min_f(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// sum over the lanes above this one (exclusive suffix sum)
__device__ __forceinline__ int suffix_excl(int v, int lane) {
  int incl = v;
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_down(incl, off);
    if (lane + off < kWave) incl += o;
  }
  return incl - v;
}

// Find the bin of the m-th largest element from a 256-bin histogram: returns
// (bin, count strictly above it).  Lane l owns bins 4l .. 4l+3.
__device__ __forceinline__ void hist_select(const int* hist, int m, int lane, int& bin, int& above) {
  const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
  const int sup = suffix_excl(c0 + c1 + c2 + c3, lane);  // elements in higher lanes' bins
  int found = -1, abv = 0;
  int cum = sup;
  const int cs[4] = {c3, c2, c1, c0};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (found < 0 && cum + cs[q] >= m && cum < m) {
      found = 4 * lane + 3 - q;
      abv = cum;
    }
    cum += cs[q];
  }
  const uint64_t who = __ballot(found >= 0);
  const int src = who ? __builtin_ctzll(who) : 0;
  bin = __builtin_amdgcn_readlane(found, src);
  above = __builtin_amdgcn_readlane(abv, src);
}

// Bitonic sort of buf[0 .. cnt) (cnt <= kGather; the rest is padded with
// the worst entry) by (score desc, index asc) across one wave: element
// x = 64 t + lane sits in register t of lane `lane`; on return lane e holds
// the e-th best.
__device__ __forceinline__ void sort_gathered(const float2* buf, int cnt, float& out_s, int& out_i) {
  const int lane = __lane_id();
  float s0, s1;
  int i0, i1;
  {
    const float2 e0 = lane < cnt ? buf[lane] : make_float2(-__builtin_inff(), __int_as_float(INT_MAX));
    const float2 e1 = lane + kWave < cnt ? buf[lane + kWave] : make_float2(-__builtin_inff(), __int_as_float(INT_MAX));
    s0 = e0.x;
    i0 = __float_as_int(e0.y);
    s1 = e1.x;
    i1 = __float_as_int(e1.y);
  }
  auto step = [&](float& sv, int& iv, int x, int k2, int jj) {
    const float os = __shfl_xor(sv, jj);
    const int oi = __shfl_xor(iv, jj);
    const bool lower = (x & jj) == 0;
    const bool asc = (x & k2) == 0;  // this run sorts best first
    const bool keep_better = lower == asc;
    const bool mine_better = better(sv, iv, os, oi);
    if (keep_better != mine_better) {
      sv = os;
      iv = oi;
    }
  };
  for (int k2 = 2; k2 <= 2 * kWave; k2 <<= 1) {
    for (int jj = k2 >> 1; jj > 0; jj >>= 1) {
      if (jj == kWave) {  // partner is the other register of this lane (k2 = 128: best first)
        if (!better(s0, i0, s1, i1)) {
          const float ts = s0;
          const int ti = i0;
          s0 = s1;
          i0 = i1;
          s1 = ts;
          i1 = ti;
        }
      } else {
        step(s0, i0, lane, k2, jj);
        step(s1, i1, lane + kWave, k2, jj);
      }
    }
  }
  out_s = s0;
  out_i = i0;
}

// Entries equal to -inf are padding (an empty slot of a split list): they
// are neither binned nor gathered, so only the nf finite entries compete
// and lanes nf.. of the result hold padding.
__device__ __forceinline__ bool split_topk(const float* sc, int n, int idx0, int k, int* hist, float2* buf,
                                           float& out_s, int& out_i) {
  const int lane = __lane_id();
  float lo = __builtin_inff(), hi = -__builtin_inff();
  int nf = 0;
  for (int r = lane; r < n; r += kWave) {
    const float x = sc[r];
    if (x > -__builtin_inff()) {
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
      ++nf;
    }
  }
  lo = wave_min_f(lo);
  hi = wave_max_f(hi);
  for (int off = 32; off >= 1; off >>= 1) nf += __shfl_xor(nf, off);
  const int m = min(k, nf);
  // finite lo and hi whenever nf > 0, so t is finite and >= 0 for every
  // finite entry
  float inv = hi > lo ? 256.0f / (hi - lo) : 0.0f;
  if (!(inv < 1e30f)) inv = 0.0f;  // a range too narrow to bin: one bin (then gather or fall back)
  auto tval = [&](float x) { return (x - lo) * inv; };
  auto bin_of = [&](float t) { return min(255, (int)t); };
  int B1 = 0, B2 = 0;
  if (nf > kGather) {
    // pass 1
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
    for (int r = lane; r < n; r += kWave) {
      const float x = sc[r];
      if (x > -__builtin_inff()) atomicAdd(&hist[bin_of(tval(x))], 1);
    }
    int above1;
    hist_select(hist, m, lane, B1, above1);
    // pass 2: inside B1
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
    for (int r = lane; r < n; r += kWave) {
      const float x = sc[r];
      if (!(x > -__builtin_inff())) continue;
      const float t = tval(x);
      if (bin_of(t) == B1) atomicAdd(&hist[min(255, (int)((t - (float)B1) * 256.0f))], 1);
    }
    int above2;
    hist_select(hist, m - above1, lane, B2, above2);
  } else {
    B1 = 0;
    B2 = 0;  // gather every finite entry
  }
  // gather the finite entries with (bin, sub-bin) >= (B1, B2), in index order
  int cnt = 0;
  for (int r0 = 0; r0 < n; r0 += kWave) {
    const int r = r0 + lane;
    bool take = false;
    float x = 0.0f;
    if (r < n) {
      x = sc[r];
      if (x > -__builtin_inff()) {
        const float t = tval(x);
        const int b1 = bin_of(t);
        take = b1 > B1 || (b1 == B1 && min(255, (int)((t - (float)B1) * 256.0f)) >= B2);
      }
    }
    const uint64_t mk = __ballot(take);
    const int pos = cnt + __popcll(mk & ((1ull << lane) - 1ull));
    if (take && pos < kGather) buf[pos] = make_float2(x, __int_as_float(idx0 + r));
    cnt += __popcll(mk);
  }
  if (cnt > kGather) return false;
  sort_gathered(buf, cnt, out_s, out_i);
  return true;
}

// ---------------------------------------------------------------- 1. scan
template <typename T, int D, int G>
__global__ __launch_bounds__(kScanThreads) void decode_scan_kernel(const typename T::storage* __restrict__ q,
                                                                   const typename T::storage* __restrict__ lm,
                                                                   float2* __restrict__ cand, int Hkv, int64_t Nc,
                                                                   int rows_per_split, int splits, int k,
                                                                   float scale, const int64_t* __restrict__ lens,
                                                                   int64_t T_len) {
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
  // complete chunks of this sequence's cache (varlen batches: lens[b] tokens)
  const int64_t ncb = lens ? min(max(lens[b], (int64_t)0), T_len) / 64 : Nc;
  const int n = (int)min((int64_t)rows_per_split, ncb - r_begin);
  if (n <= 0) {  // a split past the end of this cache: empty candidate lists
    for (int h = wave; h < G; h += WAVES)
      if (lane < k)
        cand[((((int64_t)b * Hkv + g) * splits + sp) * G + h) * k + lane] =
            make_float2(-__builtin_inff(), __int_as_float(INT_MAX));
    return;
  }
  const int col = (lane % LPR) * EPL;

  u32x4 qv[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const u32x4*>(q + ((int64_t)b * Hkv * G + (int64_t)g * G + h) * D + col);

  const typename T::storage* base = lm + (((int64_t)b * Hkv + g) * Nc + r_begin) * D + col;
  // with HSA_ATTN_SCAN_PREFETCH the next iteration's rows are in flight while
  // the current ones are scored (register double buffer)
  u32x4 nxt[kScanUnroll];
  auto fetch = [&](int it) {
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int r = it + (wave * kScanUnroll + u) * RPI + lane / LPR;
      const u32x4* src = reinterpret_cast<const u32x4*>(base + (int64_t)r * D);
      if (r < n) nxt[u] = HSA_ATTN_SCAN_NT ? __builtin_nontemporal_load(src) : *src;
      else nxt[u] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (HSA_ATTN_SCAN_PREFETCH) fetch(0);
  for (int it = 0; it < n; it += ROWS_PER_ITER) {
    if (!HSA_ATTN_SCAN_PREFETCH) fetch(it);
    u32x4 v[kScanUnroll];
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) v[u] = nxt[u];
    if (HSA_ATTN_SCAN_PREFETCH && it + ROWS_PER_ITER < n) fetch(it + ROWS_PER_ITER);
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

  int* hist = reinterpret_cast<int*>(sc + G * rows_per_split) + wave * 256;
  float2* gbuf = reinterpret_cast<float2*>(sc + G * rows_per_split + WAVES * 256) + wave * kGather;
  for (int h = wave; h < G; h += WAVES) {
    float os;
    int oi;
    if (!split_topk(sc + h * rows_per_split, n, (int)r_begin, k, hist, gbuf, os, oi)) {
      // many equal scores around the k-th: ordered insertion
      WaveTopK list;
      list.init();
      for (int i0 = 0; i0 < n; i0 += kWave) {
        const int r = i0 + lane;
        const bool valid = r < n;
        const float s = valid ? sc[h * rows_per_split + r] : -__builtin_inff();
        offer_wave(list, k, s, (int)(r_begin + r), valid);
      }
      os = list.s;
      oi = list.i;
    }
    if (lane < k) {
      float2 c;
      c.x = os;
      c.y = __int_as_float(oi);
      cand[((((int64_t)b * Hkv + g) * splits + sp) * G + h) * k + lane] = c;
    }
  }
}

// ---------------------------------------------------------------- 2. merge
// One workgroup per (b, g), one wave per query head of the group: merge the
// split candidates of the head into its global top-k (total order: score
// desc, index asc), then list the group's distinct selected chunks once,
// each with the slot it holds in every head's selection (0xff = not
// selected).  The list order is deterministic (first occurrence in head-major
// slot order).
// Adaptive budget (k_base > 0, k = 2 * k_base; value-of-information router
// abstract, k-th versus (k+1)-th gap): a head whose k_base-th best score
// beats its (k_base+1)-th by less than gap_tau keeps all k entries, any
// other head only its first k_base (the rest become padding before the
// group's chunk list is built).
template <int G>
__global__ __launch_bounds__(kWave* G) void decode_merge_kernel(const float2* __restrict__ cand,
                                                                int32_t* __restrict__ sel_idx,
                                                                float* __restrict__ sel_score,
                                                                int4* __restrict__ ulist, int* __restrict__ ucount,
                                                                int Hkv, int splits, int k, int k_base,
                                                                float gap_tau) {
  constexpr int kMaxVals = 1024;  // threshold sample held in LDS per head
  __shared__ int ls[G * 64];
  __shared__ int wave_cnt[G];
  __shared__ float tvals[G][kMaxVals];
  __shared__ int hist[G][256];
  __shared__ float2 gbuf[G][kGather];
  __shared__ int gcnt[G];
  const int g = blockIdx.x, b = blockIdx.y;
  const int lane = __lane_id(), hh = threadIdx.x / kWave;
  const int64_t bh = (int64_t)b * Hkv * G + (int64_t)g * G + hh;
  const float2* cb = cand + (((int64_t)b * Hkv + g) * splits * G + hh) * k;
  WaveTopK list;
  list.init();

  // Fast path: the k-th best of the first r entries of every split's sorted
  // list (at least 2k values) is a lower bound tau of the head's k-th best
  // score; every entry at or above tau is gathered and sorted: the first r
  // of each list by one parallel read, deeper entries only from the lists
  // whose r-th entry reached tau (walked until they drop below it).  Too
  // many gathered entries fall back to merging every candidate.
  bool done = false;
  {
    const int r = min(k, max(1, (2 * k + splits - 1) / splits));
    const int nv = splits * r;
    if (nv > 0 && nv <= kMaxVals) {
      for (int v = lane; v < nv; v += kWave) {
        const float2 c = cb[(int64_t)(v / r) * G * k + v % r];
        tvals[hh][v] = __float_as_int(c.y) != INT_MAX ? c.x : -__builtin_inff();
      }
      if (lane == 0) gcnt[hh] = 0;
      float ts;
      int ti;
      if (split_topk(tvals[hh], nv, 0, k, hist[hh], gbuf[hh], ts, ti)) {
        const float tau = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ts), min(k, nv) - 1));
        if (tau > -__builtin_inff()) {
          // an entry at or above the finite tau is a valid one
          for (int v = lane; v < nv; v += kWave) {
            if (tvals[hh][v] >= tau) {
              const float2 c = cb[(int64_t)(v / r) * G * k + v % r];
              const int pos = atomicAdd(&gcnt[hh], 1);
              if (pos < kGather) gbuf[hh][pos] = c;
            }
          }
          for (int sp = lane; sp < splits; sp += kWave) {
            if (!(tvals[hh][sp * r + r - 1] >= tau)) continue;
            for (int e = r; e < k; ++e) {
              const float2 c = cb[(int64_t)sp * G * k + e];
              if (__float_as_int(c.y) == INT_MAX || c.x < tau) break;
              const int pos = atomicAdd(&gcnt[hh], 1);
              if (pos < kGather) gbuf[hh][pos] = c;
            }
          }
          const int cnt = gcnt[hh];
          if (cnt <= kGather) {
            sort_gathered(gbuf[hh], cnt, list.s, list.i);
            done = true;
          }
        }
      }
    }
  }
  const int total = done ? 0 : splits * k;
  // rank-major order: every split's best first, so the list fills with
  // strong candidates early and later ranks rarely get in; the loads of
  // kMergeBatch rounds are issued together (the loop is latency-bound)
  constexpr int kMergeBatch = 8;
  for (int i0 = 0; i0 < total; i0 += kWave * kMergeBatch) {
    float2 c[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int j = i0 + u * kWave + lane;
      c[u] = make_float2(-__builtin_inff(), __int_as_float(INT_MAX));
      if (j < total) {
        const int e = j / splits, sp = j % splits;
        c[u] = cb[(int64_t)sp * G * k + e];
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int ci = __float_as_int(c[u].y);
      offer_wave(list, k, c[u].x, ci, ci != INT_MAX);
    }
  }
  if (k_base > 0) {
    const float s_k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(list.s), k_base - 1));
    const float s_k1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(list.s), k_base));
    const int i_k1 = __builtin_amdgcn_readlane(list.i, k_base);
    // an invalid (k_base+1)-th entry means at most k_base candidates: no cut
    const bool doubled = i_k1 != INT_MAX && s_k - s_k1 < gap_tau;
    if (!doubled && lane >= k_base) {
      list.s = -__builtin_inff();
      list.i = INT_MAX;
    }
  }
  const bool ok = list.i != INT_MAX;
  if (lane < k) {
    sel_idx[bh * k + lane] = ok ? list.i : -1;
    sel_score[bh * k + lane] = ok ? list.s : -__builtin_inff();
    ls[hh * k + lane] = ok ? list.i : -1;
  }
  // the entries padded to a multiple of 8 with a value no entry holds
  const int nent = G * k, nent8 = (nent + 7) & ~7;
  if ((int)threadIdx.x < nent8 - nent) ls[nent + threadIdx.x] = -2;
  __syncthreads();
  // entry e = hh * k + lane owns its chunk when no earlier entry names it;
  // every entry of the group is compared through uniform LDS reads, eight
  // issued together
  const int e = hh * k + lane;
  const int c = lane < k ? ls[e] : -1;
  bool owner = c >= 0;
  uint32_t slots0 = 0xffffffffu, slots1 = 0xffffffffu;  // heads 0..3, 4..7
  int h2 = 0, s2 = 0;  // head and slot of entry f
  for (int f0 = 0; f0 < nent8; f0 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ls[f0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (v[u] == c) {
        if (f0 + u < e) owner = false;
        const int sh = 8 * (h2 & 3);
        const uint32_t put = (uint32_t)s2 << sh, keep = ~(0xffu << sh);
        if (h2 < 4) slots0 = (slots0 & keep) | put;
        else slots1 = (slots1 & keep) | put;
      }
      if (++s2 == k) {
        s2 = 0;
        ++h2;
      }
    }
  }
  const uint32_t slots[2] = {slots0, slots1};
  const uint64_t om = __ballot(owner);
  if (lane == 0) wave_cnt[hh] = __popcll(om);
  __syncthreads();
  int base = 0;
  for (int w = 0; w < hh; ++w) base += wave_cnt[w];
  if (owner) {
    const int pos = base + __popcll(om & ((1ull << lane) - 1));
    ulist[((int64_t)b * Hkv + g) * (G * k) + pos] = make_int4(c, (int)slots[0], (int)slots[1], 0);
  }
  if (threadIdx.x == 0) {
    int n = 0;
    for (int w = 0; w < G; ++w) n += wave_cnt[w];
    ucount[(int64_t)b * Hkv + g] = n;
  }
}

// ---------------------------------------------------------------- 3. chunk attention
// The waves are independent, so a workgroup holds one: 65K small
// workgroups over the group entries finish more evenly than 16K of four
// (measured 5% faster at 1M).
constexpr int kAttnWaves = 1;
// One wave per distinct selected chunk of a (b, g) group; waves are
// independent (wave-private LDS, no barriers).  Logits of all G heads on
// MFMA: S^T[token][head] = K_c . q_head (A = the chunk's keys, staged in
// LDS by whole-line direct loads, B = the group's queries padded to 32
// columns); each head's softmax stays in the two lanes
// that hold its column.  P.V on the VALU: lane l owns value rows
// l/LPR + RPI*i and a 16-byte column slice; the probabilities go through a
// wave-private LDS table [token][head]; a cross-lane sum finishes each
// output column.
template <typename T, int D, int G>
__global__ __launch_bounds__(kAttnWaves * kWave) void decode_attn_kernel(const typename T::storage* __restrict__ q,
                                                          const typename T::storage* __restrict__ kc,
                                                          const typename T::storage* __restrict__ vc,
                                                          const int4* __restrict__ ulist,
                                                          const int* __restrict__ ucount,
                                                          float* __restrict__ partial, int Hkv, int64_t T_len,
                                                          int k, float scale, uint32_t* __restrict__ dbg) {
  using st = typename T::storage;
  constexpr int S = 64;
  constexpr int KCH = D / 16;
  constexpr int EPS = 16 / T::kBytes;          // elements per 16-byte slice
  constexpr int LPR = D / EPS;                 // lanes per V row
  constexpr int RPI = kWave / LPR;             // V rows per load instruction
  constexpr int VL = S / RPI;                  // V loads per lane (whole tile)
  // more than 8 V loads per lane go in two passes (fewer live registers: 3
  // waves per SIMD instead of 2 for bf16 at D = 128)
  constexpr int VPASS = VL > 8 ? 2 : 1;
  constexpr int VLP = VL / VPASS;
  __shared__ __align__(16) float pbuf[kAttnWaves][S][G];  // per wave: probability of (token, head)
  const int b = blockIdx.z, g = blockIdx.y;
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int e = blockIdx.x * kAttnWaves + wave;
  const int64_t grp = (int64_t)b * Hkv + g;
  const int uc = ucount[grp];
  if (e >= uc) return;
  if (!dbg_ok(dbg, uc <= G * k, HSA_ATTN_DEBUG_DECODE_ENTRIES)) return;
  const int4 ent = ulist[grp * (G * k) + e];
  const int c = ent.x;
  if (!dbg_ok(dbg, c >= 0 && (int64_t)c * S + S <= T_len, HSA_ATTN_DEBUG_DECODE_CHUNK)) return;
  uint32_t slots[2] = {(uint32_t)ent.y, (uint32_t)ent.z};
  if constexpr (HSA_ATTN_DEBUG) {
    // a slot number beyond k (other than 0xff, "not selected") would index
    // past the head's partial outputs: flagged and treated as not selected
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint32_t sl = (slots[hh / 4] >> (8 * (hh % 4))) & 0xffu;
      if (!dbg_ok(dbg, sl == 0xffu || (int)sl < k, HSA_ATTN_DEBUG_DECODE_SLOT))
        slots[hh / 4] |= 0xffu << (8 * (hh % 4));
    }
  }
  const int half = lane >> 5;
  const st* ktile = kc + (grp * T_len + (int64_t)c * S) * D;
  const st* vtile = vc + (grp * T_len + (int64_t)c * S) * D;

  // queries of the group as the B operand: column j = head (lane % 32 < G)
  Frag<T> qf[KCH];
  {
    const int j = lane & 31;
    const bool okq = j < G;
    const st* qp = q + (grp * G + (okq ? j : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KCH; ++s) load_frag_global(qf[s], qp + 16 * s, okq);
  }
  // every load of the tile is issued before any use: the key tile into LDS
  // by direct global->LDS loads (whole 1 KiB pieces; row r's 16-byte slots
  // XOR-swizzled by r & 7 on the global side; read back as the A operands
  // of both 32-token blocks), and the first pass of V slices (lane owns rows
  // RPI*i + lane/LPR, elements (lane%LPR)*EPS..)
  constexpr int ROWB = D * T::kBytes, NSL = ROWB / 16, KTB = S * ROWB, NKI = KTB / (kWave * 16);
  __shared__ __align__(16) char ktl[kAttnWaves][KTB];
  {
    const char* kb = reinterpret_cast<const char*>(ktile);
#pragma unroll
    for (int ii = 0; ii < NKI; ++ii) {
      const int L = ii * kWave + lane, t = L / NSL, sp = L % NSL;
      __builtin_amdgcn_global_load_lds(kb + t * ROWB + ((sp ^ (t & 7)) * 16),
                                       (__attribute__((address_space(3))) void*)(ktl[wave] + ii * kWave * 16), 16,
                                       0, 0);
    }
  }
  u32x4 vr[VLP];
  const int vcol = (lane % LPR) * EPS;
  const int vrow0 = lane / LPR;
#pragma unroll
  for (int i = 0; i < VLP; ++i)
    vr[i] = *reinterpret_cast<const u32x4*>(vtile + (int64_t)(RPI * i + vrow0) * D + vcol);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  // the queries and the key tile are in (the value loads may still fly)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VLP) : "memory");
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const char* row = ktl[wave] + (32 * tb + (lane & 31)) * ROWB;
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      Frag<T> a;
      if constexpr (T::kBytes == 2) {
        a.load16(row + (((2 * s + half) ^ (lane & 7)) * 16));
      } else {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(row + (((4 * s + 2 * half) ^ (lane & 7)) * 16));
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(row + (((4 * s + 2 * half + 1) ^ (lane & 7)) * 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a.v[e] = x0[e];
          a.v[4 + e] = x1[e];
        }
      }
      mfma(sacc[tb], a, qf[s]);
    }
  }
  // With two value passes, the second pass's slices go into the key tile's
  // LDS (direct global->LDS loads, lane l's 16 bytes of load i at i * 1 KiB
  // + 16 l) as soon as the key fragments are read, so they fly during the
  // softmax and the first pass instead of after it.
  if constexpr (VPASS == 2) {
    static_assert(VLP * kWave * 16 <= KTB, "the second value pass fits the key tile's LDS");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the key fragments are in registers
#pragma unroll
    for (int i = 0; i < VLP; ++i)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const char*>(vtile + (int64_t)(RPI * (VLP + i) + vrow0) * D + vcol),
          (__attribute__((address_space(3))) void*)(ktl[wave] + i * kWave * 16), 16, 0, 0);
  }

  // softmax per head column: lane l (l%32 = head) holds tokens
  // 32*tb + tile_row(r, half); its partner l^32 holds the rest
  float mx = -__builtin_inff();
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[tb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float cexp = scale * 1.4426950408889634f;
  float den = 0.0f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[tb][r] = exp2f((sacc[tb][r] - mx) * cexp);
      den += sacc[tb][r];
    }
  den += __shfl_xor(den, 32);
  const float inv = 1.0f / den;
  if ((lane & 31) < G) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pbuf[wave][32 * tb + tile_row(r, half)][lane & 31] = sacc[tb][r] * inv;
  }
  // the table is private to this wave: its LDS accesses complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  bool sel_h[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) sel_h[hh] = ((slots[hh / 4] >> (8 * (hh % 4))) & 0xffu) != 0xffu;
  float o[G][EPS];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int x = 0; x < EPS; ++x) o[hh][x] = 0.0f;
#pragma unroll
  for (int ps = 0; ps < VPASS; ++ps) {
    if (ps > 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the second pass's slices are in LDS
#pragma unroll
      for (int i = 0; i < VLP; ++i)
        vr[i] = *reinterpret_cast<const u32x4*>(ktl[wave] + i * kWave * 16 + 16 * lane);
    }
#pragma unroll
    for (int i = 0; i < VLP; ++i) {
      const int t = RPI * (ps * VLP + i) + vrow0;  // the value row this lane holds in load i
      float pr[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) pr[hh] = pbuf[wave][t][hh];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        if (!sel_h[hh]) continue;  // this head did not select the chunk (wave-uniform)
        if constexpr (T::kBytes == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            o[hh][2 * w] = fmaf(pr[hh], bf16_lo(vr[i][w]), o[hh][2 * w]);
            o[hh][2 * w + 1] = fmaf(pr[hh], bf16_hi(vr[i][w]), o[hh][2 * w + 1]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) o[hh][w] = fmaf(pr[hh], __uint_as_float(vr[i][w]), o[hh][w]);
        }
      }
    }
  }
  // sum over the RPI row groups (lanes that share lane % LPR), then write
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint32_t sl = (slots[hh / 4] >> (8 * (hh % 4))) & 0xffu;
    if (sl == 0xffu) continue;
#pragma unroll
    for (int x = 0; x < EPS; ++x)
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) o[hh][x] += __shfl_xor(o[hh][x], off);
    if (lane < LPR) {
      float* dst = partial + ((grp * G + hh) * k + sl) * D + vcol;
#pragma unroll
      for (int x = 0; x < EPS; x += 4)
        *reinterpret_cast<f32x4*>(dst + x) = f32x4{o[hh][x], o[hh][x + 1], o[hh][x + 2], o[hh][x + 3]};
    }
  }
}

// ---------------------------------------------------------------- 4. fusion
// The kept slots come first (padding after them), so the loop runs over all
// k slots without an early exit: the loads are independent and overlap; a
// padding slot's partial (never written) is loaded and discarded.
__global__ void decode_fuse_kernel(const float* __restrict__ partial, const int32_t* __restrict__ sel_idx,
                                   const float* __restrict__ sel_score, float* __restrict__ out, int k, int D) {
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const float mx = sel_score[bh * k];
  float den = 0.0f, num = 0.0f;
  constexpr int U = 8;  // slots whose loads are issued together
  for (int s0 = 0; s0 < k; s0 += U) {
    bool kept[U];
    float w[U], x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      kept[u] = s < k && sel_idx[bh * k + s] >= 0;
      w[u] = kept[u] ? __expf(sel_score[bh * k + s] - mx) : 0.0f;
      x[u] = s < k ? partial[(bh * k + s) * D + d] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      den += w[u];
      num = kept[u] ? fmaf(w[u], x[u], num) : num;
    }
  }
  out[bh * D + d] = den > 0.0f ? num / den : 0.0f;
}

// ---------------------------------------------------------------- host side
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

DecodePlan plan_decode(const Geometry& g, bool own_sel) {
  DecodePlan p{};
  const int64_t bh = (int64_t)g.B * g.Hkv;
  // aim for ~8K scan workgroups in total (many rounds over the 256 CUs keep the
  // tail short), 256..1024 landmark rows each
  int64_t rows = (g.Nc * bh + 8191) / 8192;
  rows = (rows + 63) / 64 * 64;
  rows = rows < 256 ? 256 : (rows > HSA_ATTN_SCAN_MAX_ROWS ? HSA_ATTN_SCAN_MAX_ROWS : rows);
  p.rows_per_split = (int)rows;
  // caches without a complete chunk still get one split: its scan writes
  // empty candidate lists, so the merge always reads at least one list
  p.splits = g.Nc > 0 ? (int)((g.Nc + rows - 1) / rows) : 1;
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
  p.off_ulist = off;
  off = align_up(off + (size_t)bh * g.G * g.k * sizeof(int4), 256);
  p.off_ucount = off;
  off = align_up(off + (size_t)bh * sizeof(int), 256);
  p.bytes = off;
  return p;
}

template <typename T, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  const Geometry& g = a.g;
  char* ws = static_cast<char*>(a.ws);
  float2* cand = reinterpret_cast<float2*>(ws + p.off_cand);
  float* partial = reinterpret_cast<float*>(ws + p.off_partial);
  int4* ulist = reinterpret_cast<int4*>(ws + p.off_ulist);
  int* ucount = reinterpret_cast<int*>(ws + p.off_ucount);
  const float scale = 1.0f / sqrtf((float)D);
  using stg = typename T::storage;
  if (p.splits > 0) {
    // scores, then per wave a 256-bin histogram and the gather buffer
    const size_t lds = (size_t)G * p.rows_per_split * sizeof(float) +
                       (size_t)(kScanThreads / kWave) * (256 * sizeof(int) + kGather * sizeof(float2));
    launch_kernel((decode_scan_kernel<T, D, G>), dim3(p.splits, g.Hkv, g.B), dim3(kScanThreads), lds, st,
                  static_cast<const stg*>(a.q), static_cast<const stg*>(a.lm), cand, g.Hkv, g.Nc,
                  p.rows_per_split, p.splits, g.k, scale, a.lens, g.T);
  }
  launch_kernel((decode_merge_kernel<G>), dim3(g.Hkv, g.B), dim3(kWave * G), 0, st, cand, a.sel_idx,
                a.sel_score, ulist, ucount, g.Hkv, p.splits, g.k, a.k_base, a.gap_tau);
  if (g.Nc > 0) {  // no complete chunk: nothing selected, nothing to attend
    launch_kernel((decode_attn_kernel<T, D, G>), dim3((G * g.k + kAttnWaves - 1) / kAttnWaves, g.Hkv, g.B),
                  dim3(kAttnWaves * kWave), 0, st,
                  static_cast<const stg*>(a.q), static_cast<const stg*>(a.k), static_cast<const stg*>(a.v),
                  ulist, ucount, partial, g.Hkv, g.T, g.k, scale, a.dbg);
  }
  launch_kernel(decode_fuse_kernel, dim3(g.B * g.Hq), dim3(D), 0, st, partial, a.sel_idx, a.sel_score, a.out,
                g.k, D);
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
