// HSA prefill: causal HSA over a whole sequence (skill card "Every Token
// Counts 16m Context", sections "Core Technique" and "Implementation").
//
// Two kernels on one stream:
//
// prefill_select  one workgroup per (b, g, query chunk j), one wave per query
//   head of the group, 64 query rows per wave.  Landmark tiles of 32 rows are
//   staged in LDS (shared by the G waves) and contracted with the wave's
//   queries on MFMA (bf16 in, fp32 accumulate): the causal-block GEMM
//   Q . L^T restricted to the j earlier chunks.  Tiles run from the newest
//   chunk to the oldest.  After every tile the two lane halves swap
//   accumulator halves (v_permlane32_swap) so that each lane holds the 32
//   scores of one query row; the lane keeps that row's top-k in registers
//   (descending order, so a new candidate always has the lowest index so far
//   and wins ties, which realises "ties toward the lower chunk index").  The
//   score matrix never reaches memory.
//
// prefill_attn  one workgroup per (b, g, query chunk j, 32-token half), one
//   wave per query head.  The union of the rows' selected chunks is walked in
//   ascending order; each chunk's K and V tiles are staged in LDS once for all
//   the workgroup's rows.  S^T = K_c Q^T on MFMA, an fp32 softmax per row,
//   and O^T += V_c^T P'^T on MFMA, where P' is the in-chunk probability
//   already multiplied by the row's fusion weight (softmax of its kept
//   retrieval scores); rows that did not select the chunk have weight 0.
//   P' is fed to the bf16 MFMA as a hi + lo pair so it keeps ~16 bits.
#pragma once

#include <climits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace hsa_attn {

constexpr int kChunk = 64;

template <typename T>
__device__ __forceinline__ void load_frag_lds(Frag<T>& f, const char* row, int slot_xor, int kch, int half);

// bf16: 8 elements of one half k-chunk = one 16-byte slot (2*kch + half)
template <>
__device__ __forceinline__ void load_frag_lds<BF16>(Frag<BF16>& f, const char* row, int slot_xor, int kch,
                                                    int half) {
  const int slot = (2 * kch + half) ^ slot_xor;
  f.load16(row + slot * 16);
}
// fp32: 8 elements = two 16-byte slots (4*kch + 2*half, +1)
template <>
__device__ __forceinline__ void load_frag_lds<FP32>(Frag<FP32>& f, const char* row, int slot_xor, int kch,
                                                    int half) {
  const int s0 = (4 * kch + 2 * half) ^ slot_xor;
  const int s1 = (4 * kch + 2 * half + 1) ^ slot_xor;
  const f32x4 a = *reinterpret_cast<const f32x4*>(row + s0 * 16);
  const f32x4 b = *reinterpret_cast<const f32x4*>(row + s1 * 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}

// Insert x (index xi) into a descending register list; the new element wins
// ties (callers offer candidates in descending index order).
template <int K>
__device__ __forceinline__ void list_insert(float (&s)[K], int (&id)[K], float x, int xi) {
  bool c[K];
#pragma unroll
  for (int p = 0; p < K; ++p) c[p] = x >= s[p];
#pragma unroll
  for (int p = K - 1; p >= 1; --p) {
    id[p] = c[p - 1] ? id[p - 1] : (c[p] ? xi : id[p]);
    s[p] = __builtin_amdgcn_fmed3f(s[p - 1], x, s[p]);
  }
  id[0] = c[0] ? xi : id[0];
  s[0] = c[0] ? x : s[0];
}

// Insert x into a descending list of scores (ties are equal values, so no
// index is needed): one v_med3 per position.
template <int K>
__device__ __forceinline__ void score_insert(float (&s)[K], float x) {
#pragma unroll
  for (int p = K - 1; p >= 1; --p) s[p] = __builtin_amdgcn_fmed3f(s[p - 1], x, s[p]);
  s[0] = fmaxf(s[0], x);
}

// ---------------------------------------------------------------- select
//
// One workgroup per (b, g, query chunk j) and group of up to four query
// heads; one wave per head, 64 query rows per wave (lane = row).  Each wave
// streams the landmark tiles (32 chunks) of its KV head from L2 and
// contracts them with its queries on MFMA; the scores stay in registers.
//
// Pass 1 runs the tiles from the newest chunk down and keeps, per row, only
// the multiset of the k best scores (one v_med3 per list position per
// admitted candidate), which yields the row's k-th best score tau and how
// many of the k best are strictly above it.  Pass 2 recomputes the same
// tiles (bit-identical: same operands, same instruction sequence) in
// ascending chunk order and collects every candidate above tau plus the
// lowest-index candidates equal to tau until k are kept: exactly the first
// k in the order (score desc, index asc).  Tiles whose maximum cannot reach
// a row's threshold are skipped in both passes.
template <typename T, int D, int G, int KSEL>
__global__ __launch_bounds__(kWave*(G < 4 ? G : 4)) void prefill_select_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ lm,
    int32_t* __restrict__ sel_idx, float* __restrict__ sel_score, int B, int Hkv, int64_t T_len, int64_t Nc, int nqc,
    int k, float scale) {
  using st = typename T::storage;
  constexpr int HPW = G < 4 ? G : 4;  // query heads (waves) per workgroup
  constexpr int HS = G / HPW;         // workgroups per (b, g, query chunk)
  constexpr int KCH = D / 16;
  constexpr int MAXT = 2048;          // tiles with a recorded pass-1 skip
  __shared__ float2 cbuf[HPW][KSEL][kWave];
  __shared__ uint8_t tskip[HPW][MAXT];

  const int bid = blockIdx.x;
  const int g = bid % Hkv;  // consecutive workgroups on different XCDs share nothing
  int rest = bid / Hkv;
  const int hs = rest % HS;
  rest /= HS;
  const int b = rest % B;
  const int j = nqc - 1 - rest / B;  // heaviest query chunks first
  const int tid = threadIdx.x, lane = tid & 63, hh = tid >> 6, half = lane >> 5;
  const int Hq = Hkv * G, h = g * G + hs * HPW + hh;
  const int64_t n = min((int64_t)j, Nc);

  auto wave_max_i = [&](int v) {
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off));
    return __builtin_amdgcn_readfirstlane(v);
  };

  int cnt = 0;
  if (n > 0) {
    // Contraction index assignment (shared by both operands): in k-step s,
    // lane half h supplies dims 16*s + 8*h .. +8, so the two lanes of a row
    // read adjacent 16-byte pieces of one cache line.  Rows past the end of
    // the sequence or of the candidate range read a valid row instead; their
    // results are never used (query rows) or masked to -inf (landmarks).
    Frag<T> qf[2][KCH];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t tok = min((int64_t)j * kChunk + 32 * nb + (lane & 31), T_len - 1);
      const st* qp = q + (((int64_t)b * Hq + h) * T_len + tok) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < KCH; ++s) load_frag_global(qf[nb][s], qp + 16 * s, true);
    }
    const st* lmg = lm + ((int64_t)b * Hkv + g) * Nc * D + 8 * half;
    const int ntiles = (int)((n + 31) / 32);
    // landmark fragments (A operand) of one tile, double-buffered
    Frag<T> fa[KCH], fb[KCH];
    auto fetch = [&](Frag<T>(&f)[KCH], int ti) {
      const int64_t c = min((int64_t)ti * 32 + (lane & 31), n - 1);
      const st* p = lmg + c * D;
#pragma unroll
      for (int s = 0; s < KCH; ++s) load_frag_global(f[s], p + 16 * s, true);
    };
    // scores of a tile: lane l gets them for query rows (l%32) and
    // 32 + (l%32) at tile rows tile_row(r, l/32)
    auto contract = [&](const Frag<T>(&f)[KCH], f32x16& acc0, f32x16& acc1) {
      acc0 = f32x16{};
      acc1 = f32x16{};
#pragma unroll
      for (int s = 0; s < KCH; ++s) {
        mfma(acc0, f[s], qf[0][s]);
        mfma(acc1, f[s], qf[1][s]);
      }
    };
    // per-row tile maximum: the per-lane maxima of acc0/acc1, swapped like
    // the scores, combine into the maximum over the row's 32 candidates
    auto row_max = [&](const f32x16& acc0, const f32x16& acc1) {
      float m0 = acc0[0], m1 = acc1[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        m0 = fmaxf(m0, acc0[r]);
        m1 = fmaxf(m1, acc1[r]);
      }
      const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
      return fmaxf(__uint_as_float(pm[0]), __uint_as_float(pm[1]));
    };
    // lane l takes query row l: lo[r] -> tile row tile_row(r, 0), hi[r] ->
    // tile_row(r, 1); rows of the top tile past the candidate range get -inf
    auto to_rows = [&](const f32x16& acc0, const f32x16& acc1, int ti, float (&lo)[16], float (&hi)[16]) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[r]), __float_as_uint(acc1[r]), false,
                                                        false);
        lo[r] = __uint_as_float(p[0]);
        hi[r] = __uint_as_float(p[1]);
      }
      const int cbase = ti * 32;
      if ((int64_t)cbase + 32 > n) {
        const int nv = (int)(n - cbase);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (tile_row(r, 0) >= nv) lo[r] = -__builtin_inff();
          if (tile_row(r, 1) >= nv) hi[r] = -__builtin_inff();
        }
      }
    };
    // candidate ii of the tile (chunk 32*ti + ii) in the lo/hi registers
    auto cand = [](const float (&lo)[16], const float (&hi)[16], int ii) {
      const int r = (ii / 8) * 4 + (ii % 4);
      return ((ii / 4) & 1) ? hi[r] : lo[r];
    };

    // ---- pass 1: the multiset of the k best scores.  List positions above
    // k hold +inf, so ls[KSEL-1] is the k-th best once k are seen; until
    // then the -FLT_MAX seeds keep masked (-inf) candidates out.  A tile in
    // which no row reaches its running threshold is marked: the threshold
    // only grows, so pass 2 can skip it too.
    float ls[KSEL];
#pragma unroll
    for (int e = 0; e < KSEL; ++e) ls[e] = (e < KSEL - k) ? __builtin_inff() : -3.402823466e38f;
    auto pass1 = [&](const Frag<T>(&f)[KCH], int ti) {
      f32x16 acc0, acc1;
      contract(f, acc0, acc1);
      const bool top = (int64_t)ti * 32 + 32 > n;
      if (!top && !__ballot(row_max(acc0, acc1) >= ls[KSEL - 1])) {
        if (ti < MAXT && lane == 0) tskip[hh][ti] = 1;
        return;
      }
      if (ti < MAXT && lane == 0) tskip[hh][ti] = 0;
      float lo[16], hi[16];
      to_rows(acc0, acc1, ti, lo, hi);
#pragma unroll
      for (int ii = 31; ii >= 0; --ii) {
        const float x = cand(lo, hi, ii);
        if (x >= ls[KSEL - 1]) score_insert<KSEL>(ls, x);
      }
    };
    fetch(fa, ntiles - 1);
    for (int ti = ntiles - 1; ti >= 0; ti -= 2) {
      if (ti >= 1) fetch(fb, ti - 1);
      pass1(fa, ti);
      if (ti < 1) break;
      if (ti >= 2) fetch(fa, ti - 2);
      pass1(fb, ti - 1);
    }

    // ---- pass 2: collect the k best in ascending chunk order
    const float tau = ls[KSEL - 1];
    int quota = KSEL;  // entries equal to tau that still fit
#pragma unroll
    for (int e = 0; e < KSEL; ++e) quota -= ls[e] > tau;
    auto next_tile = [&](int ti) {
      while (ti < ntiles && ti < MAXT && tskip[hh][ti]) ++ti;
      return ti;
    };
    auto pass2 = [&](const Frag<T>(&f)[KCH], int ti) {
      f32x16 acc0, acc1;
      contract(f, acc0, acc1);
      const bool top = (int64_t)ti * 32 + 32 > n;
      if (!top && !__ballot(row_max(acc0, acc1) >= tau)) return;
      float lo[16], hi[16];
      to_rows(acc0, acc1, ti, lo, hi);
#pragma unroll
      for (int ii = 0; ii < 32; ++ii) {
        const float x = cand(lo, hi, ii);
        if (x >= tau) {
          const bool take = x > tau || quota > 0;
          if (x == tau) --quota;
          if (take && cnt < KSEL) {
            cbuf[hh][cnt][lane] = make_float2(x, __int_as_float(ti * 32 + ii));
            ++cnt;
          }
        }
      }
    };
    int ti = next_tile(0);
    if (ti < ntiles) fetch(fa, ti);
    while (ti < ntiles) {
      const int t1 = next_tile(ti + 1);
      if (t1 < ntiles) fetch(fb, t1);
      pass2(fa, ti);
      if (t1 >= ntiles) break;
      const int t2 = next_tile(t1 + 1);
      if (t2 < ntiles) fetch(fa, t2);
      pass2(fb, t1);
      ti = t2;
    }
  }
  const int64_t t_row = (int64_t)j * kChunk + lane;
  // order the kept set by (score desc, index asc)
  float os[KSEL];
  int oi[KSEL];
#pragma unroll
  for (int e = 0; e < KSEL; ++e) {
    os[e] = -__builtin_inff();
    oi[e] = INT_MAX;
  }
  {
    const int mx = wave_max_i(cnt);
    for (int e = 0; e < mx; ++e) {
      if (e < cnt) {
        const float2 c = cbuf[hh][e][lane];
        list_insert<KSEL>(os, oi, c.x, __float_as_int(c.y));
      }
    }
  }
  if (t_row < T_len) {
    const int64_t base = (((int64_t)b * Hq + h) * T_len + t_row) * k;
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      if (e < k) {
        const bool ok = oi[e] != INT_MAX;
        sel_idx[base + e] = ok ? oi[e] : -1;
        sel_score[base + e] = ok ? os[e] * scale + 0.0f : -__builtin_inff();
      }
    }
  }
}

// ---------------------------------------------------------------- attention
//
// A selected (row, chunk) pair is "local" when the chunk lies in the query's
// aligned window of kLocalWindow chunks and "remote" otherwise.  Local pairs
// are shared by many rows of a query block (measured: most selections fall
// in the query's own window), so prefill_local_kernel walks the union of a
// block's local selections and runs every row of the block through each
// chunk on MFMA (rows that did not select it get weight 0).  Remote pairs
// are scattered, so they are processed chunk-major: they are bucketed by
// (b, g, chunk), prefill_remote_kernel loads each chunk's K/V tile once and
// gathers its selecting rows 32 at a time into full MFMA tiles, and writes
// each pair's normalised in-chunk output; the local kernel then adds the
// weighted remote outputs of its rows.
constexpr int kLocalWindow = 64;

// V^T element position of token t inside the 64-token row of column d, in
// the order the P' fragments present tokens: k-step t/16, lane half
// (t%8)/4, element 4*((t%16)/8) + t%4.
__device__ __forceinline__ int vt_pos(int t) {
  return (t / 16) * 16 + ((t % 8) / 4) * 8 + 4 * ((t % 16) / 8) + (t % 4);
}

// XOR swizzle of the 16-byte slots of V^T column d.  Reads take eight
// consecutive columns at once (d & 7 varies); stash writes take columns
// eight apart (d >> 3 varies): both sets land on distinct slots.
__device__ __forceinline__ int vt_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// Stages one chunk's K tile (row-major, 16-byte slots XOR-swizzled by row)
// and V^T tile (column-major with the token order of vt_pos, slots swizzled
// by vt_swz) into LDS.  NTH threads cooperate; a unit of work is one
// 16-byte column slot of four consecutive tokens, so each thread writes the
// four tokens of a V^T column as one contiguous 8-byte (bf16) or 16-byte
// (fp32) piece.
template <typename T, int D, int NTH>
struct KVStage {
  using st = typename T::storage;
  static constexpr int EPS = 16 / T::kBytes;  // elements per 16-byte slot
  static constexpr int ROWB = D * T::kBytes;
  static constexpr int NSL = ROWB / 16;
  static constexpr int UNITS = NSL * (kChunk / 4);
  static constexpr int PASSES = (UNITS + NTH - 1) / NTH;
  static constexpr int VTB = kChunk * T::kBytes;
  static constexpr int BYTES = 2 * kChunk * ROWB;
  u32x4 kpre[4], vpre[4];

  __device__ __forceinline__ void fetch(const st* kg, const st* vg, int64_t c, int pass, int tid) {
    const int u = tid + pass * NTH;
    if (UNITS % NTH != 0 && u >= UNITS) return;
    const int sl = u % NSL, t0 = 4 * (u / NSL);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t off = (c * kChunk + t0 + i) * D + sl * EPS;
      kpre[i] = *reinterpret_cast<const u32x4*>(kg + off);
      vpre[i] = *reinterpret_cast<const u32x4*>(vg + off);
    }
  }
  __device__ __forceinline__ void stash(char* ks, char* vt, int pass, int tid) {
    const int u = tid + pass * NTH;
    if (UNITS % NTH != 0 && u >= UNITS) return;
    const int sl = u % NSL, t0 = 4 * (u / NSL);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + i;
      *reinterpret_cast<u32x4*>(ks + t * ROWB + ((sl ^ (t & 7)) * 16)) = kpre[i];
    }
    const int p = vt_pos(t0);  // the four tokens sit at p .. p+3
    if constexpr (T::kBytes == 2) {
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int d = sl * EPS + e;
        const int w = e / 2, sh = (e & 1) * 16;
        const uint32_t lo = ((vpre[0][w] >> sh) & 0xffffu) | (((vpre[1][w] >> sh) & 0xffffu) << 16);
        const uint32_t hi = ((vpre[2][w] >> sh) & 0xffffu) | (((vpre[3][w] >> sh) & 0xffffu) << 16);
        const int pp = (((p / 8) ^ vt_swz(d)) * 8) + (p % 8);
        *reinterpret_cast<u32x2*>(vt + d * VTB + pp * 2) = u32x2{lo, hi};
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int d = sl * EPS + e;
        const int pp = ((p / 4) ^ vt_swz(d)) * 4;
        *reinterpret_cast<u32x4*>(vt + d * VTB + pp * 4) = u32x4{vpre[0][e], vpre[1][e], vpre[2][e], vpre[3][e]};
      }
    }
  }
  // whole tile, fetch and stash pass by pass (caller synchronises)
  __device__ __forceinline__ void load(const st* kg, const st* vg, int64_t c, char* ks, char* vt, int tid) {
#pragma unroll 1
    for (int ps = 0; ps < PASSES; ++ps) {
      fetch(kg, vg, c, ps, tid);
      stash(ks, vt, ps, tid);
    }
  }
};

// One wave, 32 query rows (B operand qf, row = lane % 32; lanes l and l^32
// hold the two halves of each row): softmax attention over the 64 tokens of
// the staged chunk, accumulated into the O^T tiles as factor * o_c.
template <typename T, int D>
__device__ __forceinline__ void attend_block(const Frag<T> (&qf)[D / 16], const char* ks, const char* vt,
                                             float factor, float cexp, f32x16 (&oacc)[D / 32], int lane) {
  constexpr int ROWB = D * T::kBytes;
  constexpr int VTB = kChunk * T::kBytes;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
  const int half = lane >> 5;
  // S^T = K_c Q^T: two 32-token blocks
  f32x16 s0 = {}, s1 = {};
  const char* k0 = ks + (lane & 31) * ROWB;
  const char* k1 = ks + (32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int s = 0; s < KCH; ++s) {
    Frag<T> a0, a1;
    load_frag_lds<T>(a0, k0, lane & 7, s, half);
    load_frag_lds<T>(a1, k1, lane & 7, s, half);
    mfma(s0, a0, qf[s]);
    mfma(s1, a1, qf[s]);
  }
  // softmax over the row's 64 tokens; lane l and l^32 split them
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f((s0[r] - mx) * cexp);
    s1[r] = __builtin_amdgcn_exp2f((s1[r] - mx) * cexp);
    sum += s0[r] + s1[r];
  }
  sum += __shfl_xor(sum, 32);
  const float f = factor / sum;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] *= f;
    s1[r] *= f;
  }
  // O^T += V^T P'^T over four 16-token k-steps
#pragma unroll
  for (int ks_ = 0; ks_ < 4; ++ks_) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = (ks_ < 2) ? s0[8 * (ks_ & 1) + e] : s1[8 * (ks_ & 1) + e];
    if constexpr (T::kBytes == 2) {
      Frag<BF16> phi, plo;
      phi.from_f32(pv);
      float rem[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rem[e] = pv[e] - static_cast<float>(phi.v[e]);
      plo.from_f32(rem);
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        Frag<BF16> a;
        const int d = 32 * dm + (lane & 31);
        const int slot = (2 * ks_ + half) ^ vt_swz(d);
        a.load16(vt + d * VTB + slot * 16);
        mfma(oacc[dm], a, phi);
        mfma(oacc[dm], a, plo);
      }
    } else {
      Frag<FP32> pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.v[e] = pv[e];
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        Frag<FP32> a;
        const int d = 32 * dm + (lane & 31);
        const int s0i = (4 * ks_ + 2 * half) ^ vt_swz(d);
        const int s1i = (4 * ks_ + 2 * half + 1) ^ vt_swz(d);
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(vt + d * VTB + s0i * 16);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(vt + d * VTB + s1i * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a.v[e] = x0[e];
          a.v[4 + e] = x1[e];
        }
        mfma(oacc[dm], a, pf);
      }
    }
  }
}

// Output columns held by a lane in the O^T accumulators: for tile dm and
// register group q4, four consecutive columns starting at out_col(dm, q4).
__device__ __forceinline__ int out_col(int dm, int q4, int half) { return 32 * dm + 8 * q4 + 4 * half; }

// Buckets the remote pairs by (b, g, chunk): pair_pos[i] = position of
// pair i in `pairs` (-1 when local or empty), off[] = bucket offsets,
// pairs[] = query row of each pair.  Four launches (prefill.hip).
hipError_t launch_prefill_bucketing(const PrefillArgs& a, hipStream_t st);

// ---- chunk-major attention of the remote pairs
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prefill_remote_kernel(const typename T::storage* __restrict__ q,
                                                             const typename T::storage* __restrict__ kk,
                                                             const typename T::storage* __restrict__ vv,
                                                             const int* __restrict__ off,
                                                             const int32_t* __restrict__ pairs,
                                                             float* __restrict__ partial, int Hkv, int64_t T_len,
                                                             int64_t Nc, float scale) {
  using st = typename T::storage;
  using Stage = KVStage<T, D, 256>;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
  __shared__ __align__(16) char smem[Stage::BYTES];
  char* ks = smem;
  char* vt = smem + kChunk * Stage::ROWB;
  const int64_t bucket = blockIdx.x;
  const int begin = off[bucket], end = off[bucket + 1];
  if (begin == end) return;
  const int64_t c = bucket % Nc;
  const int64_t bg = bucket / Nc;  // b * Hkv + g
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  Stage stage;
  stage.load(kk + bg * T_len * D, vv + bg * T_len * D, c, ks, vt, tid);
  __syncthreads();
  const float cexp = scale * 1.4426950408889634f;
  for (int blk = wave; begin + 32 * blk < end; blk += 4) {
    const int p = begin + 32 * blk + (lane & 31);
    const bool ok = p < end;
    const int64_t row = ok ? pairs[p] : 0;
    Frag<T> qf[KCH];
    const st* qp = q + row * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KCH; ++s) load_frag_global(qf[s], qp + 16 * s, ok);
    f32x16 oacc[DM];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};
    attend_block<T, D>(qf, ks, vt, 1.0f, cexp, oacc, lane);
    if (ok) {
      float* op = partial + (int64_t)p * D;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(op + out_col(dm, q4, half)) =
              f32x4{oacc[dm][4 * q4], oacc[dm][4 * q4 + 1], oacc[dm][4 * q4 + 2], oacc[dm][4 * q4 + 3]};
    }
  }
}

// ---- local pairs and fusion
template <typename T, int D, int G, int KSEL>
#ifndef HSA_ATTN_LOCAL_WAVES_PER_EU
#define HSA_ATTN_LOCAL_WAVES_PER_EU 2
#endif
__global__ __launch_bounds__(kWave* G)
    __attribute__((amdgpu_waves_per_eu(HSA_ATTN_LOCAL_WAVES_PER_EU))) void prefill_local_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ kk,
    const typename T::storage* __restrict__ vv, const int32_t* __restrict__ sel_idx,
    const float* __restrict__ sel_score, const int32_t* __restrict__ pair_pos, const float* __restrict__ partial,
    float* __restrict__ out, int B, int Hkv, int64_t T_len, int64_t Nc, int nqc, int k, float scale) {
  using st = typename T::storage;
  constexpr int NTH = kWave * G;
  using Stage = KVStage<T, D, NTH>;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
  constexpr int NW = kLocalWindow / 32;  // bitmap words of one window
  extern __shared__ __align__(16) char smem[];
  char* ks = smem;
  char* vt = smem + kChunk * Stage::ROWB;
  // per row k entries: local (chunk, weight) ascending from the front,
  // remote (pair position, weight) from the back
  int2* tab = reinterpret_cast<int2*>(smem + Stage::BYTES);
  __shared__ uint32_t bm[NW];

  const int bid = blockIdx.x;
  const int g = bid % Hkv;
  int rest = bid / Hkv;
  const int b = rest % B;
  rest /= B;
  const int hc = rest & 1;
  const int j = nqc - 1 - (rest >> 1);
  const int tid = threadIdx.x, lane = tid & 63, hh = tid >> 6, half = lane >> 5;
  const int Hq = Hkv * G, h = g * G + hh;
  const int64_t n = min((int64_t)j, Nc);
  const int ws = (j / kLocalWindow) * kLocalWindow;  // first chunk of the query's window
  const int row = hh * 32 + (lane & 31);
  const int64_t tok = (int64_t)j * kChunk + 32 * hc + (lane & 31);
  const bool tok_ok = tok < T_len;

  if (tid < NW) bm[tid] = 0u;
  __syncthreads();

  // ---- per-row tables: fusion weights of all kept chunks, local ones in
  // ascending chunk order, remote ones with their pair positions
  int m = 0, rc = 0;
  if (lane < 32 && tok_ok && n > 0) {
    const int64_t base = (((int64_t)b * Hq + h) * T_len + tok) * k;
    int ci[KSEL];
    float sc[KSEL];
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      ci[e] = (e < k) ? sel_idx[base + e] : -1;
      sc[e] = (e < k && ci[e] >= 0) ? sel_score[base + e] : -__builtin_inff();
    }
    const float smax = sc[0];
    float w[KSEL], den = 0.0f;
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      w[e] = ci[e] >= 0 ? expf(sc[e] - smax) : 0.0f;
      den += w[e];
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      if (ci[e] >= ws) {
        int rank = 0;
#pragma unroll
        for (int f = 0; f < KSEL; ++f) rank += (ci[f] >= ws && ci[f] < ci[e]);
        tab[row * k + rank] = make_int2(ci[e], __float_as_int(w[e] * inv));
        atomicOr(&bm[(ci[e] - ws) >> 5], 1u << ((ci[e] - ws) & 31));
        ++m;
      } else if (ci[e] >= 0) {
        ++rc;
        tab[row * k + k - rc] = make_int2(pair_pos[base + e], __float_as_int(w[e] * inv));
      }
    }
  }
  m = __shfl(m, lane & 31);  // the partner lane of the row learns the counts
  rc = __shfl(rc, lane & 31);
  __syncthreads();

  Frag<T> qf[KCH];
  {
    const st* qp = q + (((int64_t)b * Hq + h) * T_len + (tok_ok ? tok : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KCH; ++s) load_frag_global(qf[s], qp + 16 * s, tok_ok);
  }
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  // walk the union of the block's local selections in ascending order
  int word = 0;
  uint32_t bits = bm[0];
  auto next_chunk = [&]() -> int {
    while (bits == 0u) {
      if (++word >= NW) return -1;
      bits = bm[word];
    }
    const int c = ws + word * 32 + __builtin_ctz(bits);
    bits &= bits - 1u;
    return c;
  };
  const st* kg = kk + ((int64_t)b * Hkv + g) * T_len * D;
  const st* vg = vv + ((int64_t)b * Hkv + g) * T_len * D;
  const float cexp = scale * 1.4426950408889634f;
  Stage stage;
  int ptr = 0;
  int c = next_chunk();
  if (Stage::PASSES == 1 && c >= 0) stage.fetch(kg, vg, c, 0, tid);
  while (c >= 0) {
    __syncthreads();  // everyone is done with the previous tile
    if constexpr (Stage::PASSES == 1) {
      stage.stash(ks, vt, 0, tid);
    } else {
      stage.load(kg, vg, c, ks, vt, tid);
    }
    __syncthreads();
    const int cn = next_chunk();
    if (Stage::PASSES == 1 && cn >= 0) stage.fetch(kg, vg, cn, 0, tid);
    float wgt = 0.0f;
    bool mine = false;
    if (ptr < m) {
      const int2 e = tab[row * k + ptr];
      mine = e.x == c;
      if (mine) {
        wgt = __int_as_float(e.y);
        ++ptr;
      }
    }
    if (__ballot(mine)) attend_block<T, D>(qf, ks, vt, wgt, cexp, oacc, lane);
    c = cn;
  }
  // add the weighted outputs of the row's remote pairs
  int rmax = rc;
  for (int off = 32; off >= 1; off >>= 1) rmax = max(rmax, __shfl_xor(rmax, off));
  for (int r = 0; r < rmax; ++r) {
    if (r < rc) {
      const int2 e = tab[row * k + k - 1 - r];
      const float w = __int_as_float(e.y);
      const float* pp = partial + (int64_t)e.x * D;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(pp + out_col(dm, q4, half));
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[dm][4 * q4 + i] = fmaf(w, x[i], oacc[dm][4 * q4 + i]);
        }
    }
  }
  if (tok_ok) {
    float* op = out + (((int64_t)b * Hq + h) * T_len + tok) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(op + out_col(dm, q4, half)) =
            f32x4{oacc[dm][4 * q4], oacc[dm][4 * q4 + 1], oacc[dm][4 * q4 + 2], oacc[dm][4 * q4 + 3]};
  }
}

size_t prefill_attn_lds_bytes(const Geometry& g);

template <typename T, int D, int G, int KSEL>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  using stg = typename T::storage;
  const int nqc = (int)((g.T + kChunk - 1) / kChunk);
  const float scale = 1.0f / sqrtf((float)D);
  const unsigned blocks = (unsigned)((int64_t)nqc * g.B * g.Hkv);
  const stg* q = static_cast<const stg*>(a.q);
  const stg* k = static_cast<const stg*>(a.k);
  const stg* v = static_cast<const stg*>(a.v);
  constexpr int HPW = G < 4 ? G : 4;
  mark_launch(st);
  hipLaunchKernelGGL((prefill_select_kernel<T, D, G, KSEL>), dim3(blocks * (G / HPW)), dim3(kWave * HPW), 0, st, q,
                     static_cast<const stg*>(a.lm), a.sel_idx, a.sel_score, g.B, g.Hkv, g.T, g.Nc, nqc, g.k, scale);
  mark_launch(st);
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;  // remote-pair buckets
  if (nb > 0) {
    hipError_t e = launch_prefill_bucketing(a, st);
    if (e != hipSuccess) return e;
    mark_launch(st);
    hipLaunchKernelGGL((prefill_remote_kernel<T, D, G>), dim3((unsigned)nb), dim3(256), 0, st, q, k, v, a.off,
                       a.pairs, a.partial, g.Hkv, g.T, g.Nc, scale);
    mark_launch(st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = prefill_attn_lds_bytes(g);
  auto kern = prefill_local_kernel<T, D, G, KSEL>;
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
  }
  mark_launch(st);
  hipLaunchKernelGGL(kern, dim3(2 * blocks), dim3(kWave * G), lds, st, q, k, v, a.sel_idx, a.sel_score, a.pair_pos,
                     a.partial, a.out, g.B, g.Hkv, g.T, g.Nc, nqc, g.k, scale);
  mark_launch(st);
  return hipGetLastError();
}

// Dispatch over the query-group size; instantiated once per (dtype, D, list
// size) in its own translation unit so the build parallelises.
template <typename T, int D, int KSEL>
hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_prefill_t<T, D, 1, KSEL>(a, st);
    case 2: return launch_prefill_t<T, D, 2, KSEL>(a, st);
    case 4: return launch_prefill_t<T, D, 4, KSEL>(a, st);
    default: return launch_prefill_t<T, D, 8, KSEL>(a, st);
  }
}

}  // namespace hsa_attn
